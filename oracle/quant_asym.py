"""Asymmetric (zero-point) group-wise INT4 quantization, packing and fake
quantization.

Oracle (test infrastructure only).  Sources:

* "Quantization basics: from FP32 to INT4" (量化基础：从 FP32 到 INT4 的压缩艺术):
  §2.1 the affine map q = clamp(round(x/s) + z, q_min, q_max) with inverse
  x_hat = (q - z) * s, and the zero-point bullet (z is an integer so that
  the float 0 is represented exactly); §2.3 the asymmetric case:
  s = (x_max - x_min) / (q_max - q_min), z = clamp(round(q_min - x_min/s),
  q_min, q_max); §5 / §6.2 round half to even; §3 per-group granularity.
* "Quantization-aware training" tag summary [11]: one scale per 1 x 32
  group (the same groups as the symmetric path).

Readings where the pages leave a step open (each is listed with its reason
in the design notes of the repository):

* The grid is unsigned INT4: [q_min, q_max] = [0, 15].
* The range is widened to contain 0: x_min = min(min w, 0) and
  x_max = max(max w, 0), so that 0 is always on the grid (the zero-point
  bullet); a constant group c then keeps c instead of dividing by zero.
* s = bf16(fp32(x_max - x_min) / 15): fp32 subtraction and IEEE division,
  then round to nearest even; the stored bf16 s divides and dequantizes.
* z = clamp(rint_half_even(0 - fp32(x_min) / s), 0, 15) (IEEE division),
  stored as one unsigned byte per group.
* q = clamp(rint_half_even(fp32(w) / s) + z, 0, 15) (IEEE division).
* A group whose bf16 s is 0 (all zeros, or a range that rounds to 0 in
  bf16) gets z = 0 and q = 0.
* Packing as the symmetric codes (nibble j of word w holds k = 8w + j),
  the nibble being the unsigned code q.
* Dequantized weights are bf16((q - z) * s): a 5-bit integer times an
  8-bit-mantissa scale is exact in fp32, so this is one rounding.
"""

import numpy as np

from . import bf16

GROUP = 32
QMIN, QMAX = 0, 15
PER_WORD = 8


def quantize_asym(W):
    """Asymmetric INT4 group quantization of a bf16 weight matrix.

    ``W``: uint16 bf16 bit patterns [N, K], K a multiple of 32.  Returns
    (q uint8 [N, K] in [0, 15], S uint16 bf16 bits [N, K/32], Z uint8
    [N, K/32] in [0, 15]).  Arithmetic in float32 as in the docstring.
    """
    W = np.asarray(W, dtype=np.uint16)
    n, k = W.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 32")
    w = bf16.to_f32(W).reshape(n, k // GROUP, GROUP)
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    f32 = np.float32
    x_min = np.minimum(w.min(axis=-1), f32(0))
    x_max = np.maximum(w.max(axis=-1), f32(0))
    span = (x_max - x_min).astype(f32)                       # fp32 subtraction
    S = bf16.rne((span / f32(QMAX - QMIN)).astype(f32))      # IEEE division, RNE to bf16
    s = bf16.to_f32(S)
    with np.errstate(divide="ignore", invalid="ignore"):
        zr = (f32(QMIN) - (x_min / s).astype(f32)).astype(f32)
        z = np.clip(np.rint(zr), QMIN, QMAX)
        r = (w / s[..., None]).astype(f32)
        q = np.clip(np.rint(r) + z[..., None], QMIN, QMAX)
    zero = s == 0
    z = np.where(zero, 0, z)
    q = np.where(zero[..., None], 0, q)
    return q.reshape(n, k).astype(np.uint8), S, z.astype(np.uint8)


def pack_unsigned(q):
    """Pack unsigned 4-bit codes [N, K] into int32 words [N, K/8] along K."""
    q = np.asarray(q)
    n, k = q.shape
    if k % PER_WORD:
        raise ValueError("K must be a multiple of 8")
    if np.any(q > 15):
        raise ValueError("codes must be in [0, 15]")
    nib = q.astype(np.uint32).reshape(n, k // PER_WORD, PER_WORD)
    word = np.zeros((n, k // PER_WORD), dtype=np.uint32)
    for j in range(PER_WORD):
        word |= nib[:, :, j] << np.uint32(4 * j)
    return word.view(np.int32)


def unpack_unsigned(Wq):
    """Inverse of ``pack_unsigned``: int32 [N, K/8] -> uint8 codes [N, K]."""
    u = np.asarray(Wq, dtype=np.int32).view(np.uint32)
    n, kw = u.shape
    out = np.empty((n, kw, PER_WORD), dtype=np.uint8)
    for j in range(PER_WORD):
        out[:, :, j] = ((u >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)
    return out.reshape(n, kw * PER_WORD)


def dequant_asym(q, S, Z):
    """bf16 dequantized weights w' = bf16((q - z) * s) (tutorial §2.1)."""
    q = np.asarray(q)
    n, k = q.shape
    s = bf16.to_f32(S).reshape(n, k // GROUP, 1)
    z = np.asarray(Z, dtype=np.float32).reshape(n, k // GROUP, 1)
    d = (q.astype(np.float32).reshape(n, k // GROUP, GROUP) - z).astype(np.float32)
    return bf16.rne((d * s).astype(np.float32).reshape(n, k))


def fake_quant_asym(W):
    """bf16 W -> bf16 dequant_asym(quantize_asym(W))."""
    q, S, Z = quantize_asym(W)
    return dequant_asym(q, S, Z)


def quantize_pack_asym(W):
    """quantize + pack: bf16 [N, K] -> (int32 [N, K/8], bf16 bits [N, K/32], uint8 [N, K/32])."""
    q, S, Z = quantize_asym(W)
    return pack_unsigned(q), S, Z
