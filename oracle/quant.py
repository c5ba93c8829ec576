"""Symmetric group-wise quantization, INT4 packing and fake quantization.

Oracle (test infrastructure only).  Sources:

* "Quantization basics: from FP32 to INT4" (量化基础：从 FP32 到 INT4 的压缩艺术):
  §2.1 the affine map q = clamp(round(x/s) + z, q_min, q_max) and its inverse
  x_hat = (q - z) * s; §2.2 the symmetric case z = 0, s = max|x| / q_max;
  §1.3 table: INT4 is the uniform grid [-8, 7]; §3 per-group granularity;
  §5 (1) and §6.2: round must be a true round, half-to-even like
  torch.round, never an implicit truncating cast.
* "INT4 QAT end-to-end for RL" (SGLang RL write-up): §3.2 weight-update
  quantization packs 8 INT4 values into one INT32 (8 x 4 bits = 32 bits,
  Fig. 4); §2.1 fake quantization maps weights onto the INT4 grid and
  immediately restores them, the arithmetic staying in BF16.
* "Quantization-aware training" tag summary: bullet [11], one scale per
  1 x 32 group; bullet [32], two 4-bit weights per byte.

Readings where the pages leave a step open (each is listed with its reason
in the design notes of the repository):

* The scale is max|w| / 7 computed as an IEEE fp32 division and then
  rounded to bfloat16 (round to nearest even); that stored bf16 scale is
  the one that divides w and the one that dequantizes.
* w / s is an IEEE fp32 division, rounded half-to-even to an integer and
  clamped to [-8, 7].  With s = bf16(max|w| / 7) every |q| <= 7, so the
  [-7, 7] range of the RL write-up and the [-8, 7] grid of the tutorial
  give the same codes.
* A group whose bf16 scale is 0 (all zeros, or a magnitude so small that
  max|w|/7 rounds to 0 in bf16) quantizes to q = 0.
* Packing is along K: nibble j (bits 4j..4j+3) of word w holds the two's
  complement code of element k = 8w + j.
* Dequantized weights are bf16(q * s): the fp32 product is exact, so this
  is one rounding, and fake quant equals dequant(quantize(w)) bit for bit.
"""

import numpy as np

from . import bf16

GROUP = 32          # elements per scale along K (1 x 32 groups)
QMAX = 7            # INT4 symmetric scale divisor
QMIN_INT4 = -8      # INT4 grid [-8, 7]
QMAX_INT4 = 7
PER_WORD = 8        # INT4 codes per 32-bit word


def quantize_groups(xg, qmax, qmin, dtype, store_scale=None):
    """Symmetric quantization of the last axis of ``xg``, one scale per row.

    Follows the tutorial's §2.2 step by step in the arithmetic type
    ``dtype``: s = max|x| / q_max, q = clamp(round(x / s), q_min, q_max),
    with round = half-to-even (§6.2).  ``store_scale`` maps the computed
    scale to the value that is stored and used (identity when None); a
    stored scale of 0 gives q = 0.

    Returns (q as int32, s as ``dtype``).
    """
    x = np.asarray(xg, dtype=dtype)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / dtype(qmax)).astype(dtype)
    if store_scale is not None:
        s = np.asarray(store_scale(s), dtype=dtype)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (x / s[..., None]).astype(dtype)
    q = np.clip(np.rint(r), qmin, qmax)
    q = np.where(s[..., None] == 0, 0, q)
    return q.astype(np.int32), s


def generic_symmetric(x, qmax):
    """Whole-tensor symmetric quantizer in float64 (tutorial §6.1 setting).

    s = max|x| / qmax, q = clamp(round(x/s), -qmax, qmax), x_hat = q * s.
    Returns (q, s, x_hat).  Used to reproduce the tutorial's worked INT8
    example; it is the same ``quantize_groups`` routine the INT4 path uses.
    """
    x = np.asarray(x, dtype=np.float64)
    q, s = quantize_groups(x.reshape(1, -1), qmax, -qmax, np.float64)
    q = q.reshape(x.shape)
    s = float(s[0])
    return q, s, q.astype(np.float64) * s


def _bf16_scale(s32):
    return bf16.to_f32(bf16.rne(s32))


def quantize(W):
    """INT4 symmetric group quantization of a bf16 weight matrix.

    ``W``: uint16 bf16 bit patterns of shape [N, K], K a multiple of 32.
    Returns (q int8 [N, K] with values in [-8, 7], S uint16 bf16 bits
    [N, K/32]).  Arithmetic as in the module docstring: amax exact, s =
    bf16(fp32(amax) / 7), q = clamp(rint_half_even(fp32(w) / s), -8, 7).
    """
    W = np.asarray(W, dtype=np.uint16)
    n, k = W.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 32")
    w = bf16.to_f32(W).reshape(n, k // GROUP, GROUP)
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    q, s = quantize_groups(w, QMAX, QMIN_INT4, np.float32, _bf16_scale)
    # QMAX_INT4 clamp: quantize_groups clamps to [qmin, qmax] = [-8, 7]
    return q.reshape(n, k).astype(np.int8), bf16.rne(s)


def pack(q):
    """Pack INT4 codes [N, K] into int32 words [N, K/8] along K.

    Word w of a row holds k = 8w + j in bits 4j..4j+3 as a two's
    complement nibble ("INT4 QAT end-to-end for RL", §3.2 / Fig. 4:
    eight INT4 values in one INT32).
    """
    q = np.asarray(q)
    n, k = q.shape
    if k % PER_WORD:
        raise ValueError("K must be a multiple of 8")
    nib = (q.astype(np.int64) & 0xF).astype(np.uint32).reshape(n, k // PER_WORD, PER_WORD)
    word = np.zeros((n, k // PER_WORD), dtype=np.uint32)
    for j in range(PER_WORD):
        word |= nib[:, :, j] << np.uint32(4 * j)
    return word.view(np.int32)


def unpack(Wq):
    """Inverse of ``pack``: int32 words [N, K/8] -> int8 codes [N, K]."""
    u = np.asarray(Wq, dtype=np.int32).view(np.uint32)
    n, kw = u.shape
    out = np.empty((n, kw, PER_WORD), dtype=np.int8)
    for j in range(PER_WORD):
        nib = ((u >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.int16)
        out[:, :, j] = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return out.reshape(n, kw * PER_WORD)


def dequant(q, S):
    """bf16 dequantized weights w' = bf16(q * s) (tutorial §2.1, z = 0).

    ``q`` int codes [N, K]; ``S`` bf16 bits [N, K/32].  Returns bf16 bits.
    The fp32 product of a 4-bit integer and an 8-bit-mantissa scale is
    exact, so the only rounding is the final one to bf16.
    """
    q = np.asarray(q)
    n, k = q.shape
    s = bf16.to_f32(S).reshape(n, k // GROUP, 1)
    prod = (q.astype(np.float32).reshape(n, k // GROUP, GROUP) * s).astype(np.float32)
    return bf16.rne(prod.reshape(n, k))


def fake_quant(W):
    """QAT forward fake quantization: bf16 W -> bf16 dequant(quantize(W)).

    "INT4 QAT end-to-end for RL", §2.1: the weight is mapped onto the INT4
    grid and immediately restored, so the training GEMM still sees bf16.
    """
    q, S = quantize(W)
    return dequant(q, S)


def quantize_pack(W):
    """quantize + pack: bf16 [N, K] -> (int32 [N, K/8], bf16 bits [N, K/32])."""
    q, S = quantize(W)
    return pack(q), S


def packed_bytes(N, K):
    """Storage of the packed form: N*K/2 bytes of codes + 2 bytes per group."""
    return N * K // 2 + 2 * N * (K // GROUP)
