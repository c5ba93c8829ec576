"""W4A16 product reference: Y = X * dequant(W)^T with fp64 accumulation.

Oracle (test infrastructure only).  Sources: "INT4 QAT end-to-end for RL",
§4 inference: weights stay INT4 in memory, are dequantized and multiplied
against BF16 activations on BF16 matrix units (there are no INT4 tensor
cores on the GPUs the write-up used); "Quantization basics: from FP32 to
INT4", §2.1 (x_hat = q * s) and §5 (3): accumulation error grows with the
number of terms, so the accumulator must be wide.

Reading: the dequantized operand is w' = bf16(q * s) (the same value fake
quantization produces); the reference sums X[m,k] * w'[n,k] exactly enough
in float64 and keeps the unrounded result; results on the GPU are bf16 and
are compared to this within the stated tolerance.
"""

import numpy as np

from . import bf16, quant, quant_asym


def dequant_f64(Wq, S):
    """Packed int32 [N, K/8] + bf16 scales [N, K/32] -> float64 w' [N, K]."""
    q = quant.unpack(Wq)
    return bf16.to_f32(quant.dequant(q, S)).astype(np.float64)


def w4a16_gemm(X, Wq, S):
    """fp64 reference Y[M, N] = sum_k X[m, k] * w'[n, k].

    ``X``: bf16 bits [M, K]; ``Wq``: int32 [N, K/8]; ``S``: bf16 bits
    [N, K/32].  Returns the unrounded float64 product.
    """
    x = bf16.to_f32(X).astype(np.float64)
    w = dequant_f64(Wq, S)
    return x @ w.T


def w4a16_gemm_asym(X, Wq, S, Z):
    """fp64 reference Y = X * w'^T with asymmetric weights
    w' = bf16((q - z) * s) ("Quantization basics" §2.1 inverse map).

    ``Wq`` int32 [N, K/8] unsigned codes; ``S`` bf16 bits [N, K/32];
    ``Z`` uint8 [N, K/32].  Returns the unrounded float64 product.
    """
    x = bf16.to_f32(X).astype(np.float64)
    return x @ dequant_asym_f64(Wq, S, Z).T


def dequant_asym_f64(Wq, S, Z):
    """Unsigned packed codes + bf16 scales + uint8 zero points [N, K/32] ->
    float64 w' = bf16((q - z) * s) [N, K] ("Quantization basics" §2.1)."""
    q = quant_asym.unpack_unsigned(Wq)
    return bf16.to_f32(quant_asym.dequant_asym(q, S, Z)).astype(np.float64)


def dequant_weights_f64(*w):
    """(Wq, S) -> symmetric dequant; (Wq, S, Z) -> zero-point dequant."""
    if len(w) == 2:
        return dequant_f64(*w)
    if len(w) == 3:
        return dequant_asym_f64(*w)
    raise ValueError("weights are (Wq, S) or (Wq, S, Z)")


def to_bf16(y):
    """Round a float64 result to the bf16 storage type (via float32)."""
    return bf16.rne(np.asarray(y, dtype=np.float64).astype(np.float32))


def within_tolerance(y_gpu_bits, y_ref, atol=2e-2, rtol=1e-2):
    """Element-wise |y - y_ref| <= atol + rtol * |y_ref| for bf16 outputs.

    Returns (ok, max_abs_err, max_rel_err over |y_ref| >= 1e-2).
    """
    y = bf16.to_f32(y_gpu_bits).astype(np.float64)
    ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - ref)
    ok = bool(np.all(err <= atol + rtol * np.abs(ref)))
    big = np.abs(ref) >= 1e-2
    max_rel = float(np.max(err[big] / np.abs(ref[big]))) if np.any(big) else 0.0
    return ok, float(err.max()) if err.size else 0.0, max_rel
