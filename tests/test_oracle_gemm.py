"""Pins for the oracle's fp64 W4A16 product."""

from fractions import Fraction

import numpy as np

from oracle import bf16, gemm, quant


def _integer_weights(rng, N, K):
    """bf16 weights whose every 32-group has max|w| = 7 and integer values,
    so s = 1 and q = w exactly."""
    w = rng.integers(-7, 8, size=(N, K)).astype(np.float32)
    w = w.reshape(N, K // 32, 32)
    w[:, :, 0] = np.where(rng.integers(0, 2, size=(N, K // 32)) == 1, 7.0, -7.0)
    return bf16.rne(w.reshape(N, K))


def test_integer_exact_special_case_equals_textbook_matmul():
    rng = np.random.default_rng(21)
    M, N, K = 5, 7, 96
    W = _integer_weights(rng, N, K)
    Wq, S = quant.quantize_pack(W)
    assert np.all(bf16.to_f32(S) == 1.0)
    X = bf16.rne(rng.integers(-2, 3, size=(M, K)).astype(np.float32))
    y = gemm.w4a16_gemm(X, Wq, S)
    xi = [[int(v) for v in row] for row in bf16.to_f32(X)]
    wi = [[int(v) for v in row] for row in bf16.to_f32(W)]
    for m in range(M):
        for n in range(N):
            assert y[m, n] == sum(xi[m][k] * wi[n][k] for k in range(K))
    # bf16 output is exact here too (|y| < 2^8 integers)
    assert np.array_equal(bf16.to_f32(gemm.to_bf16(y)), y.astype(np.float32))


def test_brute_force_exact_rationals_tiny():
    rng = np.random.default_rng(22)
    M, N, K = 3, 4, 64            # non-square so a transposed operand fails
    W = bf16.rne((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    X = bf16.rne(rng.standard_normal((M, K)).astype(np.float32))
    Wq, S = quant.quantize_pack(W)
    y = gemm.w4a16_gemm(X, Wq, S)
    q = quant.unpack(Wq)
    s = bf16.to_f32(S)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                wprime = Fraction(float(bf16.to_f32(
                    bf16.rne(np.float32(int(q[n, k]) * float(s[n, k // 32]))))))
                acc += Fraction(float(bf16.to_f32(X[m, k]))) * wprime
            assert abs(Fraction(float(y[m, n])) - acc) <= Fraction(1, 10 ** 12)


def test_dequant_uses_group_scale_along_k():
    """Scale index is k // 32 along K (a transposed or per-row scale fails)."""
    N, K = 2, 64
    q = np.ones((N, K), dtype=np.int8)
    S = bf16.rne(np.array([[1.0, 2.0], [4.0, 8.0]], dtype=np.float32))
    Wq = quant.pack(q)
    w = gemm.dequant_f64(Wq, S)
    assert np.all(w[0, :32] == 1.0) and np.all(w[0, 32:] == 2.0)
    assert np.all(w[1, :32] == 4.0) and np.all(w[1, 32:] == 8.0)
    X = bf16.rne(np.eye(1, K, 40, dtype=np.float32))   # picks k = 40
    y = gemm.w4a16_gemm(X, Wq, S)
    assert list(y[0]) == [2.0, 8.0]


def test_tolerance_rule():
    # all values below are exact in bf16; the bound is 2e-2 + 1e-2 * |ref|
    ref = np.array([1.0, -3.0, 0.0, 100.0])
    inside = np.array([1.0234375, -3.046875, 0.015625, 101.0])
    outside_abs = np.array([1.0, -3.0, 0.0234375, 100.0])
    outside_rel = np.array([1.0, -3.0625, 0.0, 100.0])
    for y, want in [(inside, True), (outside_abs, False), (outside_rel, False)]:
        yb = bf16.rne(y.astype(np.float32))
        assert np.array_equal(bf16.to_f32(yb), y.astype(np.float32))
        ok, _, _ = gemm.within_tolerance(yb, ref)
        assert ok is want
