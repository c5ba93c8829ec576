"""GPU parity: w4a16_gemm_asym (zero-point weights; decode path and MFMA
GEMM path) against the fp64 oracle.

Tolerance (per element, against the unrounded fp64 product):
    |y - y_ref| <= 2e-2 + 1e-2 * |y_ref|
Where every partial sum is an exact integer the output must be bit-exact:
integer weight groups spanning [lo, lo + 15] with lo in [-15, 0] quantize
to s = 1 and z = -lo (every zero point 0..15 occurs), and integer
activations keep all sums exact.  The weights fed to each side are
quantized by that side (the GPU packing is asserted bit-exact against the
oracle's first).
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import synth
from gpu_util import down, down_bits, say, up_bits
from oracle import bf16, gemm, quant_asym

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def quantized_pair(Wbits):
    """(GPU Wq, S, Z, oracle Wq, S, Z) with the two quantizations equal."""
    ref = quant_asym.quantize_pack_asym(Wbits)
    got = w4.w4_quantize_pack_asym(up_bits(Wbits))
    for g, r, name in zip(got, ref, ("Wq", "S", "Z")):
        np.testing.assert_array_equal(down_bits(g) if name == "S" else down(g), r, err_msg=name)
    return got + ref


def assert_close(y_bits, y_ref, label):
    ok, max_abs, max_rel = gemm.within_tolerance(y_bits, y_ref, ATOL, RTOL)
    assert ok, f"{label}: max abs {max_abs:.3e}, max rel {max_rel:.3e}"


def run_case(M, N, K, seed, label):
    say(f"gemm_asym {label} M={M} N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, seed))
    Xb = synth.bits(synth.activations(M, K, seed))
    Wq, S, Z, Wq_r, S_r, Z_r = quantized_pair(Wb)
    y = down_bits(w4.w4a16_gemm_asym(up_bits(Xb), Wq, S, Z))
    assert_close(y, gemm.w4a16_gemm_asym(Xb, Wq_r, S_r, Z_r), label)


def integer_weights(N, K, rng):
    """Integer groups spanning exactly [lo, lo + 15], lo uniform in [-15, 0]."""
    G = K // 32
    lo = rng.integers(-15, 1, size=(N, G, 1)).astype(np.float32)
    w = lo + rng.integers(0, 16, size=(N, G, 32)).astype(np.float32)
    w[:, :, 3] = lo[:, :, 0]
    w[:, :, 29] = lo[:, :, 0] + 15.0
    return w.reshape(N, K), (-lo[:, :, 0]).astype(np.uint8)


@pytest.mark.parametrize("M", [1, 2, 5, 16, 17, 31, 32, 33, 64, 129, 300])
@pytest.mark.parametrize("N,K", [(1, 32), (17, 96), (100, 544), (300, 64)])
def test_ragged(M, N, K):
    run_case(M, N, K, 300 + M + N + K, "ragged")


@pytest.mark.parametrize("M", [1, 8, 16, 17, 32, 33, 130])
@pytest.mark.parametrize("K", [4640, 8192, 2048, 6144])
def test_long_k(M, K):
    """K above one decode pass; 4640 also leaves K / 32 off a multiple of 8
    (byte-wise zero-point and scale loads)."""
    run_case(M, 200, K, 11 * M + K, "long K")


@pytest.mark.parametrize("M", [1, 8, 16, 17, 32, 33, 200])
@pytest.mark.parametrize("K", [4096, 8192, 1056, 16416, 20480])
def test_integer_exact(M, K):
    N = 96
    say(f"gemm_asym integer-exact M={M} K={K}")
    rng = np.random.default_rng(50 + M + K)
    w, z_expect = integer_weights(N, K, rng)
    Xi = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wb, Xb = bf16.rne(w), bf16.rne(Xi)
    Wq, S, Z, _, S_r, Z_r = quantized_pair(Wb)
    assert np.all(bf16.to_f32(S_r) == 1.0)
    np.testing.assert_array_equal(Z_r, z_expect)
    assert len(np.unique(Z_r)) == 16
    y = down_bits(w4.w4a16_gemm_asym(up_bits(Xb), Wq, S, Z))
    exact = Xi.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_array_equal(y, gemm.to_bf16(exact))


@pytest.mark.parametrize("M", [1, 8, 16, 32])
def test_decode_full(M):
    wl = synth.WORKLOADS["decode"]
    run_case(M, wl["N"], wl["K"], wl["seed"], "decode")


@pytest.mark.parametrize("M", [1, 8, 9, 16])
def test_decode_four_tiles(M):
    """N = 14336 gives each CU four 16-row tiles: M <= 8 loads its operands
    directly, 8 < M <= 16 takes the 64-byte runs and the register transpose
    (the LDS path has no registers left at four tiles)."""
    run_case(M, 14336, 4096, 77 + M, "four tiles")


@pytest.mark.parametrize("M,N,K", [(17, 12288, 4096), (24, 6000, 4096), (32, 8192, 8192),
                                   (20, 700, 4096), (32, 6000, 4608)])
def test_decode32_tiles(M, N, K):
    """16 < M <= 32 at one, two and three tiles per workgroup, one and two
    K passes (activation halves staged through LDS), and a K that is not a
    whole number of passes (half 0 through registers)."""
    run_case(M, N, K, 31 * M + N + K, "decode32 tiles")


@pytest.fixture(scope="module")
def decode_weights():
    """The decode workload's W [12288, 4096], zero-point packed by the GPU
    (asserted equal to the oracle's) and dequantized by the oracle in fp64."""
    wl = synth.WORKLOADS["decode"]
    Wq, S, Z, Wq_r, S_r, Z_r = quantized_pair(
        synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"])))
    return Wq, S, Z, gemm.dequant_asym_f64(Wq_r, S_r, Z_r)


WIDE = [("x8", 8.0, 0.0, 1.0), ("x16", 16.0, 0.0, 1.0), ("outliers_1pct_x32", 1.0, 0.01, 32.0)]


@pytest.mark.parametrize("M", [1, 8, 16, 32, 64])
@pytest.mark.parametrize("case", WIDE, ids=lambda c: c[0])
def test_wide_activations(decode_weights, M, case):
    """Zero-point weights against activations scaled x8 / x16 or with 1% of
    the channels x32: near-zero outputs of these wide-spread products pass
    the fixed absolute tolerance only if every weight multiplied is the
    definition's bf16((q - z) s).  M = 64 runs the tiled kernel."""
    name, gain, frac, ogain = case
    Wq, S, Z, w64 = decode_weights
    wl = synth.WORKLOADS["decode"]
    say(f"gemm_asym wide activations {name} M={M}")
    X, _ = synth.activations_wide(M, wl["K"], 60 + M, gain, frac, ogain)
    Xb = synth.bits(X)
    y = down_bits(w4.w4a16_gemm_asym(up_bits(Xb), Wq, S, Z))
    ref = bf16.to_f32(Xb).astype(np.float64) @ w64.T
    assert_close(y, ref, f"wide {name} M={M}")


def test_prefill_full():
    """The prefill workload (M = 4096, N = 14336, K = 4096) checked against
    the fp64 oracle in every output element."""
    wl = synth.WORKLOADS["prefill"]
    M, N, K = wl["M"][0], wl["N"], wl["K"]
    say(f"gemm_asym prefill M={M} N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, wl["seed"]))
    Xb = synth.bits(synth.activations(M, K, wl["seed"]))
    Wq, S, Z, Wq_r, S_r, Z_r = quantized_pair(Wb)
    y = down_bits(w4.w4a16_gemm_asym(up_bits(Xb), Wq, S, Z))
    assert_close(y, gemm.w4a16_gemm_asym(Xb, Wq_r, S_r, Z_r), "prefill")


def test_deterministic():
    wl = synth.WORKLOADS["decode"]
    Wq, S, Z = w4.w4_quantize_pack_asym(synth.weights(2048, wl["K"], 4).cuda())
    for M in (8, 24, 96):
        X = synth.activations(M, wl["K"], 4).cuda()
        a = down_bits(w4.w4a16_gemm_asym(X, Wq, S, Z))
        b = down_bits(w4.w4a16_gemm_asym(X, Wq, S, Z))
        np.testing.assert_array_equal(a, b)


def test_k_zero_writes_zeros():
    Y = torch.full((3, 5), 1.0, dtype=torch.bfloat16, device="cuda")
    X = torch.empty((3, 0), dtype=torch.bfloat16, device="cuda")
    Wq = torch.empty((5, 0), dtype=torch.int32, device="cuda")
    S = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    w4.w4a16_gemm_asym(X, Wq, S, Z, out=Y)
    assert torch.count_nonzero(Y).item() == 0


@pytest.mark.parametrize("M,N,K", [(1, 48, 65536), (32, 48, 65536), (33, 48, 65536),
                                   (1, 100000, 64), (4096, 1, 96)])
def test_extreme_shapes(M, N, K):
    run_case(M, N, K, 7 * M + N + K, "extreme")


@pytest.mark.parametrize("M,N,K", [(1, 310, 96), (5, 77, 4128), (17, 1, 20480), (32, 640, 1056),
                                   (33, 129, 6400), (70, 250, 22400), (200, 31, 32)])
def test_assorted_shapes(M, N, K):
    run_case(M, N, K, M * 13 + N * 17 + K, "assorted")
