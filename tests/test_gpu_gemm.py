"""GPU parity: w4a16_gemm (decode GEMV path and MFMA GEMM path) against the
fp64 oracle.

Tolerance (per element, against the unrounded fp64 product):
    |y - y_ref| <= 2e-2 + 1e-2 * |y_ref|
Where every partial sum is an exact integer the output must be bit-exact.
The weights fed to each side are quantized by that side (the GPU packing is
asserted bit-exact against the oracle's first).
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import synth
from gpu_util import down, down_bits, say, up_bits
from oracle import bf16, gemm, quant

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def quantized_pair(Wbits):
    """(GPU Wq, GPU S, oracle Wq, oracle S) with the two packings equal."""
    Wq_ref, S_ref = quant.quantize_pack(Wbits)
    Wq, S = w4.w4_quantize_pack(up_bits(Wbits))
    np.testing.assert_array_equal(down(Wq), Wq_ref)
    np.testing.assert_array_equal(down_bits(S), S_ref)
    return Wq, S, Wq_ref, S_ref


def assert_close(y_bits, y_ref, label):
    ok, max_abs, max_rel = gemm.within_tolerance(y_bits, y_ref, ATOL, RTOL)
    assert ok, f"{label}: max abs {max_abs:.3e}, max rel {max_rel:.3e}"


def run_case(M, N, K, seed, label):
    say(f"gemm {label} M={M} N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, seed))
    Xb = synth.bits(synth.activations(M, K, seed))
    Wq, S, Wq_ref, S_ref = quantized_pair(Wb)
    y = down_bits(w4.w4a16_gemm(up_bits(Xb), Wq, S))
    assert_close(y, gemm.w4a16_gemm(Xb, Wq_ref, S_ref), label)


def test_dense_small_seed0():
    wl = synth.WORKLOADS["dense_small"]
    run_case(4, wl["N"], wl["K"], wl["seed"], "512x512")


@pytest.mark.parametrize("M", [1, 2, 5, 16, 17, 31, 32, 33, 64, 127, 129, 300])
@pytest.mark.parametrize("N,K", [(1, 32), (17, 96), (100, 544), (300, 64)])
def test_ragged(M, N, K):
    run_case(M, N, K, 100 + M + N + K, "ragged")


@pytest.mark.parametrize("M", [1, 8, 17, 32, 33, 200])
def test_integer_exact(M):
    """amax = 7 in every group gives s = 1 and q = w; integer activations in
    [-2, 2] keep every fp32 partial sum an exact integer, so Y must equal
    bf16(X @ q^T) bit for bit whatever the summation order."""
    N, K = 96, 4096
    say(f"gemm integer-exact M={M}")
    rng = np.random.default_rng(M)
    q = rng.integers(-7, 8, size=(N, K)).astype(np.float32)
    q.reshape(N, K // 32, 32)[:, :, 0] = 7.0
    Xi = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wb, Xb = bf16.rne(q), bf16.rne(Xi)
    Wq, S, _, S_ref = quantized_pair(Wb)
    assert np.all(bf16.to_f32(S_ref) == 1.0)
    y = down_bits(w4.w4a16_gemm(up_bits(Xb), Wq, S))
    exact = Xi.astype(np.float64) @ q.astype(np.float64).T
    np.testing.assert_array_equal(y, gemm.to_bf16(exact))


@pytest.mark.parametrize("M", [1, 8, 16, 17, 32, 33, 130])
@pytest.mark.parametrize("K", [4640, 8192, 2048, 6144])
def test_long_k(M, K):
    """K above one 4096-wide decode pass (the pass partials carry in LDS);
    4640 also leaves K / 32 off a multiple of 8 (unaligned scale rows);
    2048 and 6144 have aligned scale rows but a partial decode pass (the
    range-checked offsets), 8192 whole passes (offsets without checks)."""
    run_case(M, 200, K, 7 * M + K, "long K")


@pytest.mark.parametrize("M,K", [(1, 8192), (16, 8192), (32, 8192),
                                 (1, 16416), (16, 20480), (32, 20480), (33, 20480)])
def test_integer_exact_two_passes(M, K):
    """As test_integer_exact over several decode K passes (the pass partials
    carry in LDS); 16416 also leaves K / 32 off a multiple of 8."""
    N = 64
    say(f"gemm integer-exact multi-pass M={M} K={K}")
    rng = np.random.default_rng(1000 + M)
    q = rng.integers(-7, 8, size=(N, K)).astype(np.float32)
    q.reshape(N, K // 32, 32)[:, :, 5] = -7.0
    Xi = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    Wb, Xb = bf16.rne(q), bf16.rne(Xi)
    Wq, S, _, S_ref = quantized_pair(Wb)
    assert np.all(bf16.to_f32(S_ref) == 1.0)
    y = down_bits(w4.w4a16_gemm(up_bits(Xb), Wq, S))
    exact = Xi.astype(np.float64) @ q.astype(np.float64).T
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
    """The decode workload's W [12288, 4096], packed by the GPU (asserted
    equal to the oracle's packing) and dequantized by the oracle in fp64."""
    wl = synth.WORKLOADS["decode"]
    Wq, S, Wq_ref, S_ref = quantized_pair(synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"])))
    return Wq, S, gemm.dequant_f64(Wq_ref, S_ref)


WIDE = [("x8", 8.0, 0.0, 1.0), ("x16", 16.0, 0.0, 1.0), ("outliers_1pct_x32", 1.0, 0.01, 32.0),
        ("x4_outliers_1pct_x32", 4.0, 0.01, 32.0)]


@pytest.mark.parametrize("M", [1, 8, 16, 32, 64])
@pytest.mark.parametrize("case", WIDE, ids=lambda c: c[0])
def test_wide_activations(decode_weights, M, case):
    """Activations far from N(0, 1) against the decode workload's weights:
    scaled x8 / x16 (output spread about 10 / 21) and 1% of the K channels
    x32.  The tolerance has a fixed absolute part, so the near-zero outputs
    of such a wide-spread product pass only if every weight the product
    multiplies is the definition's bf16(q s).  M = 64 runs the tiled
    kernel on the same data."""
    name, gain, frac, ogain = case
    Wq, S, w64 = decode_weights
    wl = synth.WORKLOADS["decode"]
    say(f"gemm wide activations {name} M={M}")
    X, _ = synth.activations_wide(M, wl["K"], 40 + M, gain, frac, ogain)
    Xb = synth.bits(X)
    y = down_bits(w4.w4a16_gemm(up_bits(Xb), Wq, S))
    ref = bf16.to_f32(Xb).astype(np.float64) @ w64.T
    assert float(np.std(ref)) > 4.0 * max(1.0, gain / 4)
    assert_close(y, ref, f"wide {name} M={M}")


def test_prefill_full():
    """The prefill workload (M = 4096, N = 14336, K = 4096) checked against
    the fp64 oracle in every output element."""
    wl = synth.WORKLOADS["prefill"]
    M, N, K = wl["M"][0], wl["N"], wl["K"]
    say(f"gemm prefill M={M} N={N} K={K}")
    Wb = synth.bits(synth.weights(N, K, wl["seed"]))
    Xb = synth.bits(synth.activations(M, K, wl["seed"]))
    Wq, S, Wq_ref, S_ref = quantized_pair(Wb)
    y = down_bits(w4.w4a16_gemm(up_bits(Xb), Wq, S))
    assert_close(y, gemm.w4a16_gemm(Xb, Wq_ref, S_ref), "prefill")


def test_deterministic():
    wl = synth.WORKLOADS["decode"]
    Wq, S = w4.w4_quantize_pack(synth.weights(2048, wl["K"], 3).cuda())
    for M in (8, 96):
        X = synth.activations(M, wl["K"], 3).cuda()
        a = down_bits(w4.w4a16_gemm(X, Wq, S))
        b = down_bits(w4.w4a16_gemm(X, Wq, S))
        np.testing.assert_array_equal(a, b)


def test_k_zero_writes_zeros_and_m_zero_is_noop():
    Y = torch.full((3, 5), 1.0, dtype=torch.bfloat16, device="cuda")
    X = torch.empty((3, 0), dtype=torch.bfloat16, device="cuda")
    Wq = torch.empty((5, 0), dtype=torch.int32, device="cuda")
    S = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_gemm(X, Wq, S, out=Y)
    assert torch.count_nonzero(Y).item() == 0
    X0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Wq0 = torch.zeros((5, 8), dtype=torch.int32, device="cuda")
    S0 = torch.zeros((5, 2), dtype=torch.bfloat16, device="cuda")
    assert w4.w4a16_gemm(X0, Wq0, S0).shape == (0, 5)


def test_binding_uses_the_current_stream():
    """The binding passes the caller's current stream (the raw-handle fast
    path agrees with torch.cuda.current_stream), and a product enqueued on a
    side stream equals the one on the default stream."""
    from int4_weight_only_amd import _stream
    wl = synth.WORKLOADS["decode"]
    X = synth.activations(4, wl["K"], 5).cuda()
    assert _stream(X) == torch.cuda.current_stream().cuda_stream
    Wq, S = w4.w4_quantize_pack(synth.weights(512, wl["K"], 5).cuda())
    ref = down_bits(w4.w4a16_gemm(X, Wq, S))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert _stream(X) == side.cuda_stream != torch.cuda.default_stream().cuda_stream
        Y = w4.w4a16_gemm(X, Wq, S)
    side.synchronize()
    np.testing.assert_array_equal(down_bits(Y), ref)


@pytest.mark.parametrize("M,N,K", [(1, 48, 65536), (16, 48, 65536), (32, 48, 65536),
                                   (33, 48, 65536), (1, 100000, 64), (20, 100000, 96),
                                   (4096, 1, 96), (300, 3, 32), (40000, 64, 64)])
def test_extreme_shapes(M, N, K):
    """Long K (16 decode passes; 1024 pipeline steps with 128 scale
    windows), very wide N (about 1600 decode workgroups), a single weight
    row against 4096 activation rows, the smallest K."""
    run_case(M, N, K, 5 * M + N + K, "extreme")


def random_shapes(seed, n):
    """Seeded (M, N, K): M over the decode kernels and the tiled kernel, K
    over aligned / unaligned scale rows, one or several decode passes and the
    dequantizing decode variant, N ragged."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([1, 2, 7, 16, 17, 24, 32, 33, 65, 128, 200]))
        K = 32 * int(rng.choice([1, 3, 8, 33, 128, 129, 200, 520, 700]))
        N = int(rng.integers(1, 700))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", random_shapes(2024, 24))
def test_random_shapes(M, N, K):
    run_case(M, N, K, M * 7919 + N * 31 + K, "random")
