"""GPU parity: routing, moe_align_block_size, the grouped W4A16 expert GEMM,
SwiGLU, the top-k combine and the whole MoE layer, against the oracle.

* moe_align_block_size: bit-exact over the whole output buffers (sentinels
  and the -1 tail included), many shapes, block sizes and id patterns.
* routing: ids exact (the oracle orders the same fp32 logits), weights to
  fp32 rounding.
* GEMMs and the layer: |y - y_ref| <= 2e-2 + 1e-2 |y_ref| against fp64.
* Full-size expert layers.  128 experts x [3072 x 4096] + [4096 x 1536]:
  alignment in full for each block size, every gate_up and down row of
  every expert, the layer output of every token.  384 experts x
  [4096 x 7168] + [7168 x 2048] with skewed routing: alignment in full,
  every row of the 8 hot experts and 24 random ones, the layer output of
  64 tokens.  The GPU side is fed the oracle's routing (ids, weights) so
  that the later stages never depend on a near-tie in fp32 softmax.
Expert weight sources are drawn on the GPU by ``synth`` (seeded); the
oracle gets the same bf16 sources downloaded and quantizes them itself.
"""

import collections
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
from int4_weight_only_amd import moe as wmoe
import synth
from gpu_util import CANARY, canary_bf16, down, down_bits, say, up, up_bits
from oracle import bf16, gemm, quant
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def assert_rows_close(y_bits, ref_rows, label):
    assert ref_rows, f"{label}: nothing to compare"
    fs = sorted(ref_rows)
    ref = np.stack([ref_rows[f] for f in fs])
    ok, max_abs, max_rel = gemm.within_tolerance(y_bits[fs], ref, ATOL, RTOL)
    assert ok, f"{label}: max abs {max_abs:.3e}, max rel {max_rel:.3e} over {len(fs)} rows"


# ------------------------------------------------------------------ align --

def id_cases():
    rng = np.random.default_rng(0)
    c3 = synth.WORKLOADS["moe_qwen"]
    c4 = synth.WORKLOADS["moe_kimi"]
    lg3 = synth.router_logits(c3["T"], c3["E"], c3["seed"]).numpy()
    lg4 = synth.router_logits(c4["T"], c4["E"], c4["seed"], c4["skew"]).numpy()
    ids3 = omoe.route(lg3, c3["k"])[0]
    ids4 = omoe.route(lg4, c4["k"])[0]
    cases = []
    for B in (16, 32, 64):
        cases.append(("qwen_route", ids3, c3["E"], B))
    for B in (32, 64):
        cases.append(("kimi_skew_route", ids4, c4["E"], B))
    cases.append(("random_B1", synth.random_ids(256, 8, 128, 1).numpy(), 128, 1))
    cases.append(("random_B5", synth.random_ids(97, 3, 40, 2).numpy(), 40, 5))
    cases.append(("one_expert", np.zeros((300, 1), np.int32), 1, 16))
    cases.append(("empty_T0", np.zeros((0, 8), np.int32), 16, 16))
    cases.append(("single_pair", np.array([[3]], np.int32), 8, 16))
    cases.append(("out_of_range", rng.integers(-3, 67, size=(500, 6)).astype(np.int32), 64, 16))
    cases.append(("all_same", np.full((1000, 8), 5, np.int32), 64, 64))
    cases.append(("E1024_B1024", rng.integers(0, 1024, size=(50, 4)).astype(np.int32), 1024, 1024))
    cases.append(("big_T_small_E", rng.integers(0, 4, size=(9000, 2)).astype(np.int32), 4, 64))
    return cases


@pytest.mark.parametrize("case", id_cases(), ids=lambda c: c[0])
def test_align_bit_exact(case):
    name, ids, E, B = case
    T, k = ids.shape
    say(f"align {name} T={T} k={k} E={E} B={B}")
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    cap = w4.w4_moe_align_capacity(T, k, E, B)
    # poison the outputs so that any slot the kernel leaves alone shows up
    s = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    e = torch.full((cap // B,), -7, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    w4.moe_align_block_size(up(ids.astype(np.int32)), E, B, s, e, n)
    np.testing.assert_array_equal(down(s), s_ref)
    np.testing.assert_array_equal(down(e), e_ref)
    assert int(down(n)[0]) == n_ref


# ------------------------------------------------------------------ route --

@pytest.mark.parametrize("T,E,k,kind", [(256, 128, 8, "qwen"), (4096, 384, 8, "kimi"),
                                        (33, 5, 5, "rand"), (17, 1000, 16, "rand"),
                                        (10, 64, 1, "rand"), (9, 200, 6, "rand"),
                                        (6, 32, 4, "ties")])
def test_route(T, E, k, kind):
    say(f"route {kind} T={T} E={E} k={k}")
    if kind == "qwen":
        c = synth.WORKLOADS["moe_qwen"]
        lg = synth.router_logits(T, E, c["seed"]).numpy()
    elif kind == "kimi":
        c = synth.WORKLOADS["moe_kimi"]
        lg = synth.router_logits(T, E, c["seed"], c["skew"]).numpy()
    elif kind == "ties":
        lg = np.zeros((T, E), np.float32)
        lg[1, 7] = lg[1, 3] = 2.0
        lg[2, :] = -1.5
    else:
        lg = synth.router_logits(T, E, T * E).numpy()
    ids_ref, w_ref = omoe.route(lg, k)
    ids, w = w4.w4_moe_route(up(lg), k)
    np.testing.assert_array_equal(down(ids), ids_ref)
    np.testing.assert_allclose(down(w), w_ref, rtol=2e-6, atol=1e-7)


# ------------------------------------------------------ element-wise steps --

def test_route_masked_and_tied_logits():
    """Rows with fewer finite logits than k (masked experts at -inf), all
    -inf, all equal, -0 beside +0 (equal logits), NaN logits among numbers
    (never picked) and a row with only 3 numbers among NaNs (the remaining
    picks are the lowest NaN indices, as the oracle's order gives): the ids
    are distinct and follow (logit desc, index asc), as the oracle orders
    them."""
    T, E, k = 9, 40, 8
    lg = np.zeros((T, E), np.float32)
    lg[0, :] = -np.inf                                  # all masked
    lg[1, :] = -np.inf
    lg[1, [5, 17, 30]] = [0.5, 2.0, -1.0]               # 3 finite < k
    lg[2, :] = 1.25                                     # all tied
    lg[3, :] = np.linspace(-1, 1, E)[::-1]
    lg[4, ::2] = -np.inf
    lg[5, :] = np.random.default_rng(3).normal(size=E)
    lg[6, :] = -1.0
    lg[6, [3, 9, 20, 33]] = [-0.0, 0.0, -0.0, 0.0]
    lg[7, :] = np.random.default_rng(4).normal(size=E)
    lg[7, [0, 7, 11, 12, 39]] = np.nan
    lg[8, :] = np.nan
    lg[8, [6, 21, 2]] = [0.25, -3.0, 1.5]
    ids_ref, w_ref = omoe.route(lg, k)
    ids, w = w4.w4_moe_route(up(lg), k)
    ids = down(ids)
    np.testing.assert_array_equal(ids, ids_ref)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
    fin = np.isfinite(w_ref)
    np.testing.assert_allclose(down(w)[fin], w_ref[fin], rtol=2e-6, atol=1e-7)


def test_silu_mul():
    R, I = 37, 96
    say("silu_mul")
    g = torch.Generator().manual_seed(9)
    H1 = (torch.randn((R, 2 * I), generator=g) * 3.0).to(torch.bfloat16)
    H1[0, :4] = torch.tensor([-100.0, 100.0, 0.0, -0.0])
    Hb = synth.bits(H1)
    ref = omoe.silu_mul(Hb)
    A = down_bits(w4.w4_silu_mul(up_bits(Hb)))
    a = bf16.to_f32(A).astype(np.float64)
    # one bf16 rounding of an fp32 result: at most half a bf16 ulp + fp32 noise
    assert np.all(np.abs(a - ref) <= 2.0 ** -8 * np.abs(ref) * 1.0001 + 1e-30)


@pytest.mark.parametrize("weighted", [True, False])
def test_moe_sum(weighted):
    T, k, H = 23, 8, 96
    say(f"moe_sum weighted={weighted}")
    H2b = synth.bits(synth.activations(T * k, H, 5))
    if weighted:
        w = omoe.route(synth.router_logits(T, 64, 5).numpy(), k)[1]
    else:
        w = np.ones((T, k), np.float32)
    ref = omoe.moe_sum(H2b, w)
    out = down_bits(w4.w4_moe_sum(up_bits(H2b), up(w) if weighted else None, T, k))
    o = bf16.to_f32(out).astype(np.float64)
    scale = np.abs(bf16.to_f32(H2b)).max()
    assert np.all(np.abs(o - ref) <= 2.0 ** -8 * np.abs(ref) * 1.0001 + 1e-5 * scale)


@pytest.mark.parametrize("T,k,H", [(23, 8, 96), (70000, 2, 16), (5, 3, 4096)])
def test_moe_sum_vector_and_scalar_paths_agree(T, k, H):
    """H % 8 == 0 with 16-byte aligned rows runs the 16-byte vector kernel
    (T above the grid's y limit loops over tokens); a view 4 bytes off that
    alignment runs the element-pair kernel.  Same sum order: equal bits."""
    say(f"moe_sum paths T={T} k={k} H={H}")
    n = T * k * H
    H2b = synth.bits(synth.activations(T * k, H, 6))
    w = np.random.default_rng(T).random((T, k)).astype(np.float32)
    base = torch.empty(n + 8, dtype=torch.bfloat16, device="cuda")
    out_base = torch.empty(T * H + 8, dtype=torch.bfloat16, device="cuda")
    aligned = base[:n].view(T * k, H)
    shifted = base[2:2 + n].view(T * k, H)              # 4-byte aligned only
    aligned.copy_(up_bits(H2b))
    a = down_bits(w4.w4_moe_sum(aligned, up(w), T, k, out=out_base[:T * H].view(T, H)))
    shifted.copy_(up_bits(H2b))
    b = down_bits(w4.w4_moe_sum(shifted, up(w), T, k, out=out_base[2:2 + T * H].view(T, H)))
    np.testing.assert_array_equal(a, b)
    toks = [0, T // 2, T - 1]
    ref = omoe.moe_sum(H2b.reshape(T, k, H)[toks].reshape(-1, H), w[toks])
    o = bf16.to_f32(a[toks]).astype(np.float64)
    assert np.all(np.abs(o - ref) <= 2.0 ** -8 * np.abs(ref) * 1.0001 + 1e-5 * np.abs(ref).max())


# ------------------------------------------------------------ grouped GEMM --

def small_experts(E, N, K, seed):
    """E experts of bf16 [N, K] -> (GPU Wq [E,N,K/8], GPU S, oracle lookup)."""
    srcs = [synth.bits(synth.weights(N, K, seed, stream=50 + e)) for e in range(E)]
    ref = [quant.quantize_pack(s) for s in srcs]
    Wq = torch.stack([up(r[0]) for r in ref])
    S = torch.stack([up_bits(r[1]) for r in ref])
    # the GPU packing of the same sources must match bit for bit
    for e in range(E):
        q, s = w4.w4_quantize_pack(up_bits(srcs[e]))
        np.testing.assert_array_equal(down(q), ref[e][0])
        np.testing.assert_array_equal(down_bits(s), ref[e][1])
        Wq[e].copy_(q)
        S[e].copy_(s)
    return Wq, S, (lambda e: ref[e])


@pytest.mark.parametrize("B", [1, 4, 16, 20, 32, 64, 200])
@pytest.mark.parametrize("x_row_div_is_k", [True, False])
@pytest.mark.parametrize("weighted", [True, False])
def test_moe_gemm_small(B, x_row_div_is_k, weighted):
    """Blocks of at most 32 rows run the 32-row tile (runs of 32 / B
    blocks), larger ones the 128-row tile (B = 200: two slots per block)."""
    E, T, k, N, K = 6, 40, 3, 96, 160
    say(f"moe_gemm small B={B} div_k={x_row_div_is_k} weighted={weighted}")
    rng = np.random.default_rng(B)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, 0] = -1                      # skipped pair: its row stays untouched
    ids[5, 2] = E + 2
    Wq, S, ref_w = small_experts(E, N, K, 21)
    div = k if x_row_div_is_k else 1
    Xb = synth.bits(synth.activations(T * k // div, K, 22))
    tw = rng.random((T, k)).astype(np.float32) if weighted else None
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    Y = canary_bf16((T * k, N))
    w4.w4a16_moe_gemm(up_bits(Xb), Wq, S, s, e, n, T, k, B, div,
                      topk_weights=None if tw is None else up(tw), out=Y)
    y = down_bits(Y)
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, div, T * k, tw)
    assert sorted(ref) == [f for f in range(T * k) if 0 <= ids.flat[f] < E]
    assert_rows_close(y, ref, "moe small")
    untouched = [f for f in range(T * k) if f not in ref]
    assert np.all(y[untouched] == CANARY)


def random_moe_cases(seed, n):
    """Seeded grouped-product configurations: block sizes on both tiles (32 and
    128 rows), K aligned and not (K % 256), ragged N, skewed and uniform ids,
    dropped pairs, x_row_div of both kinds, weighted or not."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 300))
        B = int(rng.choice([1, 3, 8, 16, 24, 32, 48, 64, 128]))
        N = int(rng.integers(1, 400))
        K = 32 * int(rng.choice([1, 5, 8, 12, 40, 72]))
        out.append((i, E, k, T, B, N, K, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


def extreme_moe_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 5, 64, 300, 1024]))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.choice([1, 3, 40, 500, 2000]))
        B = int(rng.choice([1, 2, 128, 200, 256, 1024]))
        N = int(rng.choice([2, 34, 130, 264]))       # I = N even (w4_silu_mul)
        K = 32 * int(rng.choice([1, 2, 9, 64]))
        out.append((i, E, k, T, B, N, K))
    return out


@pytest.mark.parametrize("case", extreme_moe_cases(4242, 14), ids=lambda c: f"x{c[0]}")
def test_moe_gemm_extreme(case):
    """Block sizes at the ends of the range (B = 1: runs of up to 128 blocks;
    B = 1024: eight slot parts per block), up to 1024 experts, top-16,
    single tokens, K = 32; the plain product and the fused SwiGLU product."""
    i, E, k, T, B, N, K = case
    say(f"moe_gemm extreme {case}")
    rng = np.random.default_rng(2000 + i)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    Wq, S, ref_w = small_experts(E, 2 * N, K, 100 + i)
    Xb = synth.bits(synth.activations(T, K, 101 + i))
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    X = up_bits(Xb)
    H1 = w4.w4a16_moe_gemm(X, Wq, S, s, e, n, T, k, B, k)
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, k, T * k)
    assert len(ref) == T * k
    assert_rows_close(down_bits(H1), ref, "moe extreme")
    A = down_bits(w4.w4a16_moe_gemm_swiglu(X, Wq, S, s, e, n, T, k, B, k))
    np.testing.assert_array_equal(A, down_bits(w4.w4_silu_mul(H1)))


def test_moe_gemm_many_blocks():
    """70000 alignment blocks (B = 1): more slots than one grid dimension of
    65535 holds, in the 1-D grid of N-tiles x slots."""
    E, T, k, N, K, B = 4, 70000, 1, 40, 64, 1
    say("moe_gemm 70000 blocks")
    rng = np.random.default_rng(9)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    Wq, S, ref_w = small_experts(E, N, K, 90)
    Xb = synth.bits(synth.activations(T, K, 91))
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    y = down_bits(w4.w4a16_moe_gemm(up_bits(Xb), Wq, S, s, e, n, T, k, B, 1))
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, 1, T * k)
    assert len(ref) == T
    assert_rows_close(y, ref, "70000 blocks")


@pytest.mark.parametrize("B", [1, 2, 16])
def test_moe_gemm_run_search(B):
    """Few rows per expert (the 32-row tile, whose workgroups index runs of
    up to 32 / B blocks): with B = 1 there are over 1024 blocks (several
    batches of the run search) and a hot expert spans several 64-block
    chunks of it."""
    E, T, k, N, K = 64, 600, 2, 40, 96
    say(f"moe_gemm run search B={B}")
    rng = np.random.default_rng(500 + B)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[:75, 0] = 7                                     # expert 7: >= 75 rows
    ids[:75, 1] = np.where(ids[:75, 1] == 7, 8, ids[:75, 1])
    Wq, S, ref_w = small_experts(E, N, K, 80 + B)
    Xb = synth.bits(synth.activations(T, K, 81))
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    Y = canary_bf16((T * k, N))
    w4.w4a16_moe_gemm(up_bits(Xb), Wq, S, s, e, n, T, k, B, k, out=Y)
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, k, T * k)
    assert len(ref) == T * k
    assert_rows_close(down_bits(Y), ref, f"run search B={B}")


@pytest.mark.parametrize("case", random_moe_cases(77, 16), ids=lambda c: f"r{c[0]}")
def test_moe_gemm_random(case):
    i, E, k, T, B, N, K, div_k, weighted = case
    say(f"moe_gemm random {case}")
    rng = np.random.default_rng(1000 + i)
    p = rng.dirichlet(np.full(E, 0.3))                     # uneven expert loads
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, k)) < 0.05] = -1                   # a few dropped pairs
    Wq, S, ref_w = small_experts(E, N, K, 60 + i)
    div = k if div_k else 1
    Xb = synth.bits(synth.activations(T * k // div, K, 61 + i))
    tw = rng.random((T, k)).astype(np.float32) if weighted else None
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    np.testing.assert_array_equal(down(s), s_ref)
    Y = canary_bf16((T * k, N))
    w4.w4a16_moe_gemm(up_bits(Xb), Wq, S, s, e, n, T, k, B, div,
                      topk_weights=None if tw is None else up(tw), out=Y)
    y = down_bits(Y)
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, div, T * k, tw)
    valid = [f for f in range(T * k) if 0 <= ids.flat[f] < E]
    assert sorted(ref) == valid
    assert_rows_close(y, ref, "moe random")
    untouched = [f for f in range(T * k) if f not in ref]
    assert np.all(y[untouched] == CANARY)


@pytest.mark.parametrize("I,K", [(48, 160), (200, 256), (128, 512)])
@pytest.mark.parametrize("B", [4, 32, 64, 200])
@pytest.mark.parametrize("x_row_div_is_k", [True, False])
def test_moe_gemm_swiglu_small(I, K, B, x_row_div_is_k):
    """gate_up with the SwiGLU fused: equal bit for bit to the unfused pair
    of calls, untouched rows unwritten, and within tolerance of the oracle."""
    E, T, k = 5, 37, 3
    say(f"moe_gemm_swiglu I={I} K={K} B={B} div_k={x_row_div_is_k}")
    rng = np.random.default_rng(100 + B + I)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[1, 1] = -3                      # skipped pair
    Wq, S, ref_w = small_experts(E, 2 * I, K, 41)
    div = k if x_row_div_is_k else 1
    Xb = synth.bits(synth.activations(T * k // div, K, 42))
    X = up_bits(Xb)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    H1 = w4.w4a16_moe_gemm(X, Wq, S, s, e, n, T, k, B, div)
    A_unfused = down_bits(w4.w4_silu_mul(H1))
    A = canary_bf16((T * k, I))
    w4.w4a16_moe_gemm_swiglu(X, Wq, S, s, e, n, T, k, B, div, out=A)
    a = down_bits(A)
    valid = [f for f in range(T * k) if 0 <= ids.flat[f] < E]
    np.testing.assert_array_equal(a[valid], A_unfused[valid])
    untouched = [f for f in range(T * k) if f not in valid]
    assert np.all(a[untouched] == CANARY)
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    h = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, div, T * k)
    ref = {f: omoe.silu(r[:I]) * r[I:] for f, r in h.items()}
    assert_rows_close(a, ref, "moe swiglu small")


def test_moe_gemm_one_expert_is_dense():
    """E = 1, k = 1: the grouped product is the dense product of all rows."""
    T, N, K = 300, 100, 544
    say("moe_gemm E=1 k=1")
    Wq, S, ref_w = small_experts(1, N, K, 31)
    Xb = synth.bits(synth.activations(T, K, 32))
    ids = np.zeros((T, 1), np.int32)
    s, e, n = w4.moe_align_block_size(up(ids), 1, 16)
    y = down_bits(w4.w4a16_moe_gemm(up_bits(Xb), Wq, S, s, e, n, T, 1, 16, 1))
    Wq_r, S_r = ref_w(0)
    ok, a, r = gemm.within_tolerance(y, gemm.w4a16_gemm(Xb, Wq_r, S_r), ATOL, RTOL)
    assert ok, (a, r)


# --------------------------------------------------- full-size MoE layers --

class Experts:
    """Full-size stacked experts quantized on the GPU from GPU-drawn sources.
    ``sources(e)`` downloads expert e's bf16 sources and the GPU's packing
    of them; the oracle quantizes the sources itself (``oracle_pack``)."""

    def __init__(self, wl):
        self.wl = wl
        H, I, E, seed = wl["H"], wl["I"], wl["E"], wl["seed"]
        dev = torch.device("cuda")
        self.gate_up = wmoe.quantize_experts(
            E, 2 * I, H, lambda e: synth.expert_gate_up(e, I, H, seed, dev), dev)
        self.down = wmoe.quantize_experts(
            E, H, I, lambda e: synth.expert_down(e, I, H, seed, dev), dev)

    def sources(self, e):
        H, I, seed = self.wl["H"], self.wl["I"], self.wl["seed"]
        dev = torch.device("cuda")
        out = {}
        for kind, draw, st in (("gate_up", synth.expert_gate_up, self.gate_up),
                               ("down", synth.expert_down, self.down)):
            out[kind] = (synth.bits(draw(e, I, H, seed, dev)), down(st.Wq[e]), down_bits(st.S[e]))
        return out


def oracle_pack(src):
    """The oracle's packing of one expert's sources, asserted equal to the
    GPU's (bit-exact quantize + pack on the full-size expert weights)."""
    packed = {}
    for kind, (w_bits, gpu_wq, gpu_s) in src.items():
        Wq, S = quant.quantize_pack(w_bits)
        np.testing.assert_array_equal(gpu_wq, Wq, err_msg=f"{kind} codes")
        np.testing.assert_array_equal(gpu_s, S, err_msg=f"{kind} scales")
        packed[kind] = (Wq, S)
    return packed


def oracle_threads():
    """Threads for the per-expert oracle work (numpy releases the GIL in its
    array operations); the GPU machine gives a process 16 CPUs."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_layer(name, B_list, n_random_experts=None, n_tokens=None):
    """Full-size layer: alignment bit-exact over the whole buffers for each
    B; every grouped gate_up row (each B) and down row of the checked
    experts; the fused SwiGLU equal to the unfused pair bit for bit; the
    layer output of the checked tokens.  ``n_random_experts`` / ``n_tokens``
    None: every expert and every token; otherwise the skew's hot experts
    plus that many seeded random experts, and the first and last token
    plus seeded random tokens up to ``n_tokens``."""
    wl = synth.WORKLOADS[name]
    T, E, k, H, I, seed = wl["T"], wl["E"], wl["k"], wl["H"], wl["I"], wl["seed"]
    say(f"moe layer {name}: drawing and quantizing {E} experts")
    ex = Experts(wl)
    lg = synth.router_logits(T, E, seed, wl["skew"]).numpy()
    ids, tw = omoe.route(lg, k)
    Xb = synth.bits(synth.activations(T, H, seed))
    X = up_bits(Xb)
    rng = np.random.default_rng(seed)
    if n_random_experts is None:
        checked = set(range(E))
    else:
        hot = set(synth.hot_experts(T, E, seed, wl["skew"])) if wl["skew"] else set()
        pool = [e for e in range(E) if e not in hot]
        checked = hot | {int(e) for e in rng.choice(pool, n_random_experts, replace=False)}
    if n_tokens is None:
        toks = list(range(T))
    else:
        toks = sorted({0, T - 1, *map(int, rng.choice(np.arange(1, T - 1), n_tokens - 2,
                                                       replace=False))})
    h1_by_B = {}
    for B in B_list:
        say(f"moe layer {name}: B={B}")
        s_ref, e_ref, n_ref = omoe.align(ids, E, B)
        out, buf = wmoe.moe_forward(X, up(ids), up(tw), ex.gate_up, ex.down, B=B, fused=False)
        np.testing.assert_array_equal(down(buf.sorted_token_ids), s_ref)
        np.testing.assert_array_equal(down(buf.expert_ids), e_ref)
        assert int(down(buf.ntpp)[0]) == n_ref
        h1_by_B[B] = down_bits(buf.H1)
        # the fused gate_up + SwiGLU gives the unfused A bit for bit
        a_unfused = down_bits(buf.A)
        del buf, out
        A = w4.w4a16_moe_gemm_swiglu(X, ex.gate_up.Wq, ex.gate_up.S, *map(
            up, (s_ref, e_ref, np.array([n_ref], np.int32))), T, k, B, k)
        np.testing.assert_array_equal(down_bits(A), a_unfused)
        del A, a_unfused
    # down projection on its own, on seeded activations
    say(f"moe layer {name}: down projection")
    B0 = B_list[0]
    s_ref, e_ref, n_ref = omoe.align(ids, E, B0)
    Ab = synth.bits(synth.activations(T * k, I, seed, stream=77))
    s, e, n = w4.moe_align_block_size(up(ids), E, B0)
    h2 = down_bits(w4.w4a16_moe_gemm(up_bits(Ab), ex.down.Wq, ex.down.S, s, e, n, T, k, B0, 1))
    say(f"moe layer {name}: layer output")
    o = down_bits(wmoe.moe_forward(X, up(ids), up(tw), ex.gate_up, ex.down, B=B0)[0])

    pairs = omoe.pairs_by_expert(ids, toks)
    todo = sorted(checked | set(pairs))
    say(f"moe layer {name}: oracle over {len(todo)} experts ({len(checked)} with every row), "
        f"{len(toks)} tokens, {oracle_threads()} threads")
    n_rows = collections.Counter()

    def check_expert(e, src):
        packed = oracle_pack(src)
        h2_layer, rows = {}, collections.Counter()
        if e in checked:
            ref = omoe.grouped_gemm(Xb, lambda _: packed["gate_up"], s_ref, e_ref, n_ref, B0, k,
                                    T * k, experts={e})
            for B, h1 in h1_by_B.items():
                assert_rows_close(h1, ref, f"{name} gate_up expert {e} B={B}")
            rows["gate_up"] += len(ref)
            ref = omoe.grouped_gemm(Ab, lambda _: packed["down"], s_ref, e_ref, n_ref, B0, 1,
                                    T * k, experts={e})
            assert_rows_close(h2, ref, f"{name} down expert {e}")
            rows["down"] += len(ref)
        if e in pairs:
            h2_layer = omoe.expert_h2(Xb, pairs[e], packed["gate_up"], packed["down"])
        return h2_layer, rows

    h2_layer = {}

    def collect(fut):
        got, rows = fut.result()
        h2_layer.update(got)
        n_rows.update(rows)

    with concurrent.futures.ThreadPoolExecutor(oracle_threads()) as pool:
        futs = collections.deque()
        for e in todo:
            futs.append(pool.submit(check_expert, e, ex.sources(e)))
            while len(futs) >= 2 * oracle_threads():      # bound the sources held at once
                collect(futs.popleft())
        while futs:
            collect(futs.popleft())
    say(f"moe layer {name}: rows checked gate_up {n_rows['gate_up']} down {n_rows['down']}")
    ref = omoe.combine_tokens(tw, h2_layer, toks)
    assert_rows_close(o, ref, f"{name} layer output over {len(toks)} tokens")
    if n_random_experts is None:
        assert n_rows["gate_up"] == n_rows["down"] == int(np.sum((ids >= 0) & (ids < E)))


@pytest.mark.timeout(900)
def test_moe_qwen_layer():
    """128-expert layer: every expert, every row, every token."""
    run_layer("moe_qwen", [16, 32, 64])


@pytest.mark.timeout(900)
def test_moe_kimi_layer():
    """384-expert skewed layer: all rows of the 8 hot experts and 24 random
    ones, and the layer output of 64 tokens."""
    run_layer("moe_kimi", [64], n_random_experts=24, n_tokens=64)
