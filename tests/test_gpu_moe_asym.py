"""GPU parity: the grouped products with zero-point experts
(w4a16_moe_gemm_asym, w4a16_moe_gemm_swiglu_asym) and a routed layer built
on them, against the oracle.

* Per element |y - y_ref| <= 2e-2 + 1e-2 |y_ref| against the fp64 product
  of the oracle's own dequantization w' = bf16((q - z) s).
* Integer experts (every group spans exactly [lo, lo + 15], so s = 1 and
  z = -lo, with lo drawn per group) and integer activations keep every sum
  exact: the output must equal the textbook integer product bit for bit.
* The fused SwiGLU form equals the unfused pair of calls bit for bit.
* Both tile shapes run: blocks of at most 32 rows with few rows per expert
  take the 32-row tile, larger blocks or more rows per expert the 128-row
  tile; K a multiple of 256 and not (the byte-wise zero-point loads).
The GPU quantizes the same bf16 sources and its packing is asserted equal
to the oracle's before any product is compared.
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
from int4_weight_only_amd import moe as wmoe
import synth
from gpu_util import CANARY, canary_bf16, down, down_bits, say, up, up_bits
from oracle import bf16, gemm, quant_asym
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def assert_rows_close(y_bits, ref_rows, label):
    assert ref_rows, f"{label}: nothing to compare"
    fs = sorted(ref_rows)
    ref = np.stack([ref_rows[f] for f in fs])
    ok, max_abs, max_rel = gemm.within_tolerance(y_bits[fs], ref, ATOL, RTOL)
    assert ok, f"{label}: max abs {max_abs:.3e}, max rel {max_rel:.3e} over {len(fs)} rows"


def stack_experts(srcs):
    """bf16 bit sources -> (GPU Wq [E,N,K/8], S, Z, oracle lookup)."""
    ref = [quant_asym.quantize_pack_asym(s) for s in srcs]
    got = [w4.w4_quantize_pack_asym(up_bits(s)) for s in srcs]
    for (q, s, z), (q_r, s_r, z_r) in zip(got, ref):
        np.testing.assert_array_equal(down(q), q_r)
        np.testing.assert_array_equal(down_bits(s), s_r)
        np.testing.assert_array_equal(down(z), z_r)
    Wq = torch.stack([g[0] for g in got])
    S = torch.stack([g[1] for g in got])
    Z = torch.stack([g[2] for g in got])
    return Wq, S, Z, (lambda e: ref[e])


def random_experts(E, N, K, seed):
    return stack_experts([synth.bits(synth.weights(N, K, seed, stream=70 + e)) for e in range(E)])


def integer_expert(rng, N, K):
    G = K // 32
    lo = rng.integers(-15, 1, size=(N, G, 1)).astype(np.float32)
    w = lo + rng.integers(0, 16, size=(N, G, 32)).astype(np.float32)
    w[:, :, 2] = lo[:, :, 0]
    w[:, :, 30] = lo[:, :, 0] + 15.0
    return w.reshape(N, K)


@pytest.mark.parametrize("B", [1, 4, 16, 32, 64, 200])
@pytest.mark.parametrize("K", [160, 512])
@pytest.mark.parametrize("x_row_div_is_k", [True, False])
@pytest.mark.parametrize("weighted", [True, False])
def test_moe_gemm_asym_small(B, K, x_row_div_is_k, weighted):
    E, T, k, N = 6, 40, 3, 96
    say(f"moe_gemm_asym B={B} K={K} div_k={x_row_div_is_k} weighted={weighted}")
    rng = np.random.default_rng(300 + B + K)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, 1] = -1                      # skipped pairs: their rows stay untouched
    ids[7, 0] = E
    Wq, S, Z, ref_w = random_experts(E, N, K, 23)
    div = k if x_row_div_is_k else 1
    Xb = synth.bits(synth.activations(T * k // div, K, 24))
    tw = rng.random((T, k)).astype(np.float32) if weighted else None
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    Y = canary_bf16((T * k, N))
    w4.w4a16_moe_gemm_asym(up_bits(Xb), Wq, S, Z, s, e, n, T, k, B, div,
                           topk_weights=None if tw is None else up(tw), out=Y)
    y = down_bits(Y)
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, div, T * k, tw)
    assert sorted(ref) == [f for f in range(T * k) if 0 <= ids.flat[f] < E]
    assert_rows_close(y, ref, "moe asym")
    untouched = [f for f in range(T * k) if f not in ref]
    assert np.all(y[untouched] == CANARY)


@pytest.mark.parametrize("B", [4, 32, 64, 200])
@pytest.mark.parametrize("I,K", [(48, 160), (128, 512)])
def test_moe_gemm_swiglu_asym_small(B, I, K):
    E, T, k = 5, 37, 3
    say(f"moe_gemm_swiglu_asym I={I} K={K} B={B}")
    rng = np.random.default_rng(400 + B + I)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[2, 2] = -5
    Wq, S, Z, ref_w = random_experts(E, 2 * I, K, 43)
    Xb = synth.bits(synth.activations(T, K, 44))
    X = up_bits(Xb)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    H1 = w4.w4a16_moe_gemm_asym(X, Wq, S, Z, s, e, n, T, k, B, k)
    A_unfused = down_bits(w4.w4_silu_mul(H1))
    A = canary_bf16((T * k, I))
    w4.w4a16_moe_gemm_swiglu_asym(X, Wq, S, Z, s, e, n, T, k, B, k, out=A)
    a = down_bits(A)
    valid = [f for f in range(T * k) if 0 <= ids.flat[f] < E]
    np.testing.assert_array_equal(a[valid], A_unfused[valid])
    assert np.all(a[[f for f in range(T * k) if f not in valid]] == CANARY)
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    h = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, k, T * k)
    ref = {f: omoe.silu(r[:I]) * r[I:] for f, r in h.items()}
    assert_rows_close(a, ref, "moe swiglu asym")


@pytest.mark.parametrize("T,E,k,B", [(40, 6, 3, 16), (300, 4, 2, 64)])
@pytest.mark.parametrize("K", [1056, 2048])
def test_moe_gemm_asym_integer_exact(T, E, k, B, K):
    """Zero points 0..15 varying by row, group and expert; integer
    activations: the grouped rows equal the integer product bit for bit
    (the first case runs the 32-row tile, the second the 128-row tile)."""
    N = 64
    say(f"moe_gemm_asym integer-exact T={T} E={E} B={B} K={K}")
    rng = np.random.default_rng(500 + T + K)
    ws = [integer_expert(rng, N, K) for _ in range(E)]
    Wq, S, Z, ref_w = stack_experts([bf16.rne(w) for w in ws])
    for e in range(E):
        assert np.all(bf16.to_f32(ref_w(e)[1]) == 1.0)
    assert len(np.unique(down(Z))) == 16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = rng.integers(-2, 3, size=(T, K)).astype(np.float32)
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    y = down_bits(w4.w4a16_moe_gemm_asym(up_bits(bf16.rne(x)), Wq, S, Z, s, e, n, T, k, B, k))
    for f in range(T * k):
        ex = int(ids.reshape(-1)[f])
        exact = x[f // k].astype(np.float64) @ ws[ex].astype(np.float64).T
        np.testing.assert_array_equal(y[f], gemm.to_bf16(exact), err_msg=f"row {f}")


def layer_case(T, E, k, H, I, seed, B):
    """A routed layer with zero-point experts through ``moe_forward``
    (fused and unfused), checked stage by stage and at the output."""
    dev = torch.device("cuda")
    srcs_gu = [synth.bits(synth.expert_gate_up(e, I, H, seed, dev)) for e in range(E)]
    srcs_dn = [synth.bits(synth.expert_down(e, I, H, seed, dev)) for e in range(E)]
    gWq, gS, gZ, ref_gu = stack_experts(srcs_gu)
    dWq, dS, dZ, ref_dn = stack_experts(srcs_dn)
    gate_up = wmoe.ExpertWeights(gWq, gS, gZ)
    down_w = wmoe.ExpertWeights(dWq, dS, dZ)
    lg = synth.router_logits(T, E, seed).numpy()
    ids, tw = omoe.route(lg, k)
    Xb = synth.bits(synth.activations(T, H, seed))
    X = up_bits(Xb)
    out_u, buf = wmoe.moe_forward(X, up(ids), up(tw), gate_up, down_w, B=B, fused=False)
    o_u = down_bits(out_u)
    a_u = down_bits(buf.A)
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    ref_h1 = omoe.grouped_gemm(Xb, ref_gu, s_ref, e_ref, n_ref, B, k, T * k)
    assert_rows_close(down_bits(buf.H1), ref_h1, "asym layer gate_up")
    out_f, buf_f = wmoe.moe_forward(X, up(ids), up(tw), gate_up, down_w, B=B, fused=True)
    np.testing.assert_array_equal(down_bits(buf_f.A), a_u)
    np.testing.assert_array_equal(down_bits(out_f), o_u)
    ref = omoe.moe_layer(Xb, ids, tw, ref_gu, ref_dn)
    assert_rows_close(o_u, ref, "asym layer output")


@pytest.mark.parametrize("T,E,k,H,I,B", [(64, 16, 4, 256, 128, 16), (512, 8, 2, 512, 256, 64)])
def test_moe_layer_asym(T, E, k, H, I, B):
    say(f"moe layer asym T={T} E={E} k={k} H={H} I={I} B={B}")
    layer_case(T, E, k, H, I, 13, B)


@pytest.mark.parametrize("T,E,k,N,K,B", [(5, 1024, 4, 1, 32, 1), (300, 3, 1, 17, 96, 1),
                                         (64, 7, 3, 130, 4640, 128), (1, 2, 2, 64, 256, 1024)])
def test_moe_gemm_asym_extreme(T, E, k, N, K, B):
    """The most experts, one weight row, one group, blocks of one row and of
    1024 rows, K past 4096 with K / 32 off a multiple of 8."""
    say(f"moe_gemm_asym extreme T={T} E={E} k={k} N={N} K={K} B={B}")
    rng = np.random.default_rng(T + E + N + K + B)
    used = min(E, 6)
    Wq, S, Z, ref_w = random_experts(used, N, K, 90)
    if E > used:   # experts that no pair routes to: zero codes, scales and zero points
        pad = E - used
        Wq = torch.cat([Wq, torch.zeros((pad,) + tuple(Wq.shape[1:]), dtype=Wq.dtype, device=Wq.device)])
        S = torch.cat([S, torch.zeros((pad,) + tuple(S.shape[1:]), dtype=S.dtype, device=S.device)])
        Z = torch.cat([Z, torch.zeros((pad,) + tuple(Z.shape[1:]), dtype=Z.dtype, device=Z.device)])
    ids = rng.integers(0, used, size=(T, k)).astype(np.int32)
    Xb = synth.bits(synth.activations(T, K, 91))
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    Y = canary_bf16((T * k, N))
    w4.w4a16_moe_gemm_asym(up_bits(Xb), Wq, S, Z, s, e, n, T, k, B, k, out=Y)
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    ref = omoe.grouped_gemm(Xb, ref_w, s_ref, e_ref, n_ref, B, k, T * k)
    assert_rows_close(down_bits(Y), ref, "moe asym extreme")
