"""GPU parity: the kernel-order layouts of the codes (w4_repack /
w4_restore) and of the per-group scales and zero points (w4_repack_groups /
w4_restore_groups), and the products that read them.

* w4_repack and w4_repack_groups are bit-exact against the oracle's layouts
  (oracle/layout.py), padding included; restore(repack(x)) == x bit for bit.
* Every *_tiled product equals the canonical-layout call bit for bit (the
  same arithmetic in the same order; only the addresses differ): the
  decode kernels (M <= 32), the tiled product, the grouped products of both
  tile shapes with and without the fused SwiGLU, symmetric and zero-point
  codes, ragged N and K (K % 64 == 32 leaves half of the last 64-wide step
  empty), and the full-size workloads.  The canonical calls are themselves
  checked against the fp64 oracle elsewhere; one direct oracle comparison
  per kernel family is repeated here.
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
from int4_weight_only_amd import moe as wmoe
import synth
from gpu_util import down, down_bits, say, up, up_bits
from oracle import gemm, layout, quant
from oracle import moe as omoe

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def codes(N, K, seed, asym=False, E=None):
    shape = (N, K) if E is None else (E * N, K)
    W = synth.weights(*shape, seed).cuda()
    if asym:
        Wq, S, Z = w4.w4_quantize_pack_asym(W)
    else:
        (Wq, S), Z = w4.w4_quantize_pack(W), None
    if E is not None:
        Wq, S = Wq.view(E, N, K // 8), S.view(E, N, K // 32)
        Z = None if Z is None else Z.view(E, N, K // 32)
    return Wq, S, Z


@pytest.mark.parametrize("E,N,K", [(1, 1, 32), (1, 31, 96), (1, 33, 64), (3, 100, 544),
                                   (2, 64, 4096), (1, 12288, 4096), (128, 3072, 64)])
def test_repack_bit_exact_and_restore(E, N, K):
    say(f"repack E={E} N={N} K={K}")
    Wq, _, _ = codes(N, K, E + N + K, E=E)
    Wt = w4.w4_repack(Wq)
    got = down(Wt)
    np.testing.assert_array_equal(got, layout.repack(down(Wq)))
    back = w4.w4_restore(Wt, N, K)
    np.testing.assert_array_equal(down(back).reshape(E, N, K // 8), down(Wq))


def test_restore_ignores_padding_and_leaves_other_memory():
    """Padding units of the kernel-order buffer (rows past N, groups past
    K) are never read back: poison them and restore still gives Wq."""
    N, K = 45, 96
    say("restore with poisoned padding")
    Wq, _, _ = codes(N, K, 3)
    Wt = w4.w4_repack(Wq)
    n, g, valid = layout._unit_map(N, K)
    pad_words = np.repeat(~valid, 4)
    Wt.view(-1)[up(np.nonzero(pad_words)[0].astype(np.int64))] = 0x5A5A5A5A
    out = torch.full((N + 2, K // 8), 0x77, dtype=torch.int32, device="cuda")
    w4.w4_restore(Wt, N, K, out=out[1:N + 1])
    o = down(out)
    np.testing.assert_array_equal(o[1:N + 1], down(Wq))
    assert np.all(o[0] == 0x77) and np.all(o[N + 1] == 0x77)


def down_raw(t):
    """The tensor's bits as numpy (bf16 as int16)."""
    return down(t.view(torch.int16) if t.dtype == torch.bfloat16 else t)


def tiled(S, Z):
    """Scales and zero points in kernel order."""
    return w4.w4_repack_groups(S), (None if Z is None else w4.w4_repack_groups(Z))


@pytest.mark.parametrize("E,N,K", [(1, 1, 32), (1, 31, 96), (1, 33, 288), (3, 100, 544),
                                   (2, 64, 4096), (1, 12288, 4096), (128, 3072, 2048),
                                   (1, 17, 8192)])
def test_repack_groups_bit_exact_and_restore(E, N, K):
    say(f"repack groups E={E} N={N} K={K}")
    _, S, Z = codes(N, K, E + N + K + 1, asym=True, E=E)
    for A in (S, Z):
        At = w4.w4_repack_groups(A)
        assert tuple(At.shape) == (E, layout.repacked_group_elems(N, K))
        ref = layout.repack_groups(down_raw(A).reshape(E, N, K // 32), K)
        np.testing.assert_array_equal(down_raw(At), ref)
        back = w4.w4_restore_groups(At, N, K)
        np.testing.assert_array_equal(down_raw(back).reshape(E, N, K // 32), down_raw(A))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.uint8])
def test_repack_groups_any_alignment(dtype):
    """Buffers one element off a whole piece take the element-wise kernel;
    the result is the same bits as from aligned buffers (K/32 % 8 == 0, so
    aligned buffers take the vector kernel)."""
    E, N, K = 2, 37, 512
    say(f"repack groups unaligned {dtype}")
    _, S, Z = codes(N, K, 9, asym=True, E=E)
    A = S if dtype == torch.bfloat16 else Z
    ref = down_raw(w4.w4_repack_groups(A))
    flat = torch.zeros(A.numel() + 1, dtype=dtype, device="cuda")
    src = flat[1:].view(E, N, K // 32)
    src.copy_(A)
    out = torch.zeros(E * layout.repacked_group_elems(N, K) + 1, dtype=dtype, device="cuda")
    w4.w4_repack_groups(src, out=out[1:])
    np.testing.assert_array_equal(down_raw(out[1:]).reshape(ref.shape), ref)
    back = torch.zeros(A.numel() + 1, dtype=dtype, device="cuda")
    w4.w4_restore_groups(out[1:], N, K, out=back[1:])
    np.testing.assert_array_equal(down_raw(back[1:]), down_raw(A).reshape(-1))


def test_restore_groups_ignores_padding_and_leaves_other_memory():
    """Padding elements of the kernel-order scales (rows past N, groups past
    K) are never read back: poison them and restore still gives S."""
    N, K = 45, 96 + 32 * 8
    say("restore groups with poisoned padding")
    _, S, _ = codes(N, K, 4)
    St = w4.w4_repack_groups(S)
    _, _, valid = layout._group_map(N, K)
    St.view(torch.int16).view(-1)[up(np.nonzero(~valid)[0].astype(np.int64))] = 0x5A5A
    out = torch.full((N + 2, K // 32), 7.0, dtype=torch.bfloat16, device="cuda")
    w4.w4_restore_groups(St, N, K, out=out[1:N + 1])
    o = down_raw(out)
    np.testing.assert_array_equal(o[1:N + 1], down_raw(S))
    seven = down_raw(torch.full((1,), 7.0, dtype=torch.bfloat16, device="cuda"))[0]
    assert np.all(o[0] == seven) and np.all(o[N + 1] == seven)


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 12288, 4096), (8, 12288, 4096), (16, 12288, 4096),
                                   (32, 12288, 4096), (17, 45, 544), (5, 300, 96), (33, 300, 96),
                                   (1, 48, 65536), (64, 1000, 4096), (200, 257, 544),
                                   (4096, 14336, 4096)])
def test_dense_tiled_equals_canonical(asym, M, N, K):
    say(f"gemm tiled asym={asym} M={M} N={N} K={K}")
    Wq, S, Z = codes(N, K, M + N + K, asym)
    X = synth.activations(M, K, M + 1).cuda()
    ref = w4.w4a16_gemm_asym(X, Wq, S, Z) if asym else w4.w4a16_gemm(X, Wq, S)
    Wt = w4.w4_repack(Wq)
    St, Zt = tiled(S, Z)
    y = w4.w4a16_gemm_tiled(X, Wt, St, N, Z=Zt)
    np.testing.assert_array_equal(down_bits(y), down_bits(ref))


@pytest.mark.parametrize("M", [1, 32, 300])
def test_dense_tiled_against_oracle(M):
    N, K = 333, 4128
    say(f"gemm tiled vs oracle M={M}")
    Wb = synth.bits(synth.weights(N, K, 90 + M))
    Xb = synth.bits(synth.activations(M, K, 91 + M))
    Wq_ref, S_ref = quant.quantize_pack(Wb)
    Wt = w4.w4_repack(up(Wq_ref))
    np.testing.assert_array_equal(down(Wt), layout.repack(Wq_ref))
    St = up_bits(layout.repack_groups(S_ref, K))
    y = down_bits(w4.w4a16_gemm_tiled(up_bits(Xb), Wt, St, N))
    ok, a, r = gemm.within_tolerance(y, gemm.w4a16_gemm(Xb, Wq_ref, S_ref), ATOL, RTOL)
    assert ok, (a, r)


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("T,E,k,N,K,B", [(96, 12, 4, 96, 544, 16), (96, 12, 4, 64, 4096, 32),
                                         (300, 8, 2, 160, 1056, 64), (40, 5, 3, 45, 96, 4),
                                         (200, 4, 2, 256, 4096, 200)])
def test_grouped_tiled_equals_canonical(asym, T, E, k, N, K, B):
    say(f"moe tiled asym={asym} T={T} E={E} k={k} N={N} K={K} B={B}")
    Wq, S, Z = codes(N, K, T + N + K, asym, E=E)
    ids = synth.random_ids(T, k, E, T + E).cuda()
    s, e, n = w4.moe_align_block_size(ids, E, B)
    tw = torch.rand(T * k, generator=torch.Generator().manual_seed(5)).cuda()
    Wt = w4.w4_repack(Wq)
    St, Zt = tiled(S, Z)
    X = synth.activations(T, K, 7).cuda()
    X1 = synth.activations(T * k, K, 8).cuda()
    valid = down(ids).reshape(-1)
    rows = np.nonzero((valid >= 0) & (valid < E))[0]
    if asym:
        ref_gu = w4.w4a16_moe_gemm_asym(X, Wq, S, Z, s, e, n, T, k, B, k)
        ref_dn = w4.w4a16_moe_gemm_asym(X1, Wq, S, Z, s, e, n, T, k, B, 1, topk_weights=tw)
    else:
        ref_gu = w4.w4a16_moe_gemm(X, Wq, S, s, e, n, T, k, B, k)
        ref_dn = w4.w4a16_moe_gemm(X1, Wq, S, s, e, n, T, k, B, 1, topk_weights=tw)
    gu = w4.w4a16_moe_gemm_tiled(X, Wt, St, N, s, e, n, T, k, B, k, Z=Zt)
    dn = w4.w4a16_moe_gemm_tiled(X1, Wt, St, N, s, e, n, T, k, B, 1, Z=Zt, topk_weights=tw)
    np.testing.assert_array_equal(down_bits(gu)[rows], down_bits(ref_gu)[rows])
    np.testing.assert_array_equal(down_bits(dn)[rows], down_bits(ref_dn)[rows])
    if N % 2 == 0:
        if asym:
            ref_a = w4.w4a16_moe_gemm_swiglu_asym(X, Wq, S, Z, s, e, n, T, k, B, k)
        else:
            ref_a = w4.w4a16_moe_gemm_swiglu(X, Wq, S, s, e, n, T, k, B, k)
        a = w4.w4a16_moe_gemm_swiglu_tiled(X, Wt, St, N, s, e, n, T, k, B, k, Z=Zt)
        np.testing.assert_array_equal(down_bits(a)[rows], down_bits(ref_a)[rows])


def test_grouped_tiled_against_oracle():
    T, E, k, N, K, B = 64, 6, 2, 96, 544, 16
    say("moe tiled vs oracle")
    srcs = [synth.bits(synth.weights(N, K, 70, stream=60 + e)) for e in range(E)]
    ref = [quant.quantize_pack(b) for b in srcs]
    Wt = up(layout.repack(np.stack([r[0] for r in ref])))
    St = up_bits(layout.repack_groups(np.stack([r[1] for r in ref]), K))
    ids = synth.random_ids(T, k, E, 71).numpy()
    s_ref, e_ref, n_ref = omoe.align(ids, E, B)
    Xb = synth.bits(synth.activations(T, K, 72))
    s, e, n = w4.moe_align_block_size(up(ids), E, B)
    y = down_bits(w4.w4a16_moe_gemm_tiled(up_bits(Xb), Wt, St, N, s, e, n, T, k, B, k))
    rows = omoe.grouped_gemm(Xb, lambda x: ref[x], s_ref, e_ref, n_ref, B, k, T * k)
    fs = sorted(rows)
    ok, a, r = gemm.within_tolerance(y[fs], np.stack([rows[f] for f in fs]), ATOL, RTOL)
    assert ok, (a, r)


@pytest.mark.parametrize("name", ["moe_qwen", "moe_kimi"])
def test_full_layers_tiled_equal_canonical(name):
    """The full-size expert layers: the fused gate_up + SwiGLU and the down
    product on kernel-order experts equal the canonical ones bit for bit."""
    wl = synth.WORKLOADS[name]
    T, E, k, H, I, seed = wl["T"], wl["E"], wl["k"], wl["H"], wl["I"], wl["seed"]
    say(f"tiled full layer {name}")
    dev = torch.device("cuda")
    gu = wmoe.quantize_experts(E, 2 * I, H, lambda e: synth.expert_gate_up(e, I, H, seed, dev), dev)
    dn = wmoe.quantize_experts(E, H, I, lambda e: synth.expert_down(e, I, H, seed, dev), dev)
    X = synth.activations(T, H, seed, device=dev)
    ids, tw = w4.w4_moe_route(synth.router_logits(T, E, seed, wl["skew"], device=dev), k)
    B = w4.w4_pick_block_size(T, k, E)
    s, e, n = w4.moe_align_block_size(ids, E, B)
    A = w4.w4a16_moe_gemm_swiglu(X, gu.Wq, gu.S, s, e, n, T, k, B, k)
    H2 = w4.w4a16_moe_gemm(A, dn.Wq, dn.S, s, e, n, T, k, B, 1)
    gu_t = wmoe.repack_experts(gu, keep_canonical=True)
    dn_t = wmoe.repack_experts(dn)
    A_t = wmoe.grouped_gemm_swiglu(X, gu_t, s, e, n, T, k, B, k)
    np.testing.assert_array_equal(down_bits(A_t), down_bits(A))
    H2_t = wmoe.grouped_gemm(A, dn_t, s, e, n, T, k, B, 1)
    np.testing.assert_array_equal(down_bits(H2_t), down_bits(H2))
    # and back: restore gives the canonical experts
    np.testing.assert_array_equal(
        down(w4.w4_restore(gu_t.Wt, 2 * I, H)).reshape(E, 2 * I, H // 8), down(gu.Wq))
    np.testing.assert_array_equal(
        down_raw(w4.w4_restore_groups(gu_t.St, 2 * I, H)).reshape(E, 2 * I, H // 32),
        down_raw(gu.S))
