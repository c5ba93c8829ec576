"""HIP graph capture of library calls.

With its outputs preallocated, every entry point only enqueues kernels on
the caller's current stream: no device allocation, no host synchronization,
no memset.  So a decode or prefill product, and a whole routed MoE layer,
can be captured once and replayed, which removes the per-call host cost from
a decode loop.  Each test replays its graph several times, copies new
inputs in with eager work and synchronizes between replays, and checks
every replay bit for bit against the same calls run eagerly.
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
from int4_weight_only_amd import moe as wmoe
import synth
from gpu_util import down_bits, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def capture(fn):
    """Warm fn up on a side stream (first-call host setup), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("M", [1, 16, 32, 64])
@pytest.mark.parametrize("asym", [False, True])
def test_gemm_graph_replay(M, asym):
    N, K = 1024, 4096
    say(f"graph gemm M={M} asym={asym}")
    W = synth.weights(N, K, 9, device=DEV)
    if asym:
        Wq, S, Z = w4.w4_quantize_pack_asym(W)
        call = lambda X, Y: w4.w4a16_gemm_asym(X, Wq, S, Z, out=Y)
    else:
        Wq, S = w4.w4_quantize_pack(W)
        call = lambda X, Y: w4.w4a16_gemm(X, Wq, S, out=Y)
    X = synth.activations(M, K, 10, device=DEV)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    g = capture(lambda: call(X, Y))
    for r in range(4):
        X.copy_(synth.activations(M, K, 20 + r, device=DEV))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        Y_eager = torch.empty_like(Y)
        call(X, Y_eager)
        np.testing.assert_array_equal(down_bits(Y), down_bits(Y_eager), err_msg=f"replay {r}")


def test_quantize_graph_replay():
    N, K = 512, 2048
    W = synth.weights(N, K, 12, device=DEV)
    Wq = torch.empty((N, K // 8), dtype=torch.int32, device=DEV)
    S = torch.empty((N, K // 32), dtype=torch.bfloat16, device=DEV)
    Wf = torch.empty_like(W)

    def step():
        w4.w4_quantize_pack(W, Wq, S)
        w4.w4_fake_quant(W, out=Wf)
    g = capture(step)
    for r in range(3):
        W.copy_(synth.weights(N, K, 30 + r, device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        q2, s2 = w4.w4_quantize_pack(W)
        np.testing.assert_array_equal(Wq.cpu().numpy(), q2.cpu().numpy())
        np.testing.assert_array_equal(down_bits(S), down_bits(s2))
        np.testing.assert_array_equal(down_bits(Wf), down_bits(w4.w4_fake_quant(W)))


@pytest.mark.parametrize("T,E,k,asym", [(64, 16, 4, False), (7, 8, 2, False), (64, 16, 4, True)])
def test_moe_layer_graph_replay(T, E, k, asym):
    """Routing, alignment, the fused gate_up + SwiGLU, down and combine in
    one graph (the block count lives on the device, so the launches do not
    depend on the routing); symmetric and zero-point experts."""
    H, I, seed = 512, 256, 11
    say(f"graph moe T={T} E={E} k={k} asym={asym}")
    gate_up = wmoe.quantize_experts(
        E, 2 * I, H, lambda e: synth.weights(2 * I, H, seed, stream=500 + e, device=DEV), DEV,
        asym=asym)
    down = wmoe.quantize_experts(
        E, H, I, lambda e: synth.weights(H, I, seed, stream=600 + e, device=DEV), DEV, asym=asym)
    B = w4.w4_pick_block_size(T, k, E)
    bufs = wmoe.alloc_buffers(T, k, E, H, I, B, DEV)
    X = synth.activations(T, H, seed, device=DEV)
    L = synth.router_logits(T, E, seed, device=DEV)
    g = capture(lambda: wmoe.moe_layer(X, L, k, gate_up, down, B=B, buffers=bufs))
    for r in range(3):
        X.copy_(synth.activations(T, H, 40 + r, device=DEV))
        L.copy_(synth.router_logits(T, E, 40 + r, device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, _, _, _ = wmoe.moe_layer(X, L, k, gate_up, down, B=B)
        np.testing.assert_array_equal(down_bits(bufs.out), down_bits(ref), err_msg=f"replay {r}")


@pytest.mark.parametrize("noalloc", [False, True])
def test_fused_combine_graph_replay(noalloc):
    """The down product with the combine fused, captured once (workspace
    counters, or the library's own with the allocation-free call) and
    replayed with new activations and routing weights copied in between:
    every replay equals the eager down product + combine bit for bit, and
    the counters are back at zero."""
    T, E, k, H, I, seed = 64, 8, 4, 512, 128, 13
    say(f"graph fused combine noalloc={noalloc}")
    down = wmoe.quantize_experts(
        E, H, I, lambda e: synth.weights(H, I, seed, stream=700 + e, device=DEV), DEV)
    ids, tw = w4.w4_moe_route(synth.router_logits(T, E, seed, device=DEV), k)
    B = w4.w4_pick_block_size(T, k, E)
    b = wmoe.alloc_buffers(T, k, E, H, I, B, DEV)
    w4.moe_align_block_size(ids, E, B, b.sorted_token_ids, b.expert_ids, b.ntpp)
    A = b.A
    A.copy_(synth.activations(T * k, I, seed, device=DEV))
    if noalloc:
        fn = lambda: w4.w4a16_moe_gemm_combine_noalloc(A, down.Wq, down.S, b.sorted_token_ids,
                                                       b.expert_ids, b.ntpp, ids, tw, B, b.H2,
                                                       b.out)
    else:
        fn = lambda: wmoe.down_combine(A, down, b.sorted_token_ids, b.expert_ids, b.ntpp, ids,
                                       tw, B, b)
    g = capture(fn)
    for r in range(3):
        A.copy_(synth.activations(T * k, I, 50 + r, device=DEV))
        tw.copy_(torch.rand((T, k), generator=torch.Generator().manual_seed(r)).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        h2 = w4.w4a16_moe_gemm(A, down.Wq, down.S, b.sorted_token_ids, b.expert_ids, b.ntpp,
                               T, k, B, 1)
        ref = w4.w4_moe_sum(h2, tw, T, k)
        np.testing.assert_array_equal(down_bits(b.out), down_bits(ref), err_msg=f"replay {r}")
        assert int(torch.count_nonzero(b.ws).item()) == 0
