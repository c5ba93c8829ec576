"""The allocation-free entry point ``w4a16_moe_gemm_combine_noalloc`` (its
arrival counters in the library's own device array) against
``w4a16_moe_gemm_combine`` (counters in a caller workspace), called through
the C ABI: H2 and the combined output identical bit for bit, on two calls in
a row on one GPU, the second with a smaller input (fewer tokens, experts,
picks and columns), on the 128-row and the 32-row tile."""

import ctypes

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
from int4_weight_only_amd import _lib
from int4_weight_only_amd import moe as wmoe
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def case(T, E, k, N, K, seed):
    down = wmoe.quantize_experts(
        E, N, K, lambda e: synth.weights(N, K, seed, stream=1300 + e, device=DEV), DEV)
    A = synth.activations(T * k, K, seed, device=DEV)
    ids, tw = w4.w4_moe_route(synth.router_logits(T, E, seed, device=DEV), k)
    B = w4.w4_pick_block_size(T, k, E)
    s, e, n = w4.moe_align_block_size(ids, E, B)
    return down, A, ids, tw, B, s, e, n


def test_noalloc_matches_workspace_call():
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 128-row tile (many rows per expert), then a smaller 32-row-tile call
    for T, E, k, N, K, seed in ((600, 8, 4, 1024, 256, 41), (96, 6, 2, 384, 128, 42)):
        say(f"noalloc combine T={T} E={E} k={k} N={N} K={K}")
        down, A, ids, tw, B, s, e, n = case(T, E, k, N, K, seed)
        words = w4.w4_moe_combine_workspace_words(T, k, E, N, B)
        ws = torch.zeros(words, dtype=torch.int32, device=DEV)
        bf = dict(dtype=torch.bfloat16, device=DEV)
        H2r, Or = torch.empty((T * k, N), **bf), torch.empty((T, N), **bf)
        H2g, Og = torch.empty((T * k, N), **bf), torch.empty((T, N), **bf)
        head = (p(A), p(down.Wq), p(down.S), p(s), p(e), p(n), p(ids), p(tw))
        assert lib.w4a16_moe_gemm_combine(*head, p(H2r), p(Or), T, k, E, N, K, B, 0, p(ws),
                                          stream) == 0
        assert lib.w4a16_moe_gemm_combine_noalloc(*head, p(H2g), p(Og), T, k, E, N, K, B, 0,
                                                  stream) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(H2g.view(torch.int16).cpu().numpy(),
                                      H2r.view(torch.int16).cpu().numpy())
        np.testing.assert_array_equal(Og.view(torch.int16).cpu().numpy(),
                                      Or.view(torch.int16).cpu().numpy())
        assert int(torch.count_nonzero(ws).item()) == 0
        assert int(torch.count_nonzero(Og.view(torch.int16)).item()) > 0
