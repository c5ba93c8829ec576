"""GPU parity: the grouped down product with the top-k combine fused
(``w4a16_moe_gemm_combine``).

* Against the unfused pair (``w4a16_moe_gemm`` then ``w4_moe_sum``, whose
  own parity with the oracle is tested elsewhere): H2 and the combined
  output bit for bit, on the 32-row and 128-row tiles, canonical and
  kernel-order experts, ragged widths, and on the full 128- and 384-expert
  layers; the arrival counters are all zero again after every call,
  including calls in a row that reuse one workspace.
* Against the oracle: the whole layer with the fused combine on a small
  case, within the GEMM tolerance.
* Pairs whose expert lies outside [0, E) take no part: the output equals the
  fp32 sum over the remaining pairs, in order, of weight * bf16 row.
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
from int4_weight_only_amd import moe as wmoe
import synth
from gpu_util import down_bits, say
from oracle import gemm, quant
from oracle import moe as omoe

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def experts(E, N, K, seed, stream0, tiled):
    w = wmoe.quantize_experts(
        E, N, K, lambda e: synth.weights(N, K, seed, stream=stream0 + e, device=DEV), DEV)
    return wmoe.repack_experts(w) if tiled else w


def layer_inputs(T, E, k, H, I, seed, skew=None):
    X = synth.activations(T, H, seed, device=DEV)
    logits = synth.router_logits(T, E, seed, skew, device=DEV)
    ids, tw = w4.w4_moe_route(logits, k)
    return X, ids, tw


def run_both(X, ids, tw, gate_up, down, B):
    """(unfused buffers, fused buffers) of the same layer."""
    ref, bref = wmoe.moe_forward(X, ids, tw, gate_up, down, B=B)
    out, bf = wmoe.moe_forward(X, ids, tw, gate_up, down, B=B, fused_combine=True)
    torch.cuda.synchronize()
    return bref, bf


def assert_same(bref, bf, label):
    np.testing.assert_array_equal(down_bits(bf.H2), down_bits(bref.H2), err_msg=f"{label}: H2")
    np.testing.assert_array_equal(down_bits(bf.out), down_bits(bref.out), err_msg=f"{label}: out")
    assert int(torch.count_nonzero(bf.ws).item()) == 0, f"{label}: counters not back at zero"


SMALL = [
    # T, E, k, H, I, B, tiled: 32-row tile (few rows per expert) and 128-row tile
    (24, 8, 2, 128, 64, 16, False),
    (64, 16, 4, 512, 256, 16, True),
    (33, 4, 3, 224, 96, 16, False),        # ragged width: 224 columns, two 128-wide tiles
    (300, 4, 2, 384, 128, 64, False),      # 128-row tile, several runs per expert
    (300, 4, 2, 384, 128, 64, True),
    (257, 8, 8, 544, 64, 32, True),        # every token on every expert, ragged width
]


@pytest.mark.parametrize("T,E,k,H,I,B,tiled", SMALL)
def test_fused_combine_matches_unfused(T, E, k, H, I, B, tiled):
    say(f"fused combine T={T} E={E} k={k} H={H} I={I} B={B} tiled={tiled}")
    gate_up = experts(E, 2 * I, H, 7, 700, tiled)
    down = experts(E, H, I, 7, 800, tiled)
    X, ids, tw = layer_inputs(T, E, k, H, I, 9)
    bref, bf = run_both(X, ids, tw, gate_up, down, B)
    assert_same(bref, bf, f"T={T}")


def test_fused_combine_calls_in_a_row():
    """One set of buffers (one workspace), three layers back to back on one
    stream without synchronizing: each fused output equals its unfused one."""
    T, E, k, H, I, B = 96, 8, 4, 256, 128, 16
    gate_up = experts(E, 2 * I, H, 3, 900, False)
    down = experts(E, H, I, 3, 1000, False)
    bufs = wmoe.alloc_buffers(T, k, E, H, I, B, DEV)
    outs, refs = [], []
    for r in range(3):
        say(f"fused combine in a row {r}")
        X, ids, tw = layer_inputs(T, E, k, H, I, 20 + r)
        out, _ = wmoe.moe_forward(X, ids, tw, gate_up, down, B=B, buffers=bufs,
                                  fused_combine=True)
        outs.append(out.clone())
        ref, _ = wmoe.moe_forward(X, ids, tw, gate_up, down, B=B)
        refs.append(ref.clone())
    for r in range(3):
        np.testing.assert_array_equal(down_bits(outs[r]), down_bits(refs[r]), err_msg=f"call {r}")
    assert int(torch.count_nonzero(bufs.ws).item()) == 0


def test_fused_combine_layer_vs_oracle():
    T, E, k, H, I, B = 40, 8, 2, 128, 64, 16
    say("fused combine layer vs oracle")
    gu_src = [synth.weights(2 * I, H, 5, stream=300 + e) for e in range(E)]
    dn_src = [synth.weights(H, I, 5, stream=400 + e) for e in range(E)]
    gate_up = wmoe.quantize_experts(E, 2 * I, H, lambda e: gu_src[e].to(DEV), DEV)
    down = wmoe.quantize_experts(E, H, I, lambda e: dn_src[e].to(DEV), DEV)
    lg = synth.router_logits(T, E, 5)
    Xm = synth.activations(T, H, 6)
    ids_ref, tw_ref = omoe.route(lg.numpy(), k)
    ids = torch.from_numpy(ids_ref).to(DEV)
    tw = torch.from_numpy(tw_ref).to(DEV)
    out, _ = wmoe.moe_forward(Xm.to(DEV), ids, tw, gate_up, down, B=B, fused_combine=True)
    gu_ref = [quant.quantize_pack(synth.bits(s)) for s in gu_src]
    dn_ref = [quant.quantize_pack(synth.bits(s)) for s in dn_src]
    ref = omoe.moe_layer(synth.bits(Xm), ids_ref, tw_ref, lambda e: gu_ref[e], lambda e: dn_ref[e])
    ok, max_abs, max_rel = gemm.within_tolerance(down_bits(out), np.stack([ref[t] for t in range(T)]))
    assert ok, f"max abs {max_abs:.3e} max rel {max_rel:.3e}"


def test_fused_combine_skips_pairs_outside_the_experts():
    T, E, k, H, I, B = 48, 8, 3, 256, 64, 16
    say("fused combine with ids outside [0, E)")
    gate_up = experts(E, 2 * I, H, 4, 1100, False)
    down = experts(E, H, I, 4, 1200, False)
    X, ids, tw = layer_inputs(T, E, k, H, I, 31)
    ids = ids.clone()
    ids[1, 2] = -1
    ids[5, 0] = E + 3
    ids[7, 1] = -5
    out, b = wmoe.moe_forward(X, ids, tw, gate_up, down, B=B, fused_combine=True)
    torch.cuda.synchronize()
    h2 = synth.bits(b.H2).astype(np.uint32) << 16
    h2 = h2.view(np.float32).reshape(T, k, H)
    idn, wn = ids.cpu().numpy(), tw.cpu().numpy()
    ref = np.zeros((T, H), np.float32)
    for t in range(T):
        s = np.zeros(H, np.float32)
        for j in range(k):
            if 0 <= idn[t, j] < E:
                s = (np.float64(wn[t, j]) * h2[t, j].astype(np.float64) + s).astype(np.float32)
        ref[t] = s
    got = down_bits(out).astype(np.uint32) << 16
    np.testing.assert_allclose(got.view(np.float32), ref, rtol=2 ** -8, atol=0)
    assert int(torch.count_nonzero(b.ws).item()) == 0


@pytest.mark.parametrize("name", ["moe_qwen", "moe_kimi"])
def test_fused_combine_full_layers(name):
    """The full 128-expert (32-row tile) and 384-expert (128-row tile,
    skewed routing) layers on kernel-order experts: bit for bit."""
    wl = synth.WORKLOADS[name]
    T, E, k, H, I, seed = wl["T"], wl["E"], wl["k"], wl["H"], wl["I"], wl["seed"]
    say(f"fused combine full layer {name}")
    gate_up = wmoe.repack_experts(wmoe.quantize_experts(
        E, 2 * I, H, lambda e: synth.expert_gate_up(e, I, H, seed, DEV), DEV))
    down = wmoe.repack_experts(wmoe.quantize_experts(
        E, H, I, lambda e: synth.expert_down(e, I, H, seed, DEV), DEV))
    X, ids, tw = layer_inputs(T, E, k, H, I, seed, wl["skew"])
    B = w4.w4_pick_block_size(T, k, E)
    bref, bf = run_both(X, ids, tw, gate_up, down, B)
    assert_same(bref, bf, name)
    del gate_up, down, bref, bf
    torch.cuda.empty_cache()
