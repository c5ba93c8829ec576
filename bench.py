"""Throughput of the INT4 weight-only hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sections ...]
                    [--no-cpu-baseline]

Headline line (one JSON object on stdout): the decode W4A16 product over
packed INT4 weights W[12288 x 4096] (group 32, bf16 scales) against
M in {1, 8, 16, 32} bf16 activation rows, with the codes and the scales in
the kernel-order layouts (w4_repack, w4_repack_groups, converted once
before timing, as an inference engine converts weights at load).  One step = those four products,
each on its own copy of the weights (24 copies rotate, 680 MB in all, so
the 256 MB last-level cache never holds the step's weights).  ``value`` is
the algorithmic HBM traffic of the step (packed codes + scales + X + Y)
over the step time, HIP events on the launch stream around exactly K steps.
Before each timed region the same work runs untimed for SETTLE_MS (after
the W warm-up steps): from idle the GPU takes a few tens of milliseconds
of sustained load to reach its steady clocks.

The other workloads of the path are timed in the same run and reported
under "detail": the prefill product (M = 4096, N = 14336, K = 4096,
TFLOP/s), quantize + pack, fake quant and dequant of that weight (GB/s), and the two
routed MoE layers (128 experts / top-8 / hidden 4096 / intermediate 1536 at
256 tokens; 384 experts / top-8 / hidden 7168 / intermediate 2048 at 4096
tokens with skewed routing), per stage and whole layer, the layer again at
the other alignment block sizes (16 / 32 / 64 and 32 / 64), and the
per-expert row distribution; and under
"asym" the zero-point variants: the decode sweep and the prefill product
with zero-point weights (one uint8 zero point per group on top of the
scale), asymmetric quantize + pack and fake quant, and the two MoE layers
with zero-point experts (whole fused layer and its two grouped products).

The CPU oracle is timed on this host as a reported baseline: whole decode
steps (the same four products over the same weight shape) for the headline
value, and once per other stage of the path on a bounded sample
(quantize + pack, fake quant, a prefill row block, routing and alignment of
the 384-expert layer, the grouped products of 8 experts of the 128-expert
layer), on the cores this process may use (BLAS threads set to match).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def host_cores():
    """CPUs this process may run on, capped by an OMP_NUM_THREADS the
    environment already sets (a container's CPU share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


# the CPU oracle's BLAS uses exactly the cores reported; set before numpy loads
CPU_CORES = host_cores()
for _var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_var] = str(CPU_CORES)

METRIC = "W4A16 GEMM: decode HBM GB/s (% peak) + prefill/MoE TFLOP/s (% MFMA peak)"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

DECODE_N, DECODE_K, DECODE_MS = 12288, 4096, (1, 8, 16, 32)
ROTATE = 24
SETTLE_MS = 150.0     # sustained untimed load before each timed region


def decode_bytes(M, N=DECODE_N, K=DECODE_K, zero_points=False):
    """Algorithmic bytes of one decode product: codes + scales (+ zero
    points) + X + Y."""
    zp = N * (K // 32) if zero_points else 0
    return N * K // 2 + 2 * N * (K // 32) + zp + 2 * M * K + 2 * M * N


def gemm_flops(M, N, K):
    return 2 * M * N * K


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--sections", default="decode,prefill,quant,moe_qwen,moe_kimi,asym")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-block-sweep", action="store_true",
                   help="MoE layers at the picked block size only")
    p.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                   help="untimed sustained load before each timed region (0 under a profiler)")
    return p.parse_args()


class Timer:
    """HIP events on the current (launch) stream around a region."""

    def __init__(self, torch, settle_ms=SETTLE_MS):
        self.torch = torch
        self.settle_scale = settle_ms / SETTLE_MS

    def run(self, fn, iters):
        torch = self.torch
        st = torch.cuda.current_stream()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(st)
        for i in range(iters):
            fn(i)
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b)          # ms for all iterations

    def settle(self, fn, min_ms=SETTLE_MS):
        """Untimed: repeat fn until min_ms of sustained work has run.  From
        idle the GPU needs a few tens of milliseconds of load to reach its
        steady clocks; numbers taken earlier describe the ramp, not the
        kernel."""
        min_ms = min_ms * self.settle_scale
        done, n = 0.0, 1
        while done < min_ms:
            done += self.run(fn, n)
            n = min(2 * n, 1024)


# the sources each measured kernel is built from
KERNEL_SOURCES = {"decode_gemv": ("gemv.hip", "common.h")}


def source_hash(files=None):
    """Hash of kernel sources (all of csrc/ by default), to tell whether
    stored counters still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_weight_only_amd", "csrc")
    for f in sorted(files or os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    ent = d.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash(KERNEL_SOURCES[kernel_key]):
        return None
    return ent.get("hbm_bytes_per_launch")


# ------------------------------------------------------------- sections --

def bench_decode(w4, synth, torch, steps, warmup, timer):
    dev = torch.device("cuda")
    src = synth.weights(DECODE_N, DECODE_K, synth.WORKLOADS["decode"]["seed"], device=dev)
    Wq0, S0 = w4.w4_quantize_pack(src)
    del src
    Wqs = [Wq0] + [Wq0.clone() for _ in range(ROTATE - 1)]
    Ss = [S0] + [S0.clone() for _ in range(ROTATE - 1)]
    # codes and scales in the kernel-order layouts, converted once as at
    # weight load
    Wts = [w4.w4_repack(W) for W in Wqs]
    Sts = [w4.w4_repack_groups(S) for S in Ss]
    Xs = {M: synth.activations(M, DECODE_K, 1, device=dev) for M in DECODE_MS}
    Ys = {M: torch.empty((M, DECODE_N), dtype=torch.bfloat16, device=dev) for M in DECODE_MS}

    def step(i):
        for j, M in enumerate(DECODE_MS):
            r = (4 * i + j) % ROTATE
            w4.w4a16_gemm_tiled(Xs[M], Wts[r], Sts[r], DECODE_N, out=Ys[M])

    timer.run(step, warmup)
    timer.settle(step)
    ms = timer.run(step, steps)
    step_bytes = sum(decode_bytes(M) for M in DECODE_MS)
    per_m = graph_per_m(
        torch, timer, steps, lambda M, r: w4.w4a16_gemm(Xs[M], Wqs[r], Ss[r], out=Ys[M]),
        lambda M: decode_bytes(M))
    per_m_tiled = graph_per_m(
        torch, timer, steps,
        lambda M, r: w4.w4a16_gemm_tiled(Xs[M], Wts[r], Sts[r], DECODE_N, out=Ys[M]),
        lambda M: decode_bytes(M))
    launches = steps * len(DECODE_MS)
    return dict(ms_step=ms / steps, step_bytes=step_bytes, launches=launches, total_ms=ms,
                per_m=per_m, per_m_tiled=per_m_tiled)


def graph_per_m(torch, timer, steps, launch, nbytes):
    """Per-M decode time from a HIP graph of ROTATE back-to-back launches
    (one per weight copy), replayed: the GPU runs the products without the
    host's per-call cost, so a lone small product is timed on the GPU, not
    on the host.  Each launch's time includes the gap between consecutive
    kernels of the graph."""
    per_m = {}
    for M in DECODE_MS:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(ROTATE):
                launch(M, r)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(ROTATE):
                launch(M, r)
        reps = max(4, steps // 6)
        replay = lambda i: g.replay()
        timer.settle(replay, SETTLE_MS / 3)
        t = timer.run(replay, reps) / (reps * ROTATE)
        gbs = nbytes(M) / (t * 1e-3) / 1e9
        per_m[str(M)] = {"us": round(t * 1e3, 3), "GB/s": round(gbs, 1),
                         "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                         "timing": f"HIP graph of {ROTATE} launches x {reps} replays"}
        del g
    return per_m


def graph_time(torch, timer, fn, n, reps=4):
    """Mean time (ms) of one fn() from a HIP graph of n back-to-back calls
    replayed reps times (one warm-up call on the capture stream first)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    timer.run(lambda i: g.replay(), 1)
    t = timer.run(lambda i: g.replay(), reps) / (reps * n)
    del g
    return t


def bench_prefill(w4, synth, torch, iters, timer):
    wl = synth.WORKLOADS["prefill"]
    M, N, K = wl["M"][0], wl["N"], wl["K"]
    dev = torch.device("cuda")
    W = synth.weights(N, K, wl["seed"], device=dev)
    X = synth.activations(M, K, wl["seed"], device=dev)
    Wq, S = w4.w4_quantize_pack(W)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    f = lambda i: w4.w4a16_gemm(X, Wq, S, out=Y)
    timer.settle(f)
    t = timer.run(f, iters) / iters
    tf = gemm_flops(M, N, K) / (t * 1e-3) / 1e12
    Wt, St = w4.w4_repack(Wq), w4.w4_repack_groups(S)
    ft = lambda i: w4.w4a16_gemm_tiled(X, Wt, St, N, out=Y)
    timer.settle(ft, SETTLE_MS / 3)
    tt = timer.run(ft, iters) / iters
    tft = gemm_flops(M, N, K) / (tt * 1e-3) / 1e12
    return {"M": M, "N": N, "K": K, "us": round(t * 1e3, 1), "TFLOP/s": round(tf, 1),
            "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4),
            "kernel_order": {"us": round(tt * 1e3, 1), "TFLOP/s": round(tft, 1),
                             "frac_mfma_bf16": round(tft / PEAK_BF16_TFLOPS, 4)}}


def bench_quant(w4, synth, torch, iters, timer):
    wl = synth.WORKLOADS["prefill"]
    N, K = wl["N"], wl["K"]
    dev = torch.device("cuda")
    W = synth.weights(N, K, wl["seed"], device=dev)
    Wq = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    S = torch.empty((N, K // 32), dtype=torch.bfloat16, device=dev)
    Wf = torch.empty_like(W)
    out = {}
    qp_bytes = 2 * N * K + N * K // 2 + 2 * N * (K // 32)
    fq_bytes = 4 * N * K
    w4.w4_quantize_pack(W, Wq, S)
    Wt = w4.w4_repack(Wq)
    Wr = torch.empty_like(Wq)
    rp_bytes = 2 * (N * K // 2)
    St = w4.w4_repack_groups(S)
    rg_bytes = 2 * (2 * N * (K // 32))
    for name, fn, nbytes in (("quantize_pack", lambda i: w4.w4_quantize_pack(W, Wq, S), qp_bytes),
                             ("fake_quant", lambda i: w4.w4_fake_quant(W, Wf), fq_bytes),
                             ("dequant", lambda i: w4.w4_dequant(Wq, S, Wf), qp_bytes),
                             ("repack", lambda i: w4.w4_repack(Wq, Wt), rp_bytes),
                             ("restore", lambda i: w4.w4_restore(Wt, N, K, Wr), rp_bytes),
                             ("repack_scales", lambda i: w4.w4_repack_groups(S, St), rg_bytes)):
        timer.settle(fn, SETTLE_MS / 3)
        t = timer.run(fn, iters) / iters
        gbs = nbytes / (t * 1e-3) / 1e9
        out[name] = {"N": N, "K": K, "us": round(t * 1e3, 2), "bytes": nbytes,
                     "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    # the QAT linear forward (pack W, then the W4A16 product on the codes)
    from int4_weight_only_amd.qat import qat_linear
    qat = {}
    for M in (16, wl["M"][0]):
        X = synth.activations(M, K, wl["seed"], device=dev)
        fn = lambda i, X=X: qat_linear(X, W)
        timer.settle(fn, SETTLE_MS / 3)
        qat[str(M)] = round(timer.run(fn, iters) / iters * 1e3, 1)
    out["qat_linear_forward_us_by_M"] = qat
    # the QAT linear's input gradient at the prefill rows: W_fq^T from the
    # codes (w4_dequant_t), then dX = dY W_fq (w4_bf16_gemm_nt)
    M = wl["M"][0]
    dY = synth.activations(M, N, wl["seed"] + 1, device=dev)
    WT = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    fn = lambda i: w4.w4_dequant_t(Wq, S, out=WT)
    timer.settle(fn, SETTLE_MS / 3)
    t_dq = timer.run(fn, iters) / iters
    fn = lambda i: w4.w4_bf16_gemm_nt(dY, WT, out=dX)
    timer.settle(fn, SETTLE_MS / 3)
    t_mm = timer.run(fn, iters) / iters
    tf = gemm_flops(M, K, N) / (t_mm * 1e-3) / 1e12
    out["qat_input_gradient"] = {
        "M": M, "N": N, "K": K, "dequant_t_us": round(t_dq * 1e3, 1),
        "dequant_t_GB/s": round(qp_bytes / (t_dq * 1e-3) / 1e9, 1),
        "gemm_nt_us": round(t_mm * 1e3, 1), "gemm_nt_TFLOP/s": round(tf, 1),
        "gemm_nt_frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4)}
    # and its weight gradient dW = dY^T X: both operands transposed (the
    # token dimension contiguous), then the same product
    X = synth.activations(M, K, wl["seed"], device=dev)
    dYT = torch.empty((N, M), dtype=torch.bfloat16, device=dev)
    XT = torch.empty((K, M), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)

    def weight_grad(i):
        w4.w4_bf16_transpose(dY, M, out=dYT)
        w4.w4_bf16_transpose(X, M, out=XT)
        w4.w4_bf16_gemm_nt(dYT, XT, out=dW)
    timer.settle(weight_grad, SETTLE_MS / 3)
    t_wg = timer.run(weight_grad, iters) / iters
    tf = gemm_flops(N, K, M) / (t_wg * 1e-3) / 1e12
    out["qat_weight_gradient"] = {"M": M, "N": N, "K": K, "us": round(t_wg * 1e3, 1),
                                  "TFLOP/s": round(tf, 1),
                                  "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def bench_asym(w4, synth, torch, steps, warmup, iters, timer):
    """Zero-point weights: decode per M (rotating weight copies as in the
    headline sweep), the prefill product, asymmetric quantize + pack and
    fake quant."""
    dev = torch.device("cuda")
    out = {}
    src = synth.weights(DECODE_N, DECODE_K, synth.WORKLOADS["decode"]["seed"], device=dev)
    Wq0, S0, Z0 = w4.w4_quantize_pack_asym(src)
    del src
    ws = [(Wq0, S0, Z0)] + [(Wq0.clone(), S0.clone(), Z0.clone()) for _ in range(ROTATE - 1)]
    Xs = {M: synth.activations(M, DECODE_K, 1, device=dev) for M in DECODE_MS}
    Ys = {M: torch.empty((M, DECODE_N), dtype=torch.bfloat16, device=dev) for M in DECODE_MS}
    out["decode_per_M"] = graph_per_m(
        torch, timer, steps, lambda M, r: w4.w4a16_gemm_asym(Xs[M], *ws[r], out=Ys[M]),
        lambda M: decode_bytes(M, zero_points=True))
    del ws, Wq0, S0, Z0

    wl = synth.WORKLOADS["prefill"]
    M, N, K = wl["M"][0], wl["N"], wl["K"]
    W = synth.weights(N, K, wl["seed"], device=dev)
    X = synth.activations(M, K, wl["seed"], device=dev)
    Wq, S, Z = w4.w4_quantize_pack_asym(W)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    f = lambda i: w4.w4a16_gemm_asym(X, Wq, S, Z, out=Y)
    timer.settle(f)
    t = timer.run(f, iters) / iters
    tf = gemm_flops(M, N, K) / (t * 1e-3) / 1e12
    out["prefill"] = {"M": M, "N": N, "K": K, "us": round(t * 1e3, 1), "TFLOP/s": round(tf, 1),
                      "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4)}

    Wf = torch.empty_like(W)
    qp_bytes = 2 * N * K + N * K // 2 + 3 * N * (K // 32)
    fq_bytes = 4 * N * K
    for name, fn, nbytes in (
            ("quantize_pack_asym", lambda i: w4.w4_quantize_pack_asym(W, Wq, S, Z), qp_bytes),
            ("fake_quant_asym", lambda i: w4.w4_fake_quant_asym(W, Wf), fq_bytes)):
        timer.settle(fn, SETTLE_MS / 3)
        t = timer.run(fn, iters) / iters
        gbs = nbytes / (t * 1e-3) / 1e9
        out[name] = {"N": N, "K": K, "us": round(t * 1e3, 2), "bytes": nbytes,
                     "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    # the QAT linear forward (pack W, then the W4A16 product on the codes)
    from int4_weight_only_amd.qat import qat_linear
    qat = {}
    for M in (16, wl["M"][0]):
        X = synth.activations(M, K, wl["seed"], device=dev)
        fn = lambda i, X=X: qat_linear(X, W)
        timer.settle(fn, SETTLE_MS / 3)
        qat[str(M)] = round(timer.run(fn, iters) / iters * 1e3, 1)
    out["qat_linear_forward_us_by_M"] = qat
    return out


def bench_copy(torch, iters, timer):
    """A plain streaming kernel of known traffic (256 MiB read, 256 MiB
    written; an elementwise bitwise NOT, whose kernel name is unique in the
    trace): the calibration kernel for the HBM byte counters."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    f = lambda i: torch.bitwise_not(a, out=b)
    timer.run(f, 2)
    t = timer.run(f, iters) / iters
    return {"bytes_read": n, "bytes_written": n, "us": round(t * 1e3, 2),
            "GB/s": round(2 * n / (t * 1e-3) / 1e9, 1)}


MOE_B_SWEEP = {"moe_qwen": (16, 32, 64), "moe_kimi": (32, 64)}


def bench_moe_layer(name, w4, wmoe, synth, torch, iters, timer, block_sweep=True):
    wl = synth.WORKLOADS[name]
    T, E, k, H, I, seed = wl["T"], wl["E"], wl["k"], wl["H"], wl["I"], wl["seed"]
    dev = torch.device("cuda")
    gate_up = wmoe.quantize_experts(E, 2 * I, H,
                                    lambda e: synth.expert_gate_up(e, I, H, seed, dev), dev)
    down = wmoe.quantize_experts(E, H, I, lambda e: synth.expert_down(e, I, H, seed, dev), dev)
    X = synth.activations(T, H, seed, device=dev)
    logits = synth.router_logits(T, E, seed, wl["skew"], device=dev)
    B = w4.w4_pick_block_size(T, k, E)
    ids, tw = w4.w4_moe_route(logits, k)
    buf = wmoe.alloc_buffers(T, k, E, H, I, B, dev, fused=False)
    tw_flat = tw.reshape(-1)

    stages = {
        "route": lambda: w4.w4_moe_route(logits, k, ids, tw),
        "align": lambda: w4.moe_align_block_size(ids, E, B, buf.sorted_token_ids,
                                                 buf.expert_ids, buf.ntpp),
        "gate_up": lambda: w4.w4a16_moe_gemm(X, gate_up.Wq, gate_up.S, buf.sorted_token_ids,
                                             buf.expert_ids, buf.ntpp, T, k, B, k, out=buf.H1),
        "silu_mul": lambda: w4.w4_silu_mul(buf.H1, out=buf.A),
        "gate_up_swiglu": lambda: w4.w4a16_moe_gemm_swiglu(X, gate_up.Wq, gate_up.S,
                                                           buf.sorted_token_ids, buf.expert_ids,
                                                           buf.ntpp, T, k, B, k, out=buf.A),
        "down": lambda: w4.w4a16_moe_gemm(buf.A, down.Wq, down.S, buf.sorted_token_ids,
                                          buf.expert_ids, buf.ntpp, T, k, B, 1, out=buf.H2),
        "combine": lambda: w4.w4_moe_sum(buf.H2, tw, T, k, out=buf.out),
    }

    # the layer runs the fused gate_up + SwiGLU; the unfused pair is timed
    # per stage for reference
    layer_stages = ("route", "align", "gate_up_swiglu", "down", "combine")

    def layer(i):
        for sname in layer_stages:
            stages[sname]()

    timer.settle(layer)
    t_layer = timer.run(layer, iters) / iters
    # the same layer on kernel-order experts
    gu_t, dn_t = wmoe.repack_experts(gate_up), wmoe.repack_experts(down)
    stages["gate_up_swiglu_kernel_order"] = lambda: wmoe.grouped_gemm_swiglu(
        X, gu_t, buf.sorted_token_ids, buf.expert_ids, buf.ntpp, T, k, B, k, out=buf.A)
    stages["down_kernel_order"] = lambda: wmoe.grouped_gemm(
        buf.A, dn_t, buf.sorted_token_ids, buf.expert_ids, buf.ntpp, T, k, B, 1, out=buf.H2)
    # the down product with the top-k combine fused (w4a16_moe_gemm_combine),
    # against down_kernel_order + combine
    stages["down_combine_kernel_order"] = lambda: wmoe.down_combine(
        buf.A, dn_t, buf.sorted_token_ids, buf.expert_ids, buf.ntpp, ids, tw, B, buf)

    def layer_t(i):
        for sname in ("route", "align", "gate_up_swiglu_kernel_order", "down_kernel_order",
                      "combine"):
            stages[sname]()

    timer.settle(layer_t, SETTLE_MS / 3)
    t_layer_t = timer.run(layer_t, iters) / iters
    # per stage: a HIP graph of back-to-back launches, replayed (the small
    # kernels would otherwise be timed on the host's launch cost)
    per = {}
    for sname, fn in stages.items():
        per[sname] = round(graph_time(torch, timer, fn, iters) * 1e3, 2)
    pairs = T * k
    fl_gu = gemm_flops(pairs, 2 * I, H)
    fl_dn = gemm_flops(pairs, H, I)
    wbytes = gate_up.nbytes() + down.nbytes()
    counts = torch.bincount(ids.reshape(-1).long(), minlength=E)
    ntpp = int(buf.ntpp.item())
    # the whole (fused) layer at other alignment block sizes
    by_B = {str(B): round(t_layer * 1e3, 1)}
    for B2 in (MOE_B_SWEEP.get(name, ()) if block_sweep else ()):
        if B2 == B:
            continue
        b2 = wmoe.alloc_buffers(T, k, E, H, I, B2, dev, fused=True)

        def layer_b(i, b2=b2, B2=B2):
            w4.w4_moe_route(logits, k, ids, tw)
            w4.moe_align_block_size(ids, E, B2, b2.sorted_token_ids, b2.expert_ids, b2.ntpp)
            w4.w4a16_moe_gemm_swiglu(X, gate_up.Wq, gate_up.S, b2.sorted_token_ids,
                                     b2.expert_ids, b2.ntpp, T, k, B2, k, out=b2.A)
            w4.w4a16_moe_gemm(b2.A, down.Wq, down.S, b2.sorted_token_ids, b2.expert_ids,
                              b2.ntpp, T, k, B2, 1, out=b2.H2)
            w4.w4_moe_sum(b2.H2, tw, T, k, out=b2.out)
        timer.settle(layer_b, SETTLE_MS / 3)
        by_B[str(B2)] = round(timer.run(layer_b, iters) / iters * 1e3, 1)
        del b2
    q = torch.quantile(counts.float(), torch.tensor([0.1, 0.5, 0.9], device=counts.device))

    def gemm_rates(us):
        """The two grouped products (fused gate_up + SwiGLU, down) taking us
        microseconds together: weight stream and MFMA rates."""
        return {"us": round(us, 1),
                "weight_GB/s": round(wbytes / (us * 1e-6) / 1e9, 1),
                "frac_hbm": round(wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                "TFLOP/s": round((fl_gu + fl_dn) / (us * 1e-6) / 1e12, 1),
                "frac_mfma_bf16": round((fl_gu + fl_dn) / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}

    res = {
        "T": T, "E": E, "k": k, "H": H, "I": I, "B": B,
        "layer_us": round(t_layer * 1e3, 1),
        "layer_us_kernel_order": round(t_layer_t * 1e3, 1),
        "layer_TFLOP/s_kernel_order": round((fl_gu + fl_dn) / (t_layer_t * 1e-3) / 1e12, 1),
        "stage_us": per,
        "layer_TFLOP/s": round((fl_gu + fl_dn) / (t_layer * 1e-3) / 1e12, 1),
        "gate_up_TFLOP/s": round(fl_gu / (per["gate_up"] * 1e-6) / 1e12, 1),
        "down_TFLOP/s": round(fl_dn / (per["down"] * 1e-6) / 1e12, 1),
        "weight_bytes": wbytes,
        "gemm_weight_GB/s": round(wbytes / ((per["gate_up"] + per["down"]) * 1e-6) / 1e9, 1),
        "frac_mfma_bf16_gemms": round((fl_gu + fl_dn) / ((per["gate_up"] + per["down"]) * 1e-6)
                                      / 1e12 / PEAK_BF16_TFLOPS, 4),
        "frac_hbm_gemms": round(wbytes / ((per["gate_up"] + per["down"]) * 1e-6) / 1e9
                                / PEAK_HBM_GBS, 4),
        "gemms_kernel_order": gemm_rates(per["gate_up_swiglu_kernel_order"]
                                         + per["down_kernel_order"]),
        "layer_us_by_B": by_B,
        "rows_per_expert_max": int(counts.max().item()),
        "rows_per_expert_min": int(counts.min().item()),
        "rows_per_expert_p10_p50_p90": [round(float(v), 1) for v in q.tolist()],
        "padding_frac": round(1.0 - pairs / ntpp, 4),
    }
    del gate_up, down, buf, gu_t, dn_t
    torch.cuda.empty_cache()
    return res


def bench_moe_layer_asym(name, w4, wmoe, synth, torch, iters, timer):
    """The routed layer with zero-point experts: the fused layer and its
    two grouped products at the picked block size."""
    wl = synth.WORKLOADS[name]
    T, E, k, H, I, seed = wl["T"], wl["E"], wl["k"], wl["H"], wl["I"], wl["seed"]
    dev = torch.device("cuda")
    gate_up = wmoe.quantize_experts(E, 2 * I, H,
                                    lambda e: synth.expert_gate_up(e, I, H, seed, dev), dev,
                                    asym=True)
    down = wmoe.quantize_experts(E, H, I, lambda e: synth.expert_down(e, I, H, seed, dev), dev,
                                 asym=True)
    X = synth.activations(T, H, seed, device=dev)
    logits = synth.router_logits(T, E, seed, wl["skew"], device=dev)
    B = w4.w4_pick_block_size(T, k, E)
    ids, tw = w4.w4_moe_route(logits, k)
    buf = wmoe.alloc_buffers(T, k, E, H, I, B, dev, fused=True)
    w4.moe_align_block_size(ids, E, B, buf.sorted_token_ids, buf.expert_ids, buf.ntpp)
    gu = lambda i: wmoe.grouped_gemm_swiglu(X, gate_up, buf.sorted_token_ids, buf.expert_ids,
                                            buf.ntpp, T, k, B, k, out=buf.A)
    dn = lambda i: wmoe.grouped_gemm(buf.A, down, buf.sorted_token_ids, buf.expert_ids,
                                     buf.ntpp, T, k, B, 1, out=buf.H2)

    def layer(i):   # route, align, gate_up + SwiGLU, down, combine
        w4.w4_moe_route(logits, k, ids, tw)
        wmoe.moe_forward(X, ids, tw, gate_up, down, B=B, buffers=buf)
    timer.settle(layer)
    t_layer = timer.run(layer, iters) / iters
    t_gu = timer.run(gu, iters) / iters
    t_dn = timer.run(dn, iters) / iters
    fl = gemm_flops(T * k, 2 * I, H) + gemm_flops(T * k, H, I)
    res = {"T": T, "E": E, "k": k, "H": H, "I": I, "B": B,
           "layer_us": round(t_layer * 1e3, 1),
           "gate_up_swiglu_us": round(t_gu * 1e3, 1), "down_us": round(t_dn * 1e3, 1),
           "layer_TFLOP/s": round(fl / (t_layer * 1e-3) / 1e12, 1),
           "weight_bytes": gate_up.nbytes() + down.nbytes()}
    del gate_up, down, buf
    torch.cuda.empty_cache()
    return res


def blas_vendor():
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        return ", ".join(f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} "
                         f"threads)" for d in info) or "unknown"
    except Exception as exc:      # threadpoolctl missing: say so, do not guess
        return f"unknown ({type(exc).__name__})"


def cpu_baseline():
    """The oracle, as it stands, timed stage by stage on this host's cores.

    The headline value is whole decode steps (the four products M = 1, 8,
    16, 32 over W[12288 x 4096]) until at least 6 s have passed; each other
    stage of the path runs once on a bounded sample of its workload, in the
    same algorithmic units as the GPU numbers.  About 20 s in all."""
    import numpy as np
    import synth
    from oracle import gemm, moe, quant

    stages = {}

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    seed = synth.WORKLOADS["decode"]["seed"]
    Wb = synth.bits(synth.weights(DECODE_N, DECODE_K, seed))
    (Wq, S), dt = timed(lambda: quant.quantize_pack(Wb))
    nb = 2 * DECODE_N * DECODE_K + DECODE_N * DECODE_K // 2 + 2 * DECODE_N * (DECODE_K // 32)
    stages["quantize_pack"] = {"s": round(dt, 3), "GB/s": round(nb / dt / 1e9, 4),
                               "sample": f"W[{DECODE_N}x{DECODE_K}]"}
    _, dt = timed(lambda: quant.fake_quant(Wb))
    nb = 4 * DECODE_N * DECODE_K
    stages["fake_quant"] = {"s": round(dt, 3), "GB/s": round(nb / dt / 1e9, 4),
                            "sample": f"W[{DECODE_N}x{DECODE_K}]"}

    Xs = {M: synth.bits(synth.activations(M, DECODE_K, 1)) for M in DECODE_MS}
    t0 = time.perf_counter()
    reps = 0
    while True:
        for M in DECODE_MS:
            gemm.w4a16_gemm(Xs[M], Wq, S)
        reps += 1
        if time.perf_counter() - t0 > 6:
            break
    dt_dec = time.perf_counter() - t0
    dec_bytes = reps * sum(decode_bytes(M) for M in DECODE_MS)
    stages["decode_gemm"] = {"s": round(dt_dec, 3), "GB/s": round(dec_bytes / dt_dec / 1e9, 4),
                             "sample": f"{reps} decode step(s)"}

    wl = synth.WORKLOADS["prefill"]
    Mp = 256
    Wp = synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"]))
    Wqp, Sp = quant.quantize_pack(Wp)
    Xp = synth.bits(synth.activations(Mp, wl["K"], wl["seed"]))
    _, dt = timed(lambda: gemm.w4a16_gemm(Xp, Wqp, Sp))
    stages["prefill_gemm"] = {"s": round(dt, 3),
                              "GFLOP/s": round(gemm_flops(Mp, wl["N"], wl["K"]) / dt / 1e9, 3),
                              "sample": f"{Mp} of {wl['M'][0]} rows x W[{wl['N']}x{wl['K']}] "
                                        "(dequant + fp64 matmul)"}

    c4 = synth.WORKLOADS["moe_kimi"]
    lg = synth.router_logits(c4["T"], c4["E"], c4["seed"], c4["skew"]).numpy()
    (ids, tw), dt = timed(lambda: moe.route(lg, c4["k"]))
    stages["route"] = {"s": round(dt, 3), "tokens/s": round(c4["T"] / dt, 1),
                       "sample": f"T={c4['T']} E={c4['E']} k={c4['k']}"}
    B4 = moe.pick_block_size(c4["T"], c4["k"], c4["E"])
    _, dt = timed(lambda: moe.align(ids, c4["E"], B4))
    stages["align"] = {"s": round(dt, 3), "pairs/s": round(c4["T"] * c4["k"] / dt, 1),
                       "sample": f"{c4['T'] * c4['k']} pairs, E={c4['E']}, B={B4}"}

    c3 = synth.WORKLOADS["moe_qwen"]
    T3, E3, k3, H3, I3 = c3["T"], c3["E"], c3["k"], c3["H"], c3["I"]
    ids3, _ = moe.route(synth.router_logits(T3, E3, c3["seed"]).numpy(), k3)
    B3 = moe.pick_block_size(T3, k3, E3)
    s3, e3, n3 = moe.align(ids3, E3, B3)
    ex = list(range(8))
    gu = {e: quant.quantize_pack(synth.bits(synth.expert_gate_up(e, I3, H3, c3["seed"])))
          for e in ex}
    dn = {e: quant.quantize_pack(synth.bits(synth.expert_down(e, I3, H3, c3["seed"])))
          for e in ex}
    X3 = synth.bits(synth.activations(T3, H3, c3["seed"]))
    A3 = synth.bits(synth.activations(T3 * k3, I3, c3["seed"], stream=77))
    rows, dt = timed(lambda: (
        moe.grouped_gemm(X3, lambda e: gu[e], s3, e3, n3, B3, k3, T3 * k3, experts=set(ex)),
        moe.grouped_gemm(A3, lambda e: dn[e], s3, e3, n3, B3, 1, T3 * k3, experts=set(ex))))
    nrows = len(rows[0])
    fl = gemm_flops(nrows, 2 * I3, H3) + gemm_flops(nrows, H3, I3)
    stages["grouped_gemms"] = {"s": round(dt, 3), "GFLOP/s": round(fl / dt / 1e9, 3),
                               "sample": f"gate_up + down of {len(ex)} of {E3} experts "
                                         f"({nrows} rows), 128-expert layer"}

    return {"value": round(dec_bytes / dt_dec / 1e9, 4), "unit": "GB/s", "cores": CPU_CORES,
            "kind": "oracle",
            "sample": f"{reps} full decode step(s): M in {{1,8,16,32}} x W[12288x4096] "
                      f"int4 g32, numpy dequant + fp64 matmul, {dt_dec:.1f} s",
            "affinity_cpus": len(os.sched_getaffinity(0)), "blas": blas_vendor(),
            "stages": stages}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(no collectives, no sharding); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import int4_weight_only_amd as w4
    from int4_weight_only_amd import moe as wmoe
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    timer = Timer(torch, args.settle_ms)
    sections = [s for s in args.sections.split(",") if s]
    detail = {}

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    dec = None
    if "decode" in sections:
        log("bench: decode sweep")
        dec = bench_decode(w4, synth, torch, args.steps, args.warmup, timer)
        detail["decode_per_M"] = dec["per_m_tiled"]
        detail["decode_per_M_canonical_layout"] = dec["per_m"]
    iters = max(3, min(args.steps, 20))
    if "prefill" in sections:
        log("bench: prefill")
        detail["prefill"] = bench_prefill(w4, synth, torch, iters, timer)
    if "quant" in sections:
        log("bench: quantize_pack / fake_quant")
        detail.update(bench_quant(w4, synth, torch, iters, timer))
    if "copy" in sections:
        log("bench: copy calibration")
        detail["copy"] = bench_copy(torch, iters, timer)
    for name in ("moe_qwen", "moe_kimi"):
        if name in sections:
            log(f"bench: {name}")
            detail[name] = bench_moe_layer(name, w4, wmoe, synth, torch, iters, timer,
                                           block_sweep=not args.no_block_sweep)

    if "asym" in sections:
        log("bench: zero-point variants")
        detail["asym"] = bench_asym(w4, synth, torch, args.steps, args.warmup, iters, timer)
        for name in ("moe_qwen", "moe_kimi"):
            if name in sections:
                log(f"bench: {name} with zero-point experts")
                detail["asym"][name] = bench_moe_layer_asym(name, w4, wmoe, synth, torch, iters,
                                                            timer)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu oracle baseline")
        cpu = cpu_baseline()

    line = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "settle_ms": args.settle_ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "decode W4A16 GEMV sweep: packed int4 W[12288x4096] group 32 "
                                   "bf16 scales, X[M,4096] bf16, M in {1,8,16,32}",
                       "rotating_weight_copies": ROTATE,
                       "code_layout": "kernel order (w4_repack and w4_repack_groups, "
                                      "converted once at load)"}}
    if dec is not None:
        value = dec["step_bytes"] / (dec["ms_step"] * 1e-3) / 1e9
        per_launch_bytes = dec["step_bytes"] / len(DECODE_MS)
        per_launch_us = dec["total_ms"] * 1e3 / dec["launches"]
        achieved = per_launch_bytes / (per_launch_us * 1e-6) / 1e9
        traffic = stored_traffic("decode_gemv")
        line.update(value=round(value, 1), ms_per_step=round(dec["ms_step"], 5))
        line["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1),
                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(achieved / PEAK_HBM_GBS, 4),
                            "traffic": traffic,
                            "kernel": "k_decode16 / k_decode32 on kernel-order codes and scales",
                            "algorithmic_bytes_per_launch": per_launch_bytes,
                            "avg_launch_us": round(per_launch_us, 3)}
    else:
        line.update(value=None, ms_per_step=None)
    line["cpu_baseline"] = cpu
    line["detail"] = detail
    line["source_hash"] = source_hash()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
