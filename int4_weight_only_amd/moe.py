"""A top-k routed MoE layer with W4A16 experts, composed from the C ABI.

Every step is one library call; this module only allocates buffers with
PyTorch and passes them along ("INT4 QAT end-to-end for RL", §4: routing,
moe_align_block_size, the fused expert GEMMs):

    logits --w4_moe_route--> ids, weights
    ids --moe_align_block_size--> sorted_token_ids, expert_ids, ntpp
    X --w4a16_moe_gemm_swiglu (gate_up + SwiGLU, x_row_div = k)--> A [T*k, I]
      (unfused: w4a16_moe_gemm --> H1 [T*k, 2I], then w4_silu_mul --> A)
    A --w4a16_moe_gemm (down, x_row_div = 1)--> H2 [T*k, H]
    H2, weights --w4_moe_sum--> Out [T, H]

The activation (silu(gate) * up, gate = the first I rows of gate_up) and
the combine (weights applied after the down projection) are readings: the
pages name the gate_up / down pair but give no formula.  Experts quantized
with zero points ("Quantization basics: from FP32 to INT4" §2.3) run the
``_asym`` forms of the two grouped products; experts converted to the
kernel-order layouts (``repack_experts``, §4's weight-layout conversion,
codes and per-group values alike) run the ``_tiled`` forms.
"""

from dataclasses import dataclass

import torch

from . import (moe_align_block_size, w4_moe_align_capacity, w4_moe_combine_workspace_words,
               w4_moe_route, w4_moe_sum, w4a16_moe_gemm_combine,
               w4_pick_block_size, w4_quantize_pack, w4_quantize_pack_asym, w4_repack,
               w4_repack_groups, w4_silu_mul, w4a16_moe_gemm, w4a16_moe_gemm_asym, w4a16_moe_gemm_swiglu,
               w4a16_moe_gemm_swiglu_asym, w4a16_moe_gemm_swiglu_tiled, w4a16_moe_gemm_tiled)


@dataclass
class ExpertWeights:
    """Stacked packed weights of E experts: Wq int32 [E, N, K/8], S bf16 [E, N, K/32],
    and for zero-point experts Z uint8 [E, N, K/32] (None: symmetric codes).
    Wt, St, Zt: the same codes, scales and zero points in the kernel-order
    layouts ([E, w4_repacked_words(N, K)], [E, w4_repacked_group_elems(N, K)],
    from ``repack_experts``); when Wt is present the products read Wt, St and
    Zt, and the canonical arrays may be None.  dims = (E, N, K), taken from S
    when not given."""
    Wq: torch.Tensor
    S: torch.Tensor
    Z: torch.Tensor = None
    Wt: torch.Tensor = None
    St: torch.Tensor = None
    Zt: torch.Tensor = None
    dims: tuple = None

    def __post_init__(self):
        if self.dims is None:
            E, N, G = self.S.shape
            self.dims = (E, N, 32 * G)

    @property
    def E(self):
        return self.dims[0]

    @property
    def N(self):
        return self.dims[1]

    @property
    def K(self):
        return self.dims[2]

    def nbytes(self):
        """Bytes of the arrays the products read."""
        if self.Wt is not None:
            arrays = (self.Wt, self.St, self.Zt)
        else:
            arrays = (self.Wq, self.S, self.Z)
        return sum(a.numel() * a.element_size() for a in arrays if a is not None)


def repack_experts(w, keep_canonical=False):
    """The experts with codes, scales and zero points converted to the
    kernel-order layouts (``w4_repack``, ``w4_repack_groups``); the canonical
    arrays are dropped unless asked for (``w4_restore`` and
    ``w4_restore_groups`` bring them back)."""
    Wt = w4_repack(w.Wq)
    St = w4_repack_groups(w.S)
    Zt = w4_repack_groups(w.Z) if w.Z is not None else None
    if keep_canonical:
        return ExpertWeights(w.Wq, w.S, w.Z, Wt, St, Zt, w.dims)
    return ExpertWeights(None, None, None, Wt, St, Zt, w.dims)


def quantize_experts(E, N, K, source, device, asym=False):
    """Quantize E expert matrices one at a time into stacked buffers.

    ``source(e)`` returns expert e's bf16 [N, K] weight on ``device``; only
    one source matrix is alive at a time.  ``asym``: zero-point codes
    (``w4_quantize_pack_asym``).
    """
    Wq = torch.empty((E, N, K // 8), dtype=torch.int32, device=device)
    S = torch.empty((E, N, K // 32), dtype=torch.bfloat16, device=device)
    Z = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device) if asym else None
    for e in range(E):
        w = source(e)
        if asym:
            w4_quantize_pack_asym(w, Wq[e], S[e], Z[e])
        else:
            w4_quantize_pack(w, Wq[e], S[e])
        del w
    return ExpertWeights(Wq, S, Z)


def grouped_gemm(X, w, sorted_token_ids, expert_ids, ntpp, T, k, B, x_row_div,
                 topk_weights=None, out=None):
    """``w4a16_moe_gemm``, its zero-point form or their kernel-order forms,
    as the experts ``w`` need."""
    if w.Wt is not None:
        return w4a16_moe_gemm_tiled(X, w.Wt, w.St, w.N, sorted_token_ids, expert_ids, ntpp, T, k,
                                    B, x_row_div, Z=w.Zt, topk_weights=topk_weights, out=out)
    if w.Z is None:
        return w4a16_moe_gemm(X, w.Wq, w.S, sorted_token_ids, expert_ids, ntpp, T, k, B,
                              x_row_div, topk_weights, out)
    return w4a16_moe_gemm_asym(X, w.Wq, w.S, w.Z, sorted_token_ids, expert_ids, ntpp, T, k, B,
                               x_row_div, topk_weights, out)


def grouped_gemm_swiglu(X, w, sorted_token_ids, expert_ids, ntpp, T, k, B, x_row_div, out=None):
    """``w4a16_moe_gemm_swiglu``, its zero-point form or their kernel-order
    forms, as the experts ``w`` need."""
    if w.Wt is not None:
        return w4a16_moe_gemm_swiglu_tiled(X, w.Wt, w.St, w.N, sorted_token_ids, expert_ids, ntpp,
                                           T, k, B, x_row_div, Z=w.Zt, out=out)
    if w.Z is None:
        return w4a16_moe_gemm_swiglu(X, w.Wq, w.S, sorted_token_ids, expert_ids, ntpp, T, k, B,
                                     x_row_div, out)
    return w4a16_moe_gemm_swiglu_asym(X, w.Wq, w.S, w.Z, sorted_token_ids, expert_ids, ntpp, T,
                                      k, B, x_row_div, out)


@dataclass
class MoEBuffers:
    sorted_token_ids: torch.Tensor
    expert_ids: torch.Tensor
    ntpp: torch.Tensor
    H1: torch.Tensor            # None when the SwiGLU is fused into gate_up
    A: torch.Tensor
    H2: torch.Tensor
    out: torch.Tensor
    ws: torch.Tensor            # arrival counters of the fused combine (zeros)


def alloc_buffers(T, k, E, H, I, B, device, fused=True):
    cap = w4_moe_align_capacity(T, k, E, B)
    i32 = dict(dtype=torch.int32, device=device)
    bf = dict(dtype=torch.bfloat16, device=device)
    H1 = None if fused else torch.empty((T * k, 2 * I), **bf)
    return MoEBuffers(torch.empty(cap, **i32), torch.empty(cap // B, **i32),
                      torch.empty(1, **i32), H1,
                      torch.empty((T * k, I), **bf), torch.empty((T * k, H), **bf),
                      torch.empty((T, H), **bf),
                      torch.zeros(w4_moe_combine_workspace_words(T, k, E, H, B), **i32))


def moe_forward(X, topk_ids, topk_weights, gate_up, down, B=None, buffers=None, fused=True,
                fused_combine=False):
    """Expert part of the layer for routed tokens.

    X bf16 [T, H]; topk_ids int32 [T, k]; topk_weights fp32 [T, k];
    gate_up: E experts of [2I, H]; down: E experts of [H, I].  B defaults to
    ``w4_pick_block_size``.  ``fused``: SwiGLU in the gate_up epilogue;
    ``fused_combine``: the top-k combine in the down product
    (``w4a16_moe_gemm_combine``, symmetric experts).  Either way the result is
    the same bit for bit.  Returns (Out bf16 [T, H], buffers).
    """
    T, H = X.shape
    k = topk_ids.shape[1]
    E = gate_up.E
    I = gate_up.N // 2
    if down.E != E or down.N != H or down.K != I or gate_up.K != H:
        raise ValueError("expert weight shapes do not match X")
    if B is None:
        B = w4_pick_block_size(T, k, E)
    b = buffers or alloc_buffers(T, k, E, H, I, B, X.device, fused)
    moe_align_block_size(topk_ids, E, B, b.sorted_token_ids, b.expert_ids, b.ntpp)
    if fused:
        grouped_gemm_swiglu(X, gate_up, b.sorted_token_ids, b.expert_ids, b.ntpp, T, k, B, k,
                            out=b.A)
    else:
        if b.H1 is None:
            raise ValueError("the unfused path needs buffers with H1 (fused=False)")
        grouped_gemm(X, gate_up, b.sorted_token_ids, b.expert_ids, b.ntpp, T, k, B, k,
                     out=b.H1)
        w4_silu_mul(b.H1, out=b.A)
    if fused_combine:
        down_combine(b.A, down, b.sorted_token_ids, b.expert_ids, b.ntpp, topk_ids, topk_weights,
                     B, b)
    else:
        grouped_gemm(b.A, down, b.sorted_token_ids, b.expert_ids, b.ntpp, T, k, B, 1, out=b.H2)
        w4_moe_sum(b.H2, topk_weights, T, k, out=b.out)
    return b.out, b


def down_combine(A, w, sorted_token_ids, expert_ids, ntpp, topk_ids, topk_weights, B, b):
    """``w4a16_moe_gemm_combine`` on canonical or kernel-order symmetric
    experts ``w``: H2 and the combined output into buffers ``b``."""
    if w.Z is not None or w.Zt is not None:
        raise ValueError("the fused combine takes symmetric experts")
    if w.Wt is not None:
        return w4a16_moe_gemm_combine(A, w.Wt, w.St, sorted_token_ids, expert_ids, ntpp,
                                      topk_ids, topk_weights, B, N=w.N, tiled=True, H2=b.H2,
                                      out=b.out, workspace=b.ws)
    return w4a16_moe_gemm_combine(A, w.Wq, w.S, sorted_token_ids, expert_ids, ntpp, topk_ids,
                                  topk_weights, B, H2=b.H2, out=b.out, workspace=b.ws)


def moe_layer(X, logits, k, gate_up, down, B=None, buffers=None, fused=True,
              fused_combine=False):
    """Routing plus ``moe_forward``: logits fp32 [T, E] -> Out bf16 [T, H]."""
    ids, w = w4_moe_route(logits, k)
    out, b = moe_forward(X, ids, w, gate_up, down, B, buffers, fused, fused_combine)
    return out, ids, w, b
