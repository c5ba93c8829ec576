"""Top-k routed MoE expert layer with W4A16 experts -- oracle.

Test infrastructure only.  Sources: "INT4 QAT end-to-end for RL", §4
inference and §5.3 rollout speed-up: the inference engine merges and aligns
each expert's token set (a dynamic ``moe_align_block_size``), fuses the
MoE operators and fuses gating into one kernel; "Quantization-aware
training" tag summary, bullet [35]: the block size is chosen automatically
from the current token count and expert distribution to use memory
bandwidth better.  The pages give no formulas for routing, alignment or the
expert activation; the readings used here are:

* Routing: p = softmax(logits[t, :]) over the E experts; the k experts with
  the largest logits (ties to the lower expert index) are selected and their
  probabilities renormalised to sum to 1.  A NaN logit is never selected
  while a number is left and takes no part in the softmax.  (parity unpinned as a choice of
  method; pinned as arithmetic by closed-form identities.)
* Block size: B = min(64, max(16, next_pow2(ceil(T*k / E)))).  (parity
  unpinned: a convention.)
* Alignment: pairs f = t*k + j with expert e = ids[t, j] (ids outside
  [0, E) are skipped); experts in ascending order, each expert's pairs in
  ascending f, each segment padded with the sentinel T*k to a multiple of
  B; one expert id per block; the total padded length; positions past the
  total hold the sentinel and blocks past it hold -1.
* Activation: SwiGLU, a = silu(gate) * up, gate = the first I rows of the
  gate_up weight, up = the last I.  (parity unpinned: a convention.)
* Combine: out[t] = sum over j = 0..k-1 of w[t, j] * down_out[t*k + j].
* Storage points: the gate_up output, the activation and the down output
  are rounded to bf16, the final output too.
* Zero-point experts ("Quantization basics: from FP32 to INT4" §2.3): an
  expert's weights given as (Wq, S, Z) are dequantized as bf16((q - z) s);
  everything else is unchanged.
"""

import numpy as np

from . import bf16, gemm


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def route(logits, k):
    """Softmax top-k routing.  ``logits`` float32 [T, E].

    Returns (ids int32 [T, k], weights float32 [T, k]); each row of ids is
    ordered by descending logit, ties by ascending expert index.
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        row = lg[t]
        num = ~np.isnan(row)           # NaN logits are never picked and carry no mass
        p = np.zeros(E)
        if num.any():
            p[num] = np.exp(row[num] - row[num].max())
            p = p / p.sum()
        p[~num] = np.nan
        order = np.lexsort((np.arange(E), -row))[:k]
        sel = p[order]
        ids[t] = order
        w[t] = (sel / sel.sum()).astype(np.float32)
    return ids, w


# --------------------------------------------------------------------------
# alignment
# --------------------------------------------------------------------------

def next_pow2(x):
    p = 1
    while p < x:
        p *= 2
    return p


def pick_block_size(T, k, E):
    """B = min(64, max(16, next_pow2(ceil(T*k / E))))."""
    mean = -(-(T * k) // E)
    return min(64, max(16, next_pow2(mean)))


def capacity(T, k, E, B):
    """Largest possible padded length: round_up(T*k + E*(B-1), B)."""
    n = T * k + E * (B - 1)
    return -(-n // B) * B


def align(ids, E, B):
    """moe_align_block_size reference.

    ``ids`` int [T, k].  Returns (sorted_token_ids int32 [cap],
    expert_ids int32 [cap / B], num_tokens_post_padded int).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    sentinel = T * k
    cap = capacity(T, k, E, B)
    flat = ids.reshape(-1)
    per_expert = [[] for _ in range(E)]
    for f in range(T * k):           # ascending f keeps each list stable
        e = int(flat[f])
        if 0 <= e < E:
            per_expert[e].append(f)
    sorted_ids = np.full(cap, sentinel, dtype=np.int32)
    expert_ids = np.full(cap // B, -1, dtype=np.int32)
    pos = 0
    for e in range(E):
        rows = per_expert[e]
        padded = -(-len(rows) // B) * B
        sorted_ids[pos:pos + len(rows)] = rows
        expert_ids[pos // B:(pos + padded) // B] = e
        pos += padded
    return sorted_ids, expert_ids, pos


# --------------------------------------------------------------------------
# expert GEMMs and the element-wise stages
# --------------------------------------------------------------------------

def grouped_gemm(X, weights, sorted_ids, expert_ids, ntpp, B, x_row_div,
                 n_pairs, topk_weights=None, experts=None):
    """Reference of the aligned grouped W4A16 GEMM.

    For every block b < ntpp / B with expert e = expert_ids[b], and every
    slot holding a valid pair f (f < n_pairs): row f of the result is
    X[f // x_row_div] * dequant(W_e)^T, multiplied by topk_weights.flat[f]
    when given.  ``weights(e)`` returns (Wq int32 [N, K/8], S bf16 [N, K/32])
    or, for zero-point experts, (Wq, S, Z uint8 [N, K/32]).
    ``experts``, when given, restricts the product to blocks of those experts
    (a sampled check at sizes where the whole product is too slow here).
    Returns {f: float64 row} for the rows written.

    The rows of one expert are stacked and multiplied by its dequantized
    weights in one float64 matmul: each row is the same dot products as a
    row-at-a-time evaluation, only the order of the float64 additions may
    differ (about 1e-16 relative, far below the bf16 outputs compared).
    """
    x = bf16.to_f32(X).astype(np.float64)
    tw = None if topk_weights is None else np.asarray(topk_weights, np.float64).reshape(-1)
    rows_of = {}                       # expert -> its valid pairs, in slot order
    for b in range(ntpp // B):
        e = int(expert_ids[b])
        if experts is not None and e not in experts:
            continue
        for i in range(B):
            f = int(sorted_ids[b * B + i])
            if f < n_pairs:
                rows_of.setdefault(e, []).append(f)
    out = {}
    for e, fs in rows_of.items():
        w = gemm.dequant_weights_f64(*weights(e))
        fa = np.asarray(fs, dtype=np.int64)
        y = x[fa // x_row_div] @ w.T
        if tw is not None:
            y = y * tw[fa][:, None]
        for i, f in enumerate(fs):
            out[f] = y[i]
    return out


def silu(v):
    """silu(v) = v / (1 + exp(-v)) in float64."""
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def silu_mul(H1):
    """SwiGLU on bf16 rows [R, 2I]: a = silu(gate) * up, returned as float64."""
    h = bf16.to_f32(H1).astype(np.float64)
    I = h.shape[1] // 2
    return silu(h[:, :I]) * h[:, I:]


def moe_sum(H2, topk_weights):
    """out[t] = sum_{j in order} w[t, j] * H2[t*k + j] in float64.

    ``H2`` bf16 bits [T*k, H]; ``topk_weights`` float32 [T, k].
    """
    w = np.asarray(topk_weights, dtype=np.float64)
    T, k = w.shape
    h = bf16.to_f32(H2).astype(np.float64).reshape(T, k, -1)
    out = np.zeros((T, h.shape[2]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * h[:, j, :]
    return out


# --------------------------------------------------------------------------
# the whole layer, straight from the definition (no alignment involved)
# --------------------------------------------------------------------------

def expert_h2(X, pairs, gate_up_w, down_w):
    """One expert's part of the layer: for each pair (t, j) routed to it,
      h1 = bf16(X[t] * dequant(Wgu_e)^T)          [2I]
      a  = bf16(silu(h1[:I]) * h1[I:])             [I]
      h2 = bf16(a * dequant(Wdn_e)^T)              [H]
    ``gate_up_w`` / ``down_w`` are (Wq, S), or (Wq, S, Z) for zero-point
    experts.  The pairs' rows are stacked into one float64 matmul per
    projection.  Returns {(t, j): float64 h2 row}."""
    x = bf16.to_f32(X).astype(np.float64)
    wgu = gemm.dequant_weights_f64(*gate_up_w)
    wdn = gemm.dequant_weights_f64(*down_w)
    I = wgu.shape[0] // 2
    toks = np.asarray([t for (t, _) in pairs], dtype=np.int64)
    h1 = bf16.to_f32(gemm.to_bf16(x[toks] @ wgu.T)).astype(np.float64)
    a = bf16.to_f32(gemm.to_bf16(silu(h1[:, :I]) * h1[:, I:])).astype(np.float64)
    h2 = bf16.to_f32(gemm.to_bf16(a @ wdn.T)).astype(np.float64)
    return {p: h2[i] for i, p in enumerate(pairs)}


def pairs_by_expert(ids, tokens):
    """{expert: [(t, j), ...]} for the given tokens' routed pairs."""
    ids = np.asarray(ids)
    need = {}
    for t in tokens:
        for j in range(ids.shape[1]):
            need.setdefault(int(ids[t, j]), []).append((int(t), j))
    return need


def combine_tokens(topk_weights, h2, tokens):
    """out[t] = sum over j = 0..k-1, in order, of w[t, j] * h2[(t, j)]."""
    w = np.asarray(topk_weights, dtype=np.float64)
    out = {}
    for t in tokens:
        acc = np.zeros_like(h2[(t, 0)])
        for j in range(w.shape[1]):
            acc = acc + w[t, j] * h2[(t, j)]
        out[t] = acc
    return out


def moe_layer(X, ids, topk_weights, gate_up, down, tokens=None):
    """MoE layer output for the given tokens, from the per-token definition:
    each token's k routed pairs go through expert_h2 (gate_up, SwiGLU, down,
    bf16 at each storage point) and are combined with the top-k weights
    (combine_tokens).  ``gate_up(e)`` / ``down(e)`` return (Wq, S), or
    (Wq, S, Z) for zero-point experts, of expert e.  Returns {t: float64
    row} for the requested tokens (all when None).  Weights are dequantized
    one expert at a time, so only the experts used by the requested tokens
    are touched."""
    T = np.asarray(ids).shape[0]
    toks = list(range(T)) if tokens is None else [int(t) for t in tokens]
    h2 = {}
    for e, pairs in sorted(pairs_by_expert(ids, toks).items()):
        h2.update(expert_h2(X, pairs, gate_up(e), down(e)))
    return combine_tokens(topk_weights, h2, toks)
