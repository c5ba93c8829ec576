"""Pins for the oracle's routing, alignment and MoE layer."""

import math

import numpy as np
import pytest

from oracle import bf16, gemm, moe, quant, quant_asym


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def test_route_identities():
    rng = np.random.default_rng(31)
    T, E, k = 50, 24, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = moe.route(lg, k)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    for t in range(T):
        sel = set(ids[t].tolist())
        assert len(sel) == k
        kth = min(lg[t, list(sel)])
        assert all(lg[t, e] <= kth for e in range(E) if e not in sel)
        # renormalised softmax == softmax over the selected logits alone
        l_sel = [float(lg[t, e]) for e in ids[t]]
        z = sum(math.exp(v - max(l_sel)) for v in l_sel)
        want = [math.exp(v - max(l_sel)) / z for v in l_sel]
        assert np.allclose(w[t], want, rtol=1e-6)
        assert all(lg[t, ids[t][i]] >= lg[t, ids[t][i + 1]] for i in range(k - 1))


def test_route_nan_logits_never_picked_and_carry_no_mass():
    """NaN logits (absent experts) are never selected while numbers are
    left, and the weights are the softmax over the selected logits alone
    (closed form exp(l_j - l_0) / sum_i exp(l_i - l_0), computed here with
    math.exp on the selected values)."""
    rng = np.random.default_rng(11)
    lg = rng.normal(size=(3, 40)).astype(np.float32)
    lg[0, [0, 7, 11, 12, 39]] = np.nan
    lg[1, ::3] = np.nan
    lg[2, :] = np.nan
    lg[2, [6, 21, 2]] = [0.25, -3.0, 1.5]
    ids, w = moe.route(lg, 8)
    for t in (0, 1):
        assert not np.any(np.isnan(lg[t, ids[t]]))
        sel = [float(lg[t, e]) for e in ids[t]]
        assert sel == sorted(sel, reverse=True)
        ex = [math.exp(v - sel[0]) for v in sel]
        np.testing.assert_allclose(w[t], np.array(ex) / math.fsum(ex), rtol=1e-6)
        finite = np.sort(lg[t][~np.isnan(lg[t])])[::-1][:8]
        np.testing.assert_array_equal(np.sort(lg[t, ids[t]])[::-1], finite)
    # fewer numbers than k: the numbers first, then the lowest NaN indices
    assert ids[2].tolist() == [2, 6, 21, 0, 1, 3, 4, 5]


def test_route_tie_break_lower_index_first():
    lg = np.zeros((1, 6), dtype=np.float32)
    lg[0, 4] = 1.0
    ids, w = moe.route(lg, 3)
    assert ids[0].tolist() == [4, 0, 1]
    assert abs(w[0, 1] - w[0, 2]) == 0


# --------------------------------------------------------------------------
# block size and capacity
# --------------------------------------------------------------------------

def test_pick_block_size_values():
    assert moe.pick_block_size(256, 8, 128) == 16        # mean 16 rows/expert
    assert moe.pick_block_size(4096, 8, 384) == 64       # mean 85.3
    assert moe.pick_block_size(1, 8, 384) == 16
    assert moe.pick_block_size(512, 8, 128) == 32
    assert moe.pick_block_size(10 ** 6, 8, 8) == 64


def test_capacity_bounds_total():
    rng = np.random.default_rng(32)
    for B in [1, 16, 64]:
        T, k, E = 37, 4, 9
        ids = rng.integers(0, E, size=(T, k))
        s, e, ntpp = moe.align(ids, E, B)
        assert ntpp <= moe.capacity(T, k, E, B)
        assert len(s) == moe.capacity(T, k, E, B) and len(s) % B == 0
    # worst case: every expert gets one pair -> E blocks
    T, k, E, B = 1, 4, 4, 64
    s, e, ntpp = moe.align(np.arange(4).reshape(1, 4), E, B)
    assert ntpp == 4 * 64 and moe.capacity(T, k, E, B) == 4 * 64


# --------------------------------------------------------------------------
# alignment
# --------------------------------------------------------------------------

def test_align_block_one_is_stable_argsort():
    rng = np.random.default_rng(33)
    T, k, E = 40, 3, 7
    ids = rng.integers(0, E, size=(T, k))
    s, e, ntpp = moe.align(ids, E, 1)
    order = np.argsort(ids.reshape(-1), kind="stable")
    assert ntpp == T * k
    assert np.array_equal(s[:ntpp], order)
    assert np.array_equal(e[:ntpp], np.sort(ids.reshape(-1), kind="stable"))


def test_align_brute_force_with_python_sorted_and_skips():
    rng = np.random.default_rng(34)
    T, k, E, B = 29, 4, 6, 4
    ids = rng.integers(-2, E + 2, size=(T, k))      # some ids outside [0, E)
    s, e, ntpp = moe.align(ids, E, B)
    pairs = sorted((int(ids.flat[f]), f) for f in range(T * k) if 0 <= ids.flat[f] < E)
    want_s, want_e = [], []
    for ex in range(E):
        rows = [f for (x, f) in pairs if x == ex]
        pad = -(-len(rows) // B) * B
        want_s += rows + [T * k] * (pad - len(rows))
        want_e += [ex] * (pad // B)
    assert ntpp == len(want_s)
    assert s[:ntpp].tolist() == want_s
    assert e[:ntpp // B].tolist() == want_e
    assert np.all(s[ntpp:] == T * k) and np.all(e[ntpp // B:] == -1)


def test_align_invariants_skewed():
    rng = np.random.default_rng(35)
    T, k, E, B = 300, 8, 16, 16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    ids[:60] = np.arange(k)                        # hot experts 0..7
    s, e, ntpp = moe.align(ids, E, B)
    valid = s[:ntpp][s[:ntpp] < T * k]
    assert sorted(valid.tolist()) == list(range(T * k))      # a permutation
    assert np.all(np.diff(e[:ntpp // B]) >= 0)               # experts ascending
    for b in range(ntpp // B):
        blk = s[b * B:(b + 1) * B]
        v = blk[blk < T * k]
        assert np.all(ids.flat[v] == e[b])
        assert np.all(np.diff(v) > 0)


# --------------------------------------------------------------------------
# element-wise stages
# --------------------------------------------------------------------------

def test_silu_closed_forms():
    assert moe.silu(0.0) == 0.0
    assert abs(moe.silu(1.0) - 1.0 / (1.0 + math.e ** -1)) < 1e-15
    assert abs(moe.silu(30.0) - 30.0) < 1e-9
    assert abs(moe.silu(-30.0)) < 1e-9
    # silu(-x) = silu(x) - x
    v = np.linspace(-5, 5, 11)
    assert np.allclose(moe.silu(-v), moe.silu(v) - v)


def test_silu_mul_gate_then_up():
    h = np.array([[1.0, 2.0, 3.0, 10.0, 20.0, 30.0]], dtype=np.float32)
    a = moe.silu_mul(bf16.rne(h))
    assert np.allclose(a[0], moe.silu(np.array([1.0, 2.0, 3.0])) * [10.0, 20.0, 30.0])


def test_moe_sum_order_and_weights():
    H2 = bf16.rne(np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]], dtype=np.float32))
    w = np.array([[0.25, 0.75], [1.0, 0.0]], dtype=np.float32)
    out = moe.moe_sum(H2, w)
    assert np.allclose(out, [[0.25 * 1 + 0.75 * 3, 0.25 * 2 + 0.75 * 4], [5.0, 6.0]])


# --------------------------------------------------------------------------
# layer-level reductions
# --------------------------------------------------------------------------

def _expert_bank(rng, E, N, K):
    bank = []
    for _ in range(E):
        W = bf16.rne((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
        bank.append(quant.quantize_pack(W))
    return bank


def test_grouped_gemm_single_expert_equals_dense():
    rng = np.random.default_rng(36)
    T, N, K = 9, 48, 64
    bank = _expert_bank(rng, 1, N, K)
    X = bf16.rne(rng.standard_normal((T, K)).astype(np.float32))
    ids = np.zeros((T, 1), dtype=np.int32)
    s, e, ntpp = moe.align(ids, 1, 4)
    rows = moe.grouped_gemm(X, lambda ex: bank[ex], s, e, ntpp, 4, 1, T)
    dense = gemm.w4a16_gemm(X, *bank[0])
    assert sorted(rows) == list(range(T))
    for f in range(T):
        assert np.array_equal(rows[f], dense[f])


@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("B,x_row_div,weighted", [(1, 3, False), (4, 3, True), (16, 1, True),
                                                  (5, 1, False)])
def test_grouped_gemm_batched_rows_equal_exact_dot_products(zp, B, x_row_div, weighted):
    """Each expert's rows are one stacked float64 matmul; every row must be
    the exact dot product X[f // x_row_div] . w'_e[n] (math.fsum of the
    products, each exact in float64: bf16 times bf16) within float64
    summation rounding, times the pair's top-k weight.  A wrong expert,
    row, block or weight index fails by orders of magnitude."""
    rng = np.random.default_rng(91 + B + 7 * x_row_div + zp)
    T, k, E, N, K = 9, 3, 4, 6, 64
    if zp:
        bank = []
        for _ in range(E):
            W = bf16.rne((rng.standard_normal((N, K)) * 0.05 + 0.01).astype(np.float32))
            bank.append(quant_asym.quantize_pack_asym(W))
    else:
        bank = _expert_bank(rng, E, N, K)
    rows = T * k // x_row_div
    X = bf16.rne(rng.standard_normal((rows, K)).astype(np.float32))
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)     # some ids skipped
    tw = rng.random((T, k)).astype(np.float32) if weighted else None
    s, ex, ntpp = moe.align(ids, E, B)
    got = moe.grouped_gemm(X, lambda e: bank[e], s, ex, ntpp, B, x_row_div, T * k,
                           topk_weights=tw)
    x = bf16.to_f32(X).astype(np.float64)
    expect_rows = {f for f in range(T * k) if 0 <= ids.flat[f] < E}
    assert set(got) == expect_rows
    for f in expect_rows:
        w = gemm.dequant_weights_f64(*bank[int(ids.flat[f])])
        xr = x[f // x_row_div]
        for n in range(N):
            exact = math.fsum(float(a) * float(b) for a, b in zip(xr, w[n]))
            if weighted:
                exact *= float(tw.flat[f])
            bound = 1e-14 * (math.fsum(abs(float(a) * float(b)) for a, b in zip(xr, w[n])) + 1e-300)
            assert abs(got[f][n] - exact) <= bound, (f, n, got[f][n], exact)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_layer_definition_equals_aligned_pipeline(B):
    """The per-token definition and the align -> grouped GEMM -> SwiGLU ->
    grouped GEMM -> combine pipeline give the same layer output."""
    rng = np.random.default_rng(37 + B)
    T, E, k, H, I = 12, 5, 2, 64, 32
    gu = _expert_bank(rng, E, 2 * I, H)
    dn = _expert_bank(rng, E, H, I)
    X = bf16.rne(rng.standard_normal((T, H)).astype(np.float32))
    ids, w = moe.route(rng.standard_normal((T, E)).astype(np.float32), k)
    ref = moe.moe_layer(X, ids, w, lambda e: gu[e], lambda e: dn[e])

    s, ex, ntpp = moe.align(ids, E, B)
    h1 = moe.grouped_gemm(X, lambda e: gu[e], s, ex, ntpp, B, k, T * k)
    H1 = np.stack([gemm.to_bf16(h1[f]) for f in range(T * k)])
    A = gemm.to_bf16(moe.silu_mul(H1))
    h2 = moe.grouped_gemm(A, lambda e: dn[e], s, ex, ntpp, B, 1, T * k)
    H2 = np.stack([gemm.to_bf16(h2[f]) for f in range(T * k)])
    out = moe.moe_sum(H2, w)
    for t in range(T):
        assert np.array_equal(out[t], ref[t])


# --------------------------------------------------------------------------
# zero-point experts ("Quantization basics: from FP32 to INT4" §2.3)
# --------------------------------------------------------------------------

def _integer_zp_expert(rng, N, K):
    """Integer weights whose groups span exactly [lo, lo + 15], lo drawn per
    group from [-15, 0]: the asymmetric quantizer gives s = 1, z = -lo, and
    the dequantized weights are the integers themselves."""
    G = K // 32
    lo = rng.integers(-15, 1, size=(N, G, 1)).astype(np.float32)
    w = lo + rng.integers(0, 16, size=(N, G, 32)).astype(np.float32)
    w[:, :, 5] = lo[:, :, 0]
    w[:, :, 20] = lo[:, :, 0] + 15.0
    return w.reshape(N, K)


def test_grouped_gemm_zero_point_integer_experts_is_integer_matmul():
    """Per-group zero points that differ by row, group and expert: every
    grouped row is the textbook integer product with its expert's weights."""
    rng = np.random.default_rng(61)
    T, E, k, N, K, B = 10, 3, 2, 40, 96, 4
    ws = [_integer_zp_expert(rng, N, K) for _ in range(E)]
    bank = [quant_asym.quantize_pack_asym(bf16.rne(w)) for w in ws]
    for w, (_, S, Z) in zip(ws, bank):
        assert np.all(bf16.to_f32(S) == 1.0)
        assert len(np.unique(Z)) > 8
    x = rng.integers(-3, 4, size=(T, K)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    s, ex, ntpp = moe.align(ids, E, B)
    rows = moe.grouped_gemm(bf16.rne(x), lambda e: bank[e], s, ex, ntpp, B, k, T * k)
    assert sorted(rows) == list(range(T * k))
    for f in range(T * k):
        e = int(ids.reshape(-1)[f])
        assert np.array_equal(rows[f], x[f // k].astype(np.float64) @ ws[e].astype(np.float64).T)


def test_layer_zero_point_reencoding_equals_symmetric():
    """Symmetric codes re-encoded as unsigned q + 8 with z = 8 dequantize to
    the same weights, so the whole layer output is unchanged."""
    rng = np.random.default_rng(62)
    T, E, k, H, I = 8, 4, 2, 64, 32
    gu = _expert_bank(rng, E, 2 * I, H)
    dn = _expert_bank(rng, E, H, I)

    def reencode(Wq, S):
        q = quant.unpack(Wq).astype(np.int16) + 8
        return quant_asym.pack_unsigned(q.astype(np.uint8)), S, np.full(S.shape, 8, np.uint8)

    gu_z = [reencode(*w) for w in gu]
    dn_z = [reencode(*w) for w in dn]
    X = bf16.rne(rng.standard_normal((T, H)).astype(np.float32))
    ids, w = moe.route(rng.standard_normal((T, E)).astype(np.float32), k)
    ref = moe.moe_layer(X, ids, w, lambda e: gu[e], lambda e: dn[e])
    got = moe.moe_layer(X, ids, w, lambda e: gu_z[e], lambda e: dn_z[e])
    for t in range(T):
        assert np.array_equal(got[t], ref[t])
