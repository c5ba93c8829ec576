"""Pins for the oracle's bf16 rounding, quantizer, packing and fake quant.

Every check compares the oracle with something other than itself: the
tutorial's printed numbers, exact rational arithmetic (fractions), torch's
own bf16 conversion, closed-form bounds, or hand-computed words.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, quant

# --------------------------------------------------------------------------
# helpers independent of the oracle
# --------------------------------------------------------------------------

_ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _finite_bf16_values():
    """All finite non-negative bf16 values as (bits, Fraction), ascending."""
    out = []
    for b in range(0x0000, 0x7F80):
        e = (b >> 7) & 0xFF
        m = b & 0x7F
        if e == 0:
            v = Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
        else:
            v = (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))
        out.append((b, v))
    return out


_BF16_POS = None


def _bf16_table():
    global _BF16_POS
    if _BF16_POS is None:
        _BF16_POS = _finite_bf16_values()
    return _BF16_POS


def _round_fraction_to_bf16(v):
    """Nearest bf16 to a non-negative rational, ties to even mantissa."""
    import bisect
    table = _bf16_table()
    vals = [t[1] for t in table]
    i = bisect.bisect_left(vals, v)
    if i < len(vals) and vals[i] == v:
        return table[i][0]
    lo, hi = table[i - 1], table[i]
    dlo, dhi = v - lo[1], hi[1] - v
    if dlo < dhi:
        return lo[0]
    if dhi < dlo:
        return hi[0]
    return lo[0] if lo[0] % 2 == 0 else hi[0]


def _bf16_value(b):
    b = int(b)
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))


def _exact_quantize_group(wbits):
    """Exact-rational quantization of one group (the stated method)."""
    vals = [_bf16_value(b) for b in wbits]
    amax = max(abs(v) for v in vals)
    s_bits = _round_fraction_to_bf16(amax / 7)
    s = _bf16_value(s_bits)
    if s == 0:
        return [0] * len(vals), s_bits
    q = [max(-8, min(7, round(v / s))) for v in vals]   # round(): half to even
    return q, s_bits


def _rand_bf16(rng, shape, lo_exp=-20, hi_exp=5):
    """Random finite bf16 bit patterns with exponents in a range."""
    sign = rng.integers(0, 2, size=shape).astype(np.uint16) << 15
    exp = rng.integers(127 + lo_exp, 127 + hi_exp, size=shape).astype(np.uint16) << 7
    man = rng.integers(0, 128, size=shape).astype(np.uint16)
    return (sign | exp | man).astype(np.uint16)


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_bf16_widen_exact():
    vals = bf16.to_f32(_ALL_BF16)
    for b in [0x0000, 0x0001, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0x0080, 0x8001]:
        assert Fraction(float(vals[b])) == _bf16_value(b)


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact half-way patterns and their neighbours
    base = rng.integers(0, 1 << 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    u = np.concatenate([u, base | 0x8000, base | 0x7FFF, base | 0x8001])
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = bf16.rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_matches_exact_rational_ties():
    # value exactly half-way between two bf16 neighbours -> even mantissa
    cases = [
        (0x3F808000, 0x3F80),   # 1 + 2^-8: between 1 and 1+2^-7 -> even (1.0)
        (0x3F818000, 0x3F82),   # between 0x3F81 and 0x3F82 -> even 0x3F82
        (0x3F817FFF, 0x3F81),
        (0x3F818001, 0x3F82),
        (0x7F7FFFFF, 0x7F80),   # rounds up to +inf
        (0x00008000, 0x0000),   # subnormal tie -> even (0)
        (0x00018000, 0x0002),   # subnormal tie -> even
    ]
    for u, want in cases:
        f = np.array([u], dtype=np.uint32).view(np.float32)
        assert int(bf16.rne(f)[0]) == want
        if want != 0x7F80:
            v = Fraction(float(f[0]))
            assert _round_fraction_to_bf16(v) == want


# --------------------------------------------------------------------------
# the tutorial's worked INT8 example (§6.1) through the same quantizer
# --------------------------------------------------------------------------

def test_tutorial_int8_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tutorial_int8_example.json")))
    rng = np.random.default_rng(42)
    w = rng.standard_normal(200_000) * 0.05
    w[:500] *= 6.0
    w16 = w.astype(np.float16).astype(np.float64)
    q, s, w_hat = quant.generic_symmetric(w16, 127)
    err = w_hat - w16
    p = g["printed"]
    assert f"{s:.6f}" == p["scale"]
    assert f"{s / 2:.6f}" == p["half_scale"]
    assert f"{np.abs(err).max():.6f}" == p["max_abs_err"]
    assert f"{np.abs(err).mean():.6f}" == p["mae"]
    assert f"{np.linalg.norm(err) / np.linalg.norm(w16) * 100:.6f}" == p["rel_l2_percent"]
    assert len(np.unique(q)) == p["codes_used"]


# --------------------------------------------------------------------------
# INT4 quantizer vs exact rational arithmetic
# --------------------------------------------------------------------------

def test_quantize_matches_exact_rationals_random_groups():
    rng = np.random.default_rng(11)
    W = _rand_bf16(rng, (24, 64))
    # a few groups with wildly different magnitudes inside
    W[3, :32] = _rand_bf16(rng, (32,), lo_exp=-60, hi_exp=-50)
    W[3, 5] = 0x3F80
    q, S = quant.quantize(W)
    for n in range(W.shape[0]):
        for g in range(W.shape[1] // 32):
            want_q, want_s = _exact_quantize_group(W[n, 32 * g:32 * g + 32])
            assert int(S[n, g]) == want_s, (n, g)
            assert list(q[n, 32 * g:32 * g + 32]) == want_q, (n, g)


def test_fp32_division_equals_exact_rounding_exhaustive():
    """rint(fl32(w / s)) == round_half_even(w / s) for all bf16 mantissa pairs.

    Justifies taking the code decision in fp32 (IEEE division): the quotient
    of two bf16 values never rounds across or onto a half-integer.  Covers
    every mantissa of s and w and every exponent gap that can give |w/s| <= 8.
    """
    man = np.arange(128, dtype=np.uint16)
    s_bits = (np.uint16(127 << 7) | man)                       # s in [1, 2)
    fails = 0
    for gap in range(-9, 4):                                    # w exponent - s exponent
        w_bits = (np.uint16((127 + gap) << 7) | man)
        s = bf16.to_f32(s_bits)[:, None]
        w = bf16.to_f32(w_bits)[None, :]
        r = np.rint((w / s).astype(np.float32))
        for i in range(128):
            for j in range(128):
                exact = Fraction(float(w[0, j])) / Fraction(float(s[i, 0]))
                if round(exact) != r[i, j]:
                    fails += 1
    assert fails == 0


def test_constructed_ties_round_half_even():
    # amax = 7 -> s = 1 exactly; w / s hits exact half-integers
    vals = [7.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 4.5, 5.5, 6.5, -6.5]
    want = [7, 0, 2, 2, 4, 0, -2, -2, -4, 4, 6, 6, -6]
    row = np.zeros(32, dtype=np.float32)
    row[:len(vals)] = vals
    W = bf16.rne(row)[None, :]
    q, S = quant.quantize(W)
    assert int(S[0, 0]) == 0x3F80
    assert list(q[0, :len(vals)]) == want


def test_truncating_round_would_fail_tie_case():
    """A truncating cast differs from half-to-even on the constructed data
    (tutorial §5 (1) and FAQ Q2 warn about it), so the tie test above can
    tell them apart."""
    r = np.array([2.5, 3.5, -2.5, 6.9], dtype=np.float32)
    assert list(np.rint(r)) != list(np.trunc(r))


def test_range_and_amax_code_exhaustive_over_scales():
    """For every bf16 amax mantissa (and several binades) the amax element
    quantizes to +-7 and no code leaves [-7, 7]."""
    man = np.arange(128, dtype=np.uint16)
    for exp in [127 - 30, 127 - 6, 127, 127 + 20]:
        amax_bits = np.uint16(exp << 7) | man
        W = np.zeros((128, 32), dtype=np.uint16)
        rng = np.random.default_rng(exp)
        amax_f = bf16.to_f32(amax_bits)
        fill = (rng.uniform(-1, 1, size=(128, 31)) * amax_f[:, None]).astype(np.float32)
        W[:, 1:] = bf16.rne(fill)
        W[:, 0] = amax_bits
        W[::2, 0] |= 0x8000                    # negative amax on even rows
        # make sure column 0 really holds the max magnitude
        mag = np.abs(bf16.to_f32(W))
        assert np.all(mag[:, 0] >= mag[:, 1:].max(axis=1))
        q, S = quant.quantize(W)
        assert np.all(np.abs(q) <= 7)
        assert np.all(np.abs(q[:, 0]) == 7)
        assert np.all(np.sign(q[:, 0]) == np.where(np.arange(128) % 2 == 0, -1, 1))


def test_error_bound_half_scale():
    """|w - q*s| <= s/2 exactly (tutorial §2.4), and the bf16 dequantized
    value adds at most half a bf16 ulp of q*s."""
    rng = np.random.default_rng(3)
    W = bf16.rne((rng.standard_normal((64, 512)) * 0.02).astype(np.float32))
    q, S = quant.quantize(W)
    w = bf16.to_f32(W).astype(np.float64).reshape(64, 16, 32)
    s = bf16.to_f32(S).astype(np.float64)[:, :, None]
    qs = q.astype(np.float64).reshape(64, 16, 32) * s
    assert np.all(np.abs(w - qs) <= s / 2)
    wd = bf16.to_f32(quant.dequant(q, S)).astype(np.float64).reshape(64, 16, 32)
    assert np.all(np.abs(w - wd) <= s / 2 + np.abs(qs) * 2.0 ** -8)


def test_mean_abs_error_is_about_quarter_scale():
    """Rounding error is about uniform on [-s/2, s/2]: mean |e| ~ s/4 (§6.1)."""
    rng = np.random.default_rng(5)
    W = bf16.rne((rng.standard_normal((256, 1024)) * 0.02).astype(np.float32))
    q, S = quant.quantize(W)
    w = bf16.to_f32(W).astype(np.float64).reshape(256, 32, 32)
    s = bf16.to_f32(S).astype(np.float64)[:, :, None]
    e = np.abs(w - q.astype(np.float64).reshape(256, 32, 32) * s) / s
    assert abs(e.mean() - 0.25) < 0.01


def test_sign_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(8)
    W = bf16.rne((rng.standard_normal((16, 256)) * 0.02).astype(np.float32))
    q, S = quant.quantize(W)
    qn, Sn = quant.quantize(W ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(Sn, S)
    W4 = bf16.rne(bf16.to_f32(W) * np.float32(4.0))
    q4, S4 = quant.quantize(W4)
    assert np.array_equal(q4, q)
    assert np.array_equal(bf16.to_f32(S4), bf16.to_f32(S) * np.float32(4.0))


def test_zero_and_underflowing_groups():
    W = np.zeros((2, 64), dtype=np.uint16)
    W[1, :32] = 0x0001            # smallest subnormal: amax/7 rounds to 0 in bf16
    W[1, 32:] = 0x8001
    q, S = quant.quantize(W)
    assert np.all(q == 0) and np.all(S == 0)
    assert np.all(quant.dequant(q, S) == 0)


def test_subnormal_group_kept():
    W = np.zeros((1, 32), dtype=np.uint16)
    W[0, :] = 0x0070              # subnormal bf16 values, no flush to zero
    W[0, 3] = 0x0075
    q, S = quant.quantize(W)
    want_q, want_s = _exact_quantize_group(W[0])
    assert int(S[0, 0]) == want_s and want_s != 0
    assert list(q[0]) == want_q


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------

def test_pack_known_word():
    q = np.array([[1, -1, 2, -2, 3, -3, 7, -8]], dtype=np.int8)
    # nibbles (low to high): 1, F, 2, E, 3, D, 7, 8  ->  0x87D3E2F1
    w = quant.pack(q)
    assert w.dtype == np.int32
    assert int(w.view(np.uint32)[0, 0]) == 0x87D3E2F1


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(9)
    q = rng.integers(-8, 8, size=(33, 256)).astype(np.int8)
    assert np.array_equal(quant.unpack(quant.pack(q)), q)


def test_packed_sizes():
    # "two 4-bit weights per byte, 75% less than BF16" before scales
    N, K = 12288, 4096
    codes = N * K // 2
    assert codes == (N * K * 2) // 4
    total = quant.packed_bytes(N, K)
    assert total == 28_311_552                   # 4.5 bits per weight
    assert total * 8 == N * K * 4.5
    assert abs(1 - total / (N * K * 2) - 0.71875) < 1e-12


# --------------------------------------------------------------------------
# fake quant
# --------------------------------------------------------------------------

def test_fake_quant_equals_dequant_of_packed():
    rng = np.random.default_rng(12)
    W = bf16.rne((rng.standard_normal((40, 320)) * 0.02).astype(np.float32))
    Wq, S = quant.quantize_pack(W)
    via_pack = quant.dequant(quant.unpack(Wq), S)
    assert np.array_equal(quant.fake_quant(W), via_pack)


def test_fake_quant_values_exact():
    """Each fake-quantized value is the bf16 nearest to q*s (exact rationals)."""
    rng = np.random.default_rng(13)
    W = _rand_bf16(rng, (4, 64), lo_exp=-8, hi_exp=2)
    fq = quant.fake_quant(W)
    for n in range(4):
        for g in range(2):
            qq, sb = _exact_quantize_group(W[n, 32 * g:32 * g + 32])
            s = _bf16_value(sb)
            for i in range(32):
                v = qq[i] * s
                want = _round_fraction_to_bf16(abs(v)) | (0x8000 if v < 0 else 0)
                got = int(fq[n, 32 * g + i])
                if v == 0:
                    assert got & 0x7FFF == 0
                else:
                    assert got == want


@pytest.mark.parametrize("exp", [127 - 12, 127 - 6, 127])
def test_fake_quant_idempotent_over_all_scale_mantissas(exp):
    """fake_quant(fake_quant(W)) == fake_quant(W) for every bf16 amax mantissa."""
    man = np.arange(128, dtype=np.uint16)
    rng = np.random.default_rng(exp)
    W = np.zeros((128, 32), dtype=np.uint16)
    amax_bits = np.uint16(exp << 7) | man
    amax_f = bf16.to_f32(amax_bits)
    W[:, 1:] = bf16.rne((rng.uniform(-1, 1, size=(128, 31)) * amax_f[:, None]).astype(np.float32))
    W[:, 0] = amax_bits
    f1 = quant.fake_quant(W)
    f2 = quant.fake_quant(f1)
    assert np.array_equal(f1, f2)
