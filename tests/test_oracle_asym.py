"""Pins for the oracle's asymmetric (zero-point) INT4 quantizer.

The pages print no worked asymmetric example, so the oracle is pinned by:
an exact-rational model of the stated method (fractions, with every fp32
rounding of the stated arithmetic done explicitly), the tutorial's error
bound |x_hat - x| <= s/2 for values that are not clamped, the zero-point
property (0 is on the grid), closed forms for constant and integer groups,
and hand-computed packed words.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, gemm, quant_asym

# --------------------------------------------------------------------------
# exact-rational helpers (independent of the oracle)
# --------------------------------------------------------------------------


def _bf16_value(b):
    b = int(b)
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(m, 1 << 7)) * (Fraction(2) ** (e - 127))


def _round_half_even(v):
    """Nearest integer to a rational, ties to even (Python's round on Fraction)."""
    return round(v)


def _round_to_precision(v, mant_bits, min_exp):
    """Nearest binary float with ``mant_bits`` significant bits (including the
    leading one) and least exponent ``min_exp`` (subnormals), ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e <= a < 2^(e+1) after adjustment
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp_exp = max(e - (mant_bits - 1), min_exp)
    ulp = Fraction(2) ** ulp_exp
    return sign * _round_half_even(a / ulp) * ulp


def _f32(v):
    return _round_to_precision(v, 24, -149)


def _bf16(v):
    return _round_to_precision(v, 8, -133)


def _exact_asym_group(wbits):
    """The stated method on one group with exact rationals and explicit fp32
    roundings: returns (q list, s, z)."""
    vals = [_bf16_value(b) for b in wbits]
    x_min = min(min(vals), Fraction(0))
    x_max = max(max(vals), Fraction(0))
    span = _f32(x_max - x_min)                  # fp32 subtraction
    s = _bf16(_f32(span / 15))                  # IEEE division, then bf16
    if s == 0:
        return [0] * len(vals), s, 0
    z = max(0, min(15, _round_half_even(-_f32(x_min / s))))
    q = [max(0, min(15, _round_half_even(_f32(v / s)) + z)) for v in vals]
    return q, s, z


def _rand_bf16(rng, shape, lo_exp=-20, hi_exp=5, signs=(0, 1)):
    sign = rng.choice(np.array(signs, dtype=np.uint16), size=shape) << 15
    exp = rng.integers(127 + lo_exp, 127 + hi_exp, size=shape).astype(np.uint16) << 7
    man = rng.integers(0, 128, size=shape).astype(np.uint16)
    return (sign | exp | man).astype(np.uint16)


def _groups(W):
    n, k = W.shape
    for r in range(n):
        for g in range(k // 32):
            yield r, g, W[r, 32 * g:32 * g + 32]


# --------------------------------------------------------------------------
# quantizer
# --------------------------------------------------------------------------

def test_quantize_matches_exact_rationals():
    rng = np.random.default_rng(5)
    W = np.concatenate([
        _rand_bf16(rng, (8, 64)),                             # mixed signs
        _rand_bf16(rng, (4, 64), signs=(0,)),                 # all positive
        _rand_bf16(rng, (4, 64), signs=(1,)),                 # all negative
        _rand_bf16(rng, (4, 64), lo_exp=-60, hi_exp=-40),     # tiny
        _rand_bf16(rng, (4, 64), lo_exp=20, hi_exp=40),       # large
    ])
    W[2, 7] = 0x0000                                          # an exact zero
    W[3, :32] = 0x4040                                        # constant group 3.0
    q, S, Z = quant_asym.quantize_asym(W)
    for r, g, wg in _groups(W):
        want_q, want_s, want_z = _exact_asym_group(wg)
        assert _bf16_value(S[r, g]) == want_s, (r, g)
        assert int(Z[r, g]) == want_z, (r, g)
        assert [int(v) for v in q[r, 32 * g:32 * g + 32]] == want_q, (r, g)


def test_constructed_ties_round_half_even():
    # range [-1, 14] -> s = 1, z = 1: w = 2.5 -> rint 2 -> q = 3; 3.5 -> 4 -> 5
    w = np.zeros((1, 32), np.float32)
    w[0, 0], w[0, 1] = -1.0, 14.0
    w[0, 2], w[0, 3], w[0, 4] = 2.5, 3.5, -0.5
    q, S, Z = quant_asym.quantize_asym(bf16.rne(w))
    assert bf16.to_f32(S)[0, 0] == 1.0 and int(Z[0, 0]) == 1
    assert [int(v) for v in q[0, :5]] == [0, 15, 3, 5, 1]


def test_error_bound_half_scale_when_not_clamped():
    rng = np.random.default_rng(6)
    W = _rand_bf16(rng, (64, 128), lo_exp=-12, hi_exp=2)
    q, S, Z = quant_asym.quantize_asym(W)
    w = bf16.to_f32(W).astype(np.float64).reshape(64, 4, 32)
    s = bf16.to_f32(S).astype(np.float64)[..., None]
    z = Z.astype(np.float64)[..., None]
    x_hat = (q.reshape(64, 4, 32).astype(np.float64) - z) * s
    err = np.abs(w - x_hat)
    # unclamped elements: |x - x_hat| <= s/2 (tutorial's core inequality),
    # up to the fp32 rounding of w / s
    unclamped = (np.rint(w / s) + z >= 0) & (np.rint(w / s) + z <= 15)
    assert np.all(err[unclamped] <= s.repeat(32, -1)[unclamped] * (0.5 + 2.0 ** -20))
    # clamped ones only at the top, by the bf16 rounding of s: < 0.55 s
    assert np.all(err <= 0.55 * s)


def test_zero_is_exactly_on_the_grid():
    rng = np.random.default_rng(7)
    W = _rand_bf16(rng, (32, 64))
    W[:, 3] = 0x0000
    W[:, 40] = 0x8000                      # -0
    q, S, Z = quant_asym.quantize_asym(W)
    d = bf16.to_f32(quant_asym.dequant_asym(q, S, Z))
    assert np.all(d[:, 3] == 0.0) and np.all(d[:, 40] == 0.0)
    assert np.all(q[:, 3] == Z[:, 0]) and np.all(q[:, 40] == Z[:, 1])


def test_minimum_codes_zero_maximum_codes_top():
    rng = np.random.default_rng(8)
    W = _rand_bf16(rng, (64, 32), lo_exp=-8, hi_exp=3)
    q, S, Z = quant_asym.quantize_asym(W)
    w = bf16.to_f32(W)
    for r in range(64):
        i_min, i_max = int(np.argmin(w[r])), int(np.argmax(w[r]))
        if w[r, i_min] < 0:
            assert q[r, i_min] == 0, r
        if w[r, i_max] > 0:
            assert q[r, i_max] >= 14, r


def test_constant_groups():
    for c in (3.0, -0.0078125, 1e-30, 12345.0):
        w = np.full((1, 32), c, np.float32)
        q, S, Z = quant_asym.quantize_asym(bf16.rne(w))
        d = float(bf16.to_f32(quant_asym.dequant_asym(q, S, Z))[0, 0])
        assert abs(d - float(bf16.to_f32(bf16.rne(w))[0, 0])) <= 2.0 ** -7 * abs(c)
        assert (int(Z[0, 0]) == 0) == (c > 0)


def test_all_zero_group():
    q, S, Z = quant_asym.quantize_asym(np.zeros((2, 64), np.uint16))
    assert np.all(q == 0) and np.all(S == 0) and np.all(Z == 0)


def test_integer_grid_is_identity():
    """Integers in [-8, 7] with both ends present: s = 1, z = 8, q = w + 8,
    and the dequantized weights are the integers themselves."""
    rng = np.random.default_rng(9)
    w = rng.integers(-8, 8, size=(16, 128)).astype(np.float32)
    w.reshape(16, 4, 32)[:, :, 0] = -8.0
    w.reshape(16, 4, 32)[:, :, 1] = 7.0
    q, S, Z = quant_asym.quantize_asym(bf16.rne(w))
    assert np.all(bf16.to_f32(S) == 1.0) and np.all(Z == 8)
    assert np.array_equal(q.astype(np.float32), w + 8)
    assert np.array_equal(bf16.to_f32(quant_asym.dequant_asym(q, S, Z)), w)


def test_gemm_integer_case_is_integer_matmul():
    rng = np.random.default_rng(10)
    w = rng.integers(-8, 8, size=(24, 96)).astype(np.float32)
    w.reshape(24, 3, 32)[:, :, 0] = -8.0
    w.reshape(24, 3, 32)[:, :, 31] = 7.0
    x = rng.integers(-3, 4, size=(5, 96)).astype(np.float32)
    Wq, S, Z = quant_asym.quantize_pack_asym(bf16.rne(w))
    y = gemm.w4a16_gemm_asym(bf16.rne(x), Wq, S, Z)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T)


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------

def test_pack_known_word():
    q = np.array([[0, 1, 2, 3, 12, 13, 14, 15]], np.uint8)
    assert int(quant_asym.pack_unsigned(q).view(np.uint32)[0, 0]) == 0xFEDC3210


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(quant_asym.unpack_unsigned(quant_asym.pack_unsigned(q)), q)


def test_fake_quant_equals_dequant_of_packed():
    rng = np.random.default_rng(12)
    W = _rand_bf16(rng, (8, 96))
    Wq, S, Z = quant_asym.quantize_pack_asym(W)
    d = quant_asym.dequant_asym(quant_asym.unpack_unsigned(Wq), S, Z)
    assert np.array_equal(d, quant_asym.fake_quant_asym(W))


def test_rejects_non_finite():
    W = np.zeros((1, 32), np.uint16)
    W[0, 3] = 0x7F80
    with pytest.raises(ValueError):
        quant_asym.quantize_asym(W)
