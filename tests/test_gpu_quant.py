"""GPU parity: w4_quantize_pack, w4_fake_quant and w4_dequant against the
oracle.

Bit-exact on every byte: the packed codes, the bf16 scales, the
fake-quantized weights and the dequantized packed codes, on the small dense workload, on the full decode and
prefill weight shapes, on ragged shapes and on hand-built groups that hit
exact rounding ties, zero groups, subnormal magnitudes and extreme values.
"""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import synth
from gpu_util import down, down_bits, say, up, up_bits
from oracle import bf16, quant

pytestmark = pytest.mark.gpu


def check_quantize(Wbits, label):
    say(f"quantize_pack {label} shape={Wbits.shape}")
    Wq_ref, S_ref = quant.quantize_pack(Wbits)
    W = up_bits(Wbits)
    Wq, S = w4.w4_quantize_pack(W)
    np.testing.assert_array_equal(down(Wq), Wq_ref)
    np.testing.assert_array_equal(down_bits(S), S_ref)
    say(f"fake_quant {label}")
    ref = quant.fake_quant(Wbits)
    np.testing.assert_array_equal(down_bits(w4.w4_fake_quant(W)), ref)
    say(f"dequant {label}")
    np.testing.assert_array_equal(down_bits(w4.w4_dequant(Wq, S)), ref)
    # in place
    W2 = W.clone()
    w4.w4_fake_quant(W2, out=W2)
    np.testing.assert_array_equal(down_bits(W2), ref)


def test_dense_small_seed0():
    wl = synth.WORKLOADS["dense_small"]
    check_quantize(synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"])), "512x512")


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (7, 160), (129, 64), (2, 4096), (5, 32 * 37)])
def test_ragged_shapes(N, K):
    check_quantize(synth.bits(synth.weights(N, K, 11 + N + K)), f"{N}x{K}")


def special_groups():
    """Rows of hand-built 32-element groups (bf16 bits), K = 32 * groups."""
    f32 = np.float32
    groups = []
    # s = bf16(7/7) = 1: w/s = w, exact half-way points must round to even
    g = np.array([7, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, -3.5, 4.5, -4.5, 5.5, -5.5, 6.5,
                  -6.5, 0.25, -0.25, 0.75, 1, 2, 3, 4, 5, 6, -1, -2, -3, -4, -5, -6, -7, 0],
                 dtype=f32)
    groups.append(g)
    groups.append(-g)
    groups.append(np.zeros(32, f32))                              # zero group: s = 0
    groups.append(np.full(32, -0.0, f32))
    tiny = np.float32(1e-39) * np.arange(-16, 16, dtype=f32)      # subnormal magnitudes
    groups.append(tiny)
    groups.append(np.full(32, np.float32(9.2e-41)))               # amax/7 underflows bf16
    big = np.linspace(-3.0e38, 3.0e38, 32, dtype=f32)             # near the top of bf16
    groups.append(big)
    one = np.zeros(32, f32)
    one[17] = -0.015625                                           # single nonzero, negative
    groups.append(one)
    rng = np.random.default_rng(5)
    for scale in (1e-30, 1e-3, 1.0, 1e20):
        groups.append((rng.standard_normal(32) * scale).astype(f32))
    row = np.concatenate(groups)
    bits = bf16.rne(row).reshape(1, -1)
    return np.concatenate([bits, bits[:, ::-1].copy()], axis=0)


def test_special_groups():
    check_quantize(special_groups(), "special groups")


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_full_size(name):
    wl = synth.WORKLOADS[name]
    check_quantize(synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"])), name)


def test_empty_is_noop():
    W = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Wq, S = w4.w4_quantize_pack(W)
    assert Wq.numel() == 0 and S.numel() == 0
    assert w4.w4_fake_quant(W).numel() == 0


def fuzz_bits(seed, N, K, max_exp):
    """Random finite bf16 bit patterns (exponent field 0 .. max_exp, so
    subnormals included), the exponent range varying per group, plus groups
    of exact ties: (m + 1/2) * s for a random bf16 scale s."""
    rng = np.random.default_rng(seed)
    G = K // 32
    lo = rng.integers(0, max_exp, size=(N, G, 1))
    width = rng.choice([1, 4, 16, 64, 255], size=(N, G, 1))
    exp = np.clip(lo + rng.integers(0, 256, size=(N, G, 32)) % width, 0, max_exp)
    sign = rng.integers(0, 2, size=(N, G, 32))
    man = rng.integers(0, 128, size=(N, G, 32))
    W = ((sign << 15) | (exp << 7) | man).astype(np.uint16)
    ties = rng.random((N, G)) < 0.1
    s = bf16.to_f32(rng.integers(0x3A00, 0x4200, size=(N, G)).astype(np.uint16))
    m = rng.integers(-7, 7, size=(N, G, 32)).astype(np.float32)
    tie_vals = bf16.rne(((m + 0.5) * s[..., None]).astype(np.float32))
    W = np.where(ties[..., None], tie_vals, W)
    return W.reshape(N, K)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_bit_pattern_fuzz(seed):
    check_quantize(fuzz_bits(seed, 256, 1024, 254), f"fuzz seed {seed}")


def _group_with_scale(s0, rng, ties):
    """32 bf16 weights whose scale bf16(amax / 7) is exactly s0 (a bf16 with
    a mantissa of at most two bits after the point, so amax = 7 s0 and every
    k s0 / 2 below are exact bf16 values): with ``ties`` the others are
    k s0 / 2, |k| <= 13 (w / s0 = k / 2: exact half-integer ties for odd
    k), else random values below amax."""
    a = 7.0 * s0
    if ties:
        v = rng.integers(-13, 14, size=32).astype(np.float64) * (s0 / 2.0)
    else:
        v = rng.uniform(-a, a, size=32)
    v[int(rng.integers(32))] = a if rng.random() < 0.5 else -a
    g = bf16.rne(v.astype(np.float32))
    if ties:
        assert np.all(bf16.to_f32(g).astype(np.float64) == v)
    return g


@pytest.mark.parametrize("ties", [False, True])
def test_scales_at_the_quotient_range_ends(ties):
    """Scales on both sides of the ends of the range where the kernels round
    w / s without a division ([2^-110, 2^100]), and on the ends themselves,
    with and without exact ties: bit-exact against the oracle."""
    rng = np.random.default_rng(77 + ties)
    scales = [f * 2.0 ** e for e in (-111, -110, -109, 99, 100, 101) for f in (1.0, 1.25, 1.5)]
    rows = [np.concatenate([_group_with_scale(s0, rng, ties) for _ in range(8)]) for s0 in scales]
    W = np.stack(rows)
    _, S = quant.quantize_pack(W)
    assert np.array_equal(bf16.to_f32(S)[:, 0].astype(np.float64), np.array(scales))
    check_quantize(W, f"scale range ends ties={ties}")


# -------------------------------------------------------------- dequant --

@pytest.mark.parametrize("N,K", [(1, 32), (7, 160), (129, 64), (300, 4096)])
def test_dequant_matches_oracle_and_fake_quant(N, K):
    """w4_dequant of the packed codes equals the oracle's dequantization of
    the same codes and, bit for bit, the fake quantization of the source."""
    Wb = synth.bits(synth.weights(N, K, 5 + N))
    Wq_r, S_r = quant.quantize_pack(Wb)
    say(f"dequant N={N} K={K}")
    Wq, S = w4.w4_quantize_pack(up_bits(Wb))
    Wd = down_bits(w4.w4_dequant(Wq, S))
    np.testing.assert_array_equal(Wd, quant.dequant(quant.unpack(Wq_r), S_r))
    np.testing.assert_array_equal(Wd, quant.fake_quant(Wb))


def test_dequant_special_groups():
    """Zero groups, subnormal and huge scales, exact ties (the hand-built
    groups of the quantizer tests)."""
    Wb = special_groups()
    Wq_r, S_r = quant.quantize_pack(Wb)
    say("dequant special groups")
    Wd = down_bits(w4.w4_dequant(up(Wq_r), up_bits(S_r)))
    np.testing.assert_array_equal(Wd, quant.dequant(quant.unpack(Wq_r), S_r))
