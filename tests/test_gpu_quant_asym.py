"""GPU parity: w4_quantize_pack_asym and w4_fake_quant_asym against the
asymmetric oracle, bit-exact on every byte (codes, bf16 scales, zero
points, fake-quantized weights) on seeded weights, ragged shapes, the full
decode and prefill weight shapes, and hand-built groups (exact ties, zero
and negative-zero groups, constant groups, one-sided groups, subnormal and
very large magnitudes)."""

import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import synth
from gpu_util import down, down_bits, say, up_bits
from oracle import bf16, quant_asym

pytestmark = pytest.mark.gpu


def check(Wbits, label):
    say(f"quantize_pack_asym {label} shape={Wbits.shape}")
    Wq_ref, S_ref, Z_ref = quant_asym.quantize_pack_asym(Wbits)
    W = up_bits(Wbits)
    Wq, S, Z = w4.w4_quantize_pack_asym(W)
    np.testing.assert_array_equal(down(Wq), Wq_ref)
    np.testing.assert_array_equal(down_bits(S), S_ref)
    np.testing.assert_array_equal(down(Z), Z_ref)
    say(f"fake_quant_asym {label}")
    ref = quant_asym.fake_quant_asym(Wbits)
    np.testing.assert_array_equal(down_bits(w4.w4_fake_quant_asym(W)), ref)
    say(f"dequant_asym {label}")
    np.testing.assert_array_equal(down_bits(w4.w4_dequant_asym(Wq, S, Z)), ref)
    W2 = W.clone()
    w4.w4_fake_quant_asym(W2, out=W2)
    np.testing.assert_array_equal(down_bits(W2), ref)


def test_dense_small_seed0():
    wl = synth.WORKLOADS["dense_small"]
    check(synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"])), "512x512")


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (7, 160), (129, 64), (2, 4096), (5, 32 * 37)])
def test_ragged_shapes(N, K):
    check(synth.bits(synth.weights(N, K, 31 + N + K)), f"{N}x{K}")


def special_groups():
    f32 = np.float32
    groups = []
    # range [-1, 14]: s = 1, z = 1, exact half-way points round to even
    g = np.array([-1, 14, -0.5, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, 7.5, 8.5, 9.5, 10.5, 11.5,
                  12.5, 13.5, -0.25, 0.25, 0.75, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 0], dtype=f32)
    groups.append(g)
    groups.append(-g)
    groups.append(np.zeros(32, f32))                              # s = 0, z = 0
    groups.append(np.full(32, -0.0, f32))
    groups.append(np.full(32, 3.0, f32))                          # constant, positive
    groups.append(np.full(32, -0.375, f32))                       # constant, negative
    groups.append(np.abs(np.linspace(0.1, 2.0, 32, dtype=f32)))   # one-sided positive
    groups.append(-np.abs(np.linspace(0.1, 2.0, 32, dtype=f32)))  # one-sided negative
    groups.append(np.float32(1e-39) * np.arange(-16, 16, dtype=f32))   # subnormals
    groups.append(np.full(32, np.float32(9.2e-41)))               # range/15 underflows bf16
    groups.append(np.linspace(-1.0e38, 1.0e38, 32, dtype=f32))    # large, range finite
    rng = np.random.default_rng(15)
    for scale in (1e-30, 1e-3, 1.0, 1e20):
        groups.append((rng.standard_normal(32) * scale).astype(f32))
        groups.append((np.abs(rng.standard_normal(32)) * scale + scale).astype(f32))
    row = np.concatenate(groups)
    bits = bf16.rne(row).reshape(1, -1)
    return np.concatenate([bits, bits[:, ::-1].copy()], axis=0)


def test_special_groups():
    check(special_groups(), "special groups")


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_full_size(name):
    wl = synth.WORKLOADS[name]
    check(synth.bits(synth.weights(wl["N"], wl["K"], wl["seed"])), name)


def test_empty_is_noop():
    W = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Wq, S, Z = w4.w4_quantize_pack_asym(W)
    assert Wq.numel() == 0 and S.numel() == 0 and Z.numel() == 0
    assert w4.w4_fake_quant_asym(W).numel() == 0


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
    check(fuzz_bits(seed, 256, 1024, 251), f"fuzz seed {seed}")
