"""Pins of the oracle's kernel-order code layout (oracle/layout.py).

The layout is this library's convention (the RL write-up's section 4 only
says that the weights are converted to the inference kernel's layout after
loading and restored before the next load), so what is pinned is that the
conversion is a lossless permutation with zero padding, and -- per code
element rather than per 16-byte unit -- that element k of row n lands where
the layout statement puts it.
"""

import numpy as np
import pytest

from oracle import layout, quant

SHAPES = [(1, 1, 32), (1, 31, 64), (1, 32, 96), (3, 33, 128), (2, 100, 4096), (1, 64, 544)]


def random_codes(E, N, K, seed):
    """Packed words with no zero word (so padding is recognisable)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 8, size=(E, N, K)).astype(np.int8)
    q[..., ::8] = rng.integers(1, 8, size=(E, N, K // 8))   # every word has a nonzero nibble
    return np.stack([quant.pack(q[e]) for e in range(E)]), q


@pytest.mark.parametrize("E,N,K", SHAPES)
def test_round_trip_and_size(E, N, K):
    Wq, _ = random_codes(E, N, K, N + K)
    Wt = layout.repack(Wq)
    words = -(-N // 32) * -(-K // 64) * 256
    assert layout.repacked_words(N, K) == words
    assert Wt.shape == (E, words)
    np.testing.assert_array_equal(layout.restore(Wt, N, K), Wq)
    # the padding is zero and nothing else is: every canonical word appears once
    assert np.count_nonzero(Wt) == E * N * (K // 8)
    if N % 32 == 0 and K % 64 == 0:
        assert words * 4 == N * K // 2     # no padding: the same bytes


@pytest.mark.parametrize("E,N,K", SHAPES[:4])
def test_every_code_lands_where_the_layout_says(E, N, K):
    """Code k of row n (any expert e) is nibble k % 8 of word
    256 (r S + c) + 4 (32 h + n % 32) + (k % 32) // 8 of matrix e, with
    r = n // 32, c = k // 64, h = (k % 64) // 32, S = ceil(K / 64)."""
    Wq, q = random_codes(E, N, K, 7 * N + K)
    Wt = layout.repack(Wq).view(np.uint32)
    S = -(-K // 64)
    for e in range(E):
        for n in range(N):
            for k in range(K):
                w = 256 * ((n // 32) * S + k // 64) + 4 * (32 * ((k % 64) // 32) + n % 32) \
                    + (k % 32) // 8
                nib = int(Wt[e, w] >> np.uint32(4 * (k % 8))) & 0xF
                assert (nib - 16 if nib >= 8 else nib) == q[e, n, k], (e, n, k)


GROUP_SHAPES = [(1, 1, 32), (1, 15, 64), (1, 16, 256), (3, 17, 288), (2, 100, 4096), (1, 48, 544)]


@pytest.mark.parametrize("E,N,K", GROUP_SHAPES)
@pytest.mark.parametrize("dtype", [np.uint16, np.uint8])
def test_group_round_trip_and_size(E, N, K, dtype):
    """Per-group values (bf16 scale bits, zero-point bytes): a lossless
    permutation with zero padding."""
    rng = np.random.default_rng(N + K)
    A = rng.integers(1, 200, size=(E, N, K // 32)).astype(dtype)   # no zero value
    At = layout.repack_groups(A, K)
    elems = -(-N // 16) * -(-(K // 32) // 8) * 128
    assert layout.repacked_group_elems(N, K) == elems
    assert At.shape == (E, elems) and At.dtype == A.dtype
    np.testing.assert_array_equal(layout.restore_groups(At, N, K), A)
    assert np.count_nonzero(At) == E * N * (K // 32)


@pytest.mark.parametrize("E,N,K", GROUP_SHAPES[:4])
def test_every_group_value_lands_where_the_layout_says(E, N, K):
    """Group g of row n is element 128 (r C + c) + 8 (n % 16) + g % 8 with
    r = n // 16, c = g // 8, C = ceil(G / 8)."""
    rng = np.random.default_rng(3 * N + K)
    G = K // 32
    A = rng.integers(0, 65535, size=(E, N, G)).astype(np.uint16)
    At = layout.repack_groups(A, K)
    C = -(-G // 8)
    for e in range(E):
        for n in range(N):
            for g in range(G):
                assert At[e, 128 * ((n // 16) * C + g // 8) + 8 * (n % 16) + g % 8] == A[e, n, g]
