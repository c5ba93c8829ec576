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
