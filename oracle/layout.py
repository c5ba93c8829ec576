"""Kernel-order code layout -- oracle.  TEST INFRASTRUCTURE ONLY.

Source: "INT4 QAT end-to-end for RL", §4 inference: after INT4 weights are
loaded, the inference engine converts them into the layout its W4A16
kernel reads (and restores the original layout before the next weight
update loads new values).  The pages give no layout; this library's
kernel order is a convention (parity unpinned as a choice; its round trip
and the equality of products on either layout are checked):

* per [N, K] matrix, ceil(N/32) x ceil(K/64) blocks of 256 int32 words,
  block (r, c) at word 256 (r ceil(K/64) + c);
* word 4u + i of a block (unit u = 0..63, i = 0..3) is word 4 g + i of
  canonical row n, with n = 32 r + u % 32 and g = 2 c + u // 32 the group
  (the canonical row holds its K/32 groups of 4 words each in order);
* units whose row is >= N or whose group is >= K/32 are zero;
* E matrices (experts) are stored one after another.
"""

import numpy as np


def repacked_words(N, K):
    """int32 words of one [N, K] matrix in kernel order."""
    return -(-N // 32) * -(-K // 64) * 256


def _unit_map(N, K):
    """For every unit of the kernel-order buffer: (row n, group g, valid)."""
    nb, nsteps = -(-N // 32), -(-K // 64)
    r = np.repeat(np.arange(nb), nsteps * 64)
    c = np.tile(np.repeat(np.arange(nsteps), 64), nb)
    u = np.tile(np.arange(64), nb * nsteps)
    n = 32 * r + u % 32
    g = 2 * c + u // 32
    return n, g, (n < N) & (g < K // 32)


def repack(Wq):
    """Canonical codes int32 [N, K/8] or [E, N, K/8] -> int32 [E, words]."""
    Wq = np.asarray(Wq, dtype=np.int32)
    if Wq.ndim == 2:
        Wq = Wq[None]
    E, N, kw = Wq.shape
    K = 8 * kw
    n, g, valid = _unit_map(N, K)
    out = np.zeros((E, n.size, 4), dtype=np.int32)
    units = Wq.reshape(E, N, K // 32, 4)           # a group's 4 words
    out[:, valid] = units[:, n[valid], g[valid]]
    return out.reshape(E, -1)


def restore(Wt, N, K):
    """Kernel order int32 [E, words] -> canonical codes int32 [E, N, K/8]."""
    Wt = np.asarray(Wt, dtype=np.int32).reshape(-1, repacked_words(N, K) // 4, 4)
    E = Wt.shape[0]
    n, g, valid = _unit_map(N, K)
    out = np.zeros((E, N, K // 32, 4), dtype=np.int32)
    out[:, n[valid], g[valid]] = Wt[:, valid]
    return out.reshape(E, N, K // 8)
