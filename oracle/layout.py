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

Per-group values (bf16 scales, uint8 zero points, [N, K/32] canonical)
have a kernel order of their own, read by the same products:

* per matrix, ceil(N/16) x ceil(G/8) blocks of 128 elements (G = K/32),
  block (r, c) at element 128 (r ceil(G/8) + c);
* element 8 i + j of a block is the value of row 16 r + i, group 8 c + j
  (16 rows x 8 groups, row-major);
* elements whose row is >= N or whose group is >= G are zero.
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


def repacked_group_elems(N, K):
    """Elements of one [N, K/32] per-group array in kernel order."""
    return -(-N // 16) * -(-(K // 32) // 8) * 128


def _group_map(N, K):
    """For every element of the kernel-order buffer: (row n, group g, valid)."""
    G = K // 32
    gb = -(-G // 8)
    idx = np.arange(repacked_group_elems(N, K))
    b, w = idx // 128, idx % 128
    n = 16 * (b // gb) + w // 8
    g = 8 * (b % gb) + w % 8
    return n, g, (n < N) & (g < G)


def repack_groups(A, K):
    """Per-group values [N, K/32] or [E, N, K/32] -> [E, elements]."""
    A = np.asarray(A)
    if A.ndim == 2:
        A = A[None]
    E, N, G = A.shape
    assert G == K // 32
    n, g, valid = _group_map(N, K)
    out = np.zeros((E, n.size), dtype=A.dtype)
    out[:, valid] = A[:, n[valid], g[valid]]
    return out


def restore_groups(At, N, K):
    """Kernel order [E, elements] -> per-group values [E, N, K/32]."""
    At = np.asarray(At).reshape(-1, repacked_group_elems(N, K))
    n, g, valid = _group_map(N, K)
    out = np.zeros((At.shape[0], N, K // 32), dtype=At.dtype)
    out[:, n[valid], g[valid]] = At[:, valid]
    return out
