"""The C ABI without a GPU: exported symbols, host-side helpers, and every
argument check that returns before anything is enqueued.

None of these calls reaches the HIP runtime: each one fails validation, or
is a pure host function, so they run on a CPU-only machine as long as the
library loads.
"""

import ctypes
import os
import re

import pytest

from oracle import moe as omoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

# fake, never-dereferenced device addresses
A16 = ctypes.c_void_p(0x10000)        # 16-byte aligned
A4 = ctypes.c_void_p(0x10004)         # 4-byte aligned only
A2 = ctypes.c_void_p(0x10002)         # 2-byte aligned only
A1 = ctypes.c_void_p(0x10001)

OK, NULL, SHAPE, MISALIGNED, UNSUPPORTED = 0, 1, 2, 3, 4


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"#[^\n]*", "", text)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}]*\)\s*;", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from int4_weight_only_amd import _lib
    return _lib.load()


def test_header_declares_the_boundary():
    names = header_functions()
    for must in ("w4_quantize_pack", "w4_fake_quant", "w4a16_gemm", "moe_align_block_size",
                 "w4a16_moe_gemm"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    from int4_weight_only_amd import _lib
    names = header_functions()
    assert sorted(_lib.SIGNATURES) == names
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_binding_names_match_the_abi():
    import int4_weight_only_amd as w
    for n in header_functions():
        if n in ("w4_status_string", "w4_last_hip_error", "w4_version"):
            continue
        assert callable(getattr(w, n)), n


def test_status_strings(lib):
    assert lib.w4_status_string(0) == b"ok"
    for s in range(1, 6):
        assert lib.w4_status_string(s) not in (b"ok", b"unknown status")
    assert lib.w4_status_string(99) == b"unknown status"
    assert lib.w4_last_hip_error() == 0
    assert lib.w4_version().startswith(b"w4a16")


def test_missing_library_fails_loudly(monkeypatch):
    from int4_weight_only_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libw4a16.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


# ---------------------------------------------------------------- helpers --

@pytest.mark.parametrize("T,k,E", [(256, 8, 128), (4096, 8, 384), (1, 1, 1), (0, 8, 16),
                                   (7, 3, 5), (100000, 8, 64), (3, 2, 1000)])
def test_pick_block_size_matches_rule(lib, T, k, E):
    assert lib.w4_pick_block_size(T, k, E) == omoe.pick_block_size(T, k, E)


def test_pick_block_size_bad_args(lib):
    assert lib.w4_pick_block_size(-1, 8, 16) == 0
    assert lib.w4_pick_block_size(4, 0, 16) == 0
    assert lib.w4_pick_block_size(4, 8, 0) == 0


@pytest.mark.parametrize("T,k,E,B", [(256, 8, 128, 16), (4096, 8, 384, 64), (0, 1, 1, 1),
                                     (5, 3, 7, 1), (3, 2, 1024, 1024), (1, 8, 3, 5)])
def test_capacity_matches_oracle(lib, T, k, E, B):
    assert lib.w4_moe_align_capacity(T, k, E, B) == omoe.capacity(T, k, E, B)


def test_capacity_bad_args(lib):
    assert lib.w4_moe_align_capacity(-1, 1, 1, 1) == -1
    assert lib.w4_moe_align_capacity(1, 0, 1, 1) == -1
    assert lib.w4_moe_align_capacity(1, 1, 0, 1) == -1
    assert lib.w4_moe_align_capacity(1, 1, 1, 0) == -1


# ---------------------------------------------------- validation, no launch --

def test_quantize_pack_validation(lib):
    f = lib.w4_quantize_pack
    assert f(A16, 4, 33, A16, A2, None) == SHAPE
    assert f(A16, -1, 32, A16, A2, None) == SHAPE
    assert f(None, 0, 32, None, None, None) == OK            # empty: no-op
    assert f(A16, 4, 0, A16, A2, None) == OK
    assert f(None, 4, 32, A16, A2, None) == NULL
    assert f(A16, 4, 32, None, A2, None) == NULL
    assert f(A16, 4, 32, A16, None, None) == NULL
    assert f(A4, 4, 32, A16, A2, None) == MISALIGNED
    assert f(A16, 4, 32, A4, A2, None) == MISALIGNED
    assert f(A16, 4, 32, A16, A1, None) == MISALIGNED
    # one thread per packed word: the grid stays within 2^31 - 1 workgroups
    assert f(A16, 3 << 29, 2048, A16, A2, None) == UNSUPPORTED     # 2^38 + 2^37 words
    assert lib.w4_fake_quant(A16, 3 << 29, 2048, A16, None) == UNSUPPORTED


def test_quantize_pack_asym_validation(lib):
    f = lib.w4_quantize_pack_asym
    assert f(A16, 4, 33, A16, A2, A1, None) == SHAPE
    assert f(None, 0, 32, None, None, None, None) == OK      # empty: no-op
    assert f(A16, 4, 32, A16, A2, None, None) == NULL
    assert f(A16, 4, 32, None, A2, A1, None) == NULL
    assert f(A4, 4, 32, A16, A2, A1, None) == MISALIGNED
    assert f(A16, 4, 32, A16, A1, A1, None) == MISALIGNED


def test_fake_quant_asym_validation(lib):
    f = lib.w4_fake_quant_asym
    assert f(A16, 4, 48, A16, None) == SHAPE
    assert f(None, 4, 32, A16, None) == NULL
    assert f(A4, 4, 32, ctypes.c_void_p(0x20000), None) == MISALIGNED
    assert f(ctypes.c_void_p(0x10000), 4, 32, ctypes.c_void_p(0x10010), None) == UNSUPPORTED


def test_fake_quant_validation(lib):
    f = lib.w4_fake_quant
    assert f(A16, 4, 48, A16, None) == SHAPE
    assert f(None, 4, 32, A16, None) == NULL
    assert f(A16, 4, 32, None, None) == NULL
    assert f(A4, 4, 32, ctypes.c_void_p(0x20000), None) == MISALIGNED
    # partial overlap is refused, exact aliasing is allowed (not launched here)
    assert f(ctypes.c_void_p(0x10000), 4, 32, ctypes.c_void_p(0x10010), None) == UNSUPPORTED


def test_gemm_validation(lib):
    f = lib.w4a16_gemm
    assert f(A16, A16, A2, A4, 4, 8, 40, None) == SHAPE
    assert f(A16, A16, A2, A4, -1, 8, 32, None) == SHAPE
    assert f(None, None, None, None, 0, 8, 32, None) == OK    # M == 0
    assert f(None, None, None, None, 4, 0, 32, None) == OK    # N == 0
    assert f(None, A16, A2, A4, 4, 8, 32, None) == NULL
    assert f(A16, None, A2, A4, 4, 8, 32, None) == NULL
    assert f(A16, A16, None, A4, 4, 8, 32, None) == NULL
    assert f(A16, A16, A2, None, 4, 8, 32, None) == NULL
    assert f(A4, A16, A2, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A4, A2, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A16, A2, A2, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A16, A2, A4, 1 << 40, 8, 32, None) == UNSUPPORTED
    # the tiled kernel's 32-bit buffer offsets: X and Wq below 2 GiB each
    assert f(A16, A16, A2, A4, 64, 8, 1 << 24, None) == UNSUPPORTED      # X = 2 GiB
    assert f(A16, A16, A2, A4, 33, 8, 1 << 25, None) == UNSUPPORTED      # K above decode
    assert f(A16, A16, A2, A4, 64, 1 << 20, 4096, None) == UNSUPPORTED   # Wq = 2 GiB


def test_gemm_asym_validation(lib):
    f = lib.w4a16_gemm_asym
    assert f(A16, A16, A2, A1, A4, 4, 8, 40, None) == SHAPE
    assert f(A16, A16, A2, A1, A4, 4, -1, 32, None) == SHAPE
    assert f(None, None, None, None, None, 0, 8, 32, None) == OK    # M == 0
    assert f(None, None, None, None, None, 4, 0, 32, None) == OK    # N == 0
    assert f(None, A16, A2, A1, A4, 4, 8, 32, None) == NULL
    assert f(A16, None, A2, A1, A4, 4, 8, 32, None) == NULL
    assert f(A16, A16, None, A1, A4, 4, 8, 32, None) == NULL
    assert f(A16, A16, A2, None, A4, 4, 8, 32, None) == NULL        # Z
    assert f(A16, A16, A2, A1, None, 4, 8, 32, None) == NULL
    assert f(A4, A16, A2, A1, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A4, A2, A1, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A16, A1, A1, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A16, A2, A1, A2, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A16, A2, A1, A4, 1 << 40, 8, 32, None) == UNSUPPORTED
    assert f(A16, A16, A2, A1, A4, 64, 8, 1 << 24, None) == UNSUPPORTED
    assert f(A16, A16, A2, A1, A4, 64, 1 << 20, 4096, None) == UNSUPPORTED


def test_align_validation(lib):
    f = lib.moe_align_block_size
    assert f(A4, 4, 0, 8, 16, A4, A4, A4, None) == SHAPE
    assert f(A4, 4, 2, 0, 16, A4, A4, A4, None) == SHAPE
    assert f(A4, 4, 2, 8, 0, A4, A4, A4, None) == SHAPE
    assert f(A4, -1, 2, 8, 16, A4, A4, A4, None) == SHAPE
    assert f(A4, 4, 2, 1025, 16, A4, A4, A4, None) == UNSUPPORTED
    assert f(A4, 4, 2, 8, 1025, A4, A4, A4, None) == UNSUPPORTED
    assert f(A4, 1 << 30, 8, 8, 16, A4, A4, A4, None) == UNSUPPORTED
    assert f(None, 4, 2, 8, 16, A4, A4, A4, None) == NULL
    assert f(A4, 4, 2, 8, 16, None, A4, A4, None) == NULL
    assert f(A4, 4, 2, 8, 16, A4, None, A4, None) == NULL
    assert f(A4, 4, 2, 8, 16, A4, A4, None, None) == NULL
    assert f(A2, 4, 2, 8, 16, A4, A4, A4, None) == MISALIGNED
    assert f(A4, 4, 2, 8, 16, A2, A4, A4, None) == MISALIGNED


def test_moe_gemm_validation(lib):
    f = lib.w4a16_moe_gemm
    good = [A16, A16, A2, A4, A4, A4, None, A4]
    assert f(*good, 4, 2, 8, 64, 48, 16, 1, None) == SHAPE        # K % 32
    assert f(*good, 4, 2, 8, 64, 64, 16, 3, None) == SHAPE        # x_row_div
    assert f(*good, 4, 2, 8, 0, 64, 16, 1, None) == SHAPE         # N
    assert f(*good, 4, 0, 8, 64, 64, 16, 1, None) == SHAPE        # k
    assert f(*good, 4, 2, 8, 64, 64, 0, 1, None) == SHAPE         # B
    assert f(*good, 4, 2, 2000, 64, 64, 16, 1, None) == UNSUPPORTED
    # X = 2^19 pair rows x 2048 = 2 GiB, within the grid's slot limit
    assert f(*good, 1 << 16, 8, 8, 64, 2048, 1024, 1, None) == UNSUPPORTED
    assert f(*good, 4, 2, 8, 1 << 20, 4096, 16, 1, None) == UNSUPPORTED   # an expert = 2 GiB
    assert f(*good, 0, 2, 8, 64, 64, 16, 1, None) == OK           # T == 0: no-op
    bad_null = list(good)
    bad_null[3] = None
    assert f(*bad_null, 4, 2, 8, 64, 64, 16, 1, None) == NULL
    bad_al = list(good)
    bad_al[0] = A4
    assert f(*bad_al, 4, 2, 8, 64, 64, 16, 1, None) == MISALIGNED
    bad_tw = list(good)
    bad_tw[6] = A2
    assert f(*bad_tw, 4, 2, 8, 64, 64, 16, 1, None) == MISALIGNED


def test_moe_gemm_swiglu_validation(lib):
    f = lib.w4a16_moe_gemm_swiglu
    good = [A16, A16, A2, A4, A4, A4, A4]
    assert f(*good, 4, 2, 8, 32, 48, 16, 1, None) == SHAPE        # K % 32
    assert f(*good, 4, 2, 8, 32, 64, 16, 3, None) == SHAPE        # x_row_div
    assert f(*good, 4, 2, 8, 0, 64, 16, 1, None) == SHAPE         # I
    assert f(*good, 4, 2, 8, 32, 64, 0, 1, None) == SHAPE         # B
    assert f(*good, 4, 2, 2000, 32, 64, 16, 1, None) == UNSUPPORTED
    assert f(*good, 1 << 16, 8, 8, 32, 2048, 1024, 1, None) == UNSUPPORTED  # X = 2 GiB
    assert f(*good, 4, 2, 8, 1 << 19, 4096, 16, 1, None) == UNSUPPORTED   # 2I rows = 2 GiB
    assert f(*good, 0, 2, 8, 32, 64, 16, 1, None) == OK           # T == 0: no-op
    bad_null = list(good)
    bad_null[6] = None
    assert f(*bad_null, 4, 2, 8, 32, 64, 16, 1, None) == NULL
    bad_al = list(good)
    bad_al[6] = A2
    assert f(*bad_al, 4, 2, 8, 32, 64, 16, 1, None) == MISALIGNED


def test_moe_gemm_asym_validation(lib):
    f = lib.w4a16_moe_gemm_asym
    good = [A16, A16, A2, A1, A4, A4, A4, None, A4]           # Z: any alignment
    assert f(*good, 4, 2, 8, 64, 48, 16, 1, None) == SHAPE        # K % 32
    assert f(*good, 4, 2, 8, 64, 64, 16, 3, None) == SHAPE        # x_row_div
    assert f(*good, 4, 2, 2000, 64, 64, 16, 1, None) == UNSUPPORTED
    assert f(*good, 4, 2, 8, 1 << 20, 4096, 16, 1, None) == UNSUPPORTED   # an expert = 2 GiB
    assert f(*good, 0, 2, 8, 64, 64, 16, 1, None) == OK           # T == 0: no-op
    no_z = list(good)
    no_z[3] = None
    assert f(*no_z, 4, 2, 8, 64, 64, 16, 1, None) == NULL
    bad_al = list(good)
    bad_al[1] = A4
    assert f(*bad_al, 4, 2, 8, 64, 64, 16, 1, None) == MISALIGNED


def test_moe_gemm_swiglu_asym_validation(lib):
    f = lib.w4a16_moe_gemm_swiglu_asym
    good = [A16, A16, A2, A1, A4, A4, A4, A4]
    assert f(*good, 4, 2, 8, 32, 48, 16, 1, None) == SHAPE        # K % 32
    assert f(*good, 4, 2, 8, 0, 64, 16, 1, None) == SHAPE         # I
    assert f(*good, 4, 2, 8, 1 << 19, 4096, 16, 1, None) == UNSUPPORTED   # 2I rows = 2 GiB
    assert f(*good, 4, 2, 8, 1 << 40, 64, 16, 1, None) == UNSUPPORTED     # 2I past int32
    assert f(*good, 0, 2, 8, 32, 64, 16, 1, None) == OK           # T == 0: no-op
    no_z = list(good)
    no_z[3] = None
    assert f(*no_z, 4, 2, 8, 32, 64, 16, 1, None) == NULL
    bad_al = list(good)
    bad_al[7] = A2
    assert f(*bad_al, 4, 2, 8, 32, 64, 16, 1, None) == MISALIGNED


def test_elementwise_validation(lib):
    assert lib.w4_silu_mul(A4, A4, 4, 3, None) == SHAPE
    assert lib.w4_silu_mul(None, A4, 4, 4, None) == NULL
    assert lib.w4_silu_mul(A2, A4, 4, 4, None) == MISALIGNED
    assert lib.w4_silu_mul(None, None, 0, 4, None) == OK
    assert lib.w4_moe_sum(A4, None, A4, 4, 2, 3, None) == SHAPE
    assert lib.w4_moe_sum(A4, None, A4, 4, 0, 4, None) == SHAPE
    assert lib.w4_moe_sum(None, None, A4, 4, 2, 4, None) == NULL
    assert lib.w4_moe_sum(A4, A2, A4, 4, 2, 4, None) == MISALIGNED
    assert lib.w4_moe_route(A4, 4, 8, 9, A4, A4, None) == UNSUPPORTED
    assert lib.w4_moe_route(A4, 4, 2000, 8, A4, A4, None) == UNSUPPORTED
    assert lib.w4_moe_route(A4, 4, 64, 17, A4, A4, None) == UNSUPPORTED
    assert lib.w4_moe_route(None, 4, 64, 8, A4, A4, None) == NULL
    assert lib.w4_moe_route(A2, 4, 64, 8, A4, A4, None) == MISALIGNED
    assert lib.w4_moe_route(None, 0, 64, 8, None, None, None) == OK


def test_moe_combine_validation(lib):
    """The fused down + combine call checks the grouped product's arguments
    and its own (top-k ids and weights, output, workspace) before anything
    is enqueued; the workspace size is one counter per token and tile."""
    f = lib.w4a16_moe_gemm_combine
    ops = (A16, A16, A2, A4, A4, A4)                 # A, Wq, S, sorted, expert_ids, ntpp
    tail = (A4, A4, A4, A2)                          # topk_ids, topk_weights, H2, Out
    assert f(*ops, *tail, -1, 2, 8, 64, 64, 16, 0, A4, None) == SHAPE
    assert f(*ops, *tail, 4, 2, 8, 64, 48, 16, 0, A4, None) == SHAPE        # K % 32
    assert f(*ops, *tail, 4, 2, 2000, 64, 64, 16, 0, A4, None) == UNSUPPORTED
    assert f(*ops, *tail, 4, 17, 64, 64, 64, 16, 0, A4, None) == UNSUPPORTED   # k > 16
    assert f(*ops, None, A4, A4, A2, 4, 2, 8, 64, 64, 16, 0, A4, None) == NULL
    assert f(*ops, A4, None, A4, A2, 4, 2, 8, 64, 64, 16, 0, A4, None) == NULL
    assert f(*ops, A4, A4, A4, None, 4, 2, 8, 64, 64, 16, 0, A4, None) == NULL
    assert f(*ops, *tail, 4, 2, 8, 64, 64, 16, 0, None, None) == NULL
    assert f(*ops, A2, A4, A4, A2, 4, 2, 8, 64, 64, 16, 0, A4, None) == MISALIGNED
    assert f(*ops, *tail, 4, 2, 8, 64, 64, 16, 0, A2, None) == MISALIGNED
    assert f(A4, *ops[1:], *tail, 4, 2, 8, 64, 64, 16, 0, A4, None) == MISALIGNED
    assert f(None, None, None, None, None, None, None, None, None, None, 0, 2, 8, 64, 64, 16, 0,
             None, None) == OK
    g = lib.w4a16_moe_gemm_combine_noalloc
    assert g(*ops, *tail, -1, 2, 8, 64, 64, 16, 0, None) == SHAPE
    assert g(*ops, None, A4, A4, A2, 4, 2, 8, 64, 64, 16, 0, None) == NULL
    assert g(*ops, *tail, 4, 17, 64, 64, 64, 16, 0, None) == UNSUPPORTED
    # more counters than the library's fixed array holds (70000 x 16 > 2^18)
    assert g(*ops, *tail, 70000, 1, 8, 4096, 64, 16, 0, None) == UNSUPPORTED
    assert g(None, None, None, None, None, None, None, None, None, None, 0, 2, 8, 64, 64, 16, 0,
             None) == OK
    w = lib.w4_moe_combine_workspace_words
    assert w(256, 8, 128, 4096, 16) == 256 * (4096 // 128)      # 32-row tile: 128 columns
    assert w(4096, 8, 384, 7168, 64) == 4096 * (7168 // 256)    # 128-row tile: 256 columns
    assert w(10, 2, 4, 300, 64) == 10 * 2
    assert w(-1, 2, 4, 300, 64) == -1 and w(1, 0, 4, 300, 64) == -1


def test_qat_op_refuses_cpu_tensors():
    """The QAT op has no CPU path: a CPU weight is rejected before any call."""
    import torch
    from int4_weight_only_amd.qat import fake_quant_ste
    W = torch.zeros((4, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fake_quant_ste(W)


def test_dequant_validation(lib):
    assert lib.w4_dequant(A4, A2, 4, 48, A16, None) == SHAPE
    assert lib.w4_dequant(A4, A2, -1, 32, A16, None) == SHAPE
    assert lib.w4_dequant(A4, A2, 0, 32, A16, None) == OK
    assert lib.w4_dequant(None, A2, 4, 32, A16, None) == NULL
    assert lib.w4_dequant(A4, A2, 4, 32, A4, None) == MISALIGNED
    assert lib.w4_dequant(A2, A2, 4, 32, A16, None) == MISALIGNED
    assert lib.w4_dequant(A4, A2, (1 << 32) + 1, 512, A16, None) == UNSUPPORTED   # > 2^38 words
    assert lib.w4_dequant_asym(A4, A2, None, 4, 32, A16, None) == NULL
    assert lib.w4_dequant_asym(A4, A2, A1, 4, 40, A16, None) == SHAPE


# ------------------------------------------------------ kernel-order codes --

@pytest.mark.parametrize("N,K", [(1, 32), (32, 64), (33, 96), (12288, 4096), (14336, 4096),
                                 (3072, 4096), (4096, 1536), (100, 0)])
def test_repacked_words_matches_oracle(lib, N, K):
    from oracle import layout
    assert lib.w4_repacked_words(N, K) == layout.repacked_words(N, K)


def test_repacked_words_bad_args(lib):
    assert lib.w4_repacked_words(-1, 32) == -1
    assert lib.w4_repacked_words(4, 33) == -1
    assert lib.w4_repacked_words(4, -32) == -1


D16 = ctypes.c_void_p(0x100000)       # a second buffer far from A16 (16-byte aligned)
D4 = ctypes.c_void_p(0x100004)


def test_repack_restore_validation(lib):
    for f in (lib.w4_repack, lib.w4_restore):
        assert f(A16, 1, 4, 33, D16, None) == SHAPE
        assert f(A16, -1, 4, 32, D16, None) == SHAPE
        assert f(None, 0, 4, 32, None, None) == OK             # empty: no-op
        assert f(None, 1, 4, 32, D16, None) == NULL
        assert f(A16, 1, 4, 32, None, None) == NULL
        assert f(A4, 1, 4, 32, D16, None) == MISALIGNED
        assert f(A16, 1, 4, 32, D4, None) == MISALIGNED
        assert f(A16, 1, 4, 32, A16, None) == UNSUPPORTED      # overlapping buffers


@pytest.mark.parametrize("N,K", [(1, 32), (16, 256), (17, 288), (12288, 4096), (45, 96),
                                 (3072, 2048), (100, 0)])
def test_repacked_group_elems_matches_oracle(lib, N, K):
    from oracle import layout
    assert lib.w4_repacked_group_elems(N, K) == layout.repacked_group_elems(N, K)


def test_repacked_group_elems_bad_args(lib):
    assert lib.w4_repacked_group_elems(-1, 32) == -1
    assert lib.w4_repacked_group_elems(4, 33) == -1
    assert lib.w4_repacked_group_elems(4, -32) == -1


def test_repack_restore_groups_validation(lib):
    for f in (lib.w4_repack_groups, lib.w4_restore_groups):
        assert f(A16, 2, 1, 4, 33, D16, None) == SHAPE
        assert f(A16, 2, -1, 4, 32, D16, None) == SHAPE
        assert f(A16, 4, 1, 4, 32, D16, None) == UNSUPPORTED    # 1- or 2-byte values only
        assert f(A16, 0, 1, 4, 32, D16, None) == UNSUPPORTED
        assert f(None, 2, 0, 4, 32, None, None) == OK           # empty: no-op
        assert f(None, 2, 1, 4, 32, D16, None) == NULL
        assert f(A16, 1, 1, 4, 32, None, None) == NULL
        assert f(A1, 2, 1, 4, 32, D16, None) == MISALIGNED
        assert f(A16, 2, 1, 4, 32, A1, None) == MISALIGNED
        assert f(A16, 2, 1, 4, 32, A16, None) == UNSUPPORTED    # overlapping buffers


def test_bf16_transpose_validation(lib):
    f = lib.w4_bf16_transpose
    assert f(A16, -1, 8, 8, D16, None) == SHAPE
    assert f(A16, 8, -1, 8, D16, None) == SHAPE
    assert f(A16, 8, 8, 7, D16, None) == SHAPE          # padded rows below the rows
    assert f(None, 8, 0, 8, None, None) == OK           # no columns: no-op
    assert f(None, 0, 8, 0, None, None) == OK           # no rows at all: no-op
    assert f(None, 8, 8, 8, D16, None) == NULL
    assert f(A16, 8, 8, 8, None, None) == NULL
    assert f(A1, 8, 8, 8, D16, None) == MISALIGNED
    assert f(A16, 8, 8, 8, A16, None) == UNSUPPORTED    # overlapping buffers


def test_gemm_tiled_validation(lib):
    f = lib.w4a16_gemm_tiled
    assert f(A16, A16, A2, None, A4, 4, 8, 33, None) == SHAPE
    assert f(A16, A16, A2, None, A4, -1, 8, 32, None) == SHAPE
    assert f(None, None, None, None, None, 0, 8, 32, None) == OK    # M == 0: no-op
    assert f(None, A16, A2, None, A4, 4, 8, 32, None) == NULL
    assert f(A16, None, A2, None, A4, 4, 8, 32, None) == NULL
    assert f(A16, A16, A2, None, None, 4, 8, 32, None) == NULL
    assert f(A4, A16, A2, None, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A4, A2, None, A4, 4, 8, 32, None) == MISALIGNED
    assert f(A16, A16, A2, None, A2, 4, 8, 32, None) == MISALIGNED
    # tiled product: the kernel-order weights must fit one 32-bit buffer
    assert f(A16, A16, A2, None, A4, 64, 1 << 20, 8192, None) == UNSUPPORTED


def test_moe_gemm_tiled_validation(lib):
    f = lib.w4a16_moe_gemm_tiled
    args = lambda **kw: dict(dict(X=A16, W=A16, S=A2, Z=None, s=A4, e=A4, n=A4, tw=None, Y=A4,
                                  T=4, k=2, E=3, N=64, K=64, B=16, div=2), **kw)
    call = lambda a: f(a["X"], a["W"], a["S"], a["Z"], a["s"], a["e"], a["n"], a["tw"], a["Y"],
                       a["T"], a["k"], a["E"], a["N"], a["K"], a["B"], a["div"], None)
    assert call(args(K=48)) == SHAPE
    assert call(args(div=3)) == SHAPE
    assert call(args(T=0)) == OK
    assert call(args(W=None)) == NULL
    assert call(args(W=A4)) == MISALIGNED
    g = lib.w4a16_moe_gemm_swiglu_tiled
    assert g(A16, A16, A2, None, A4, A4, A4, A4, 4, 2, 3, 0, 64, 16, 2, None) == SHAPE
    assert g(A16, None, A2, None, A4, A4, A4, A4, 4, 2, 3, 32, 64, 16, 2, None) == NULL
