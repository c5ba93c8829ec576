"""ctypes loader for libw4a16.so (the C ABI declared in include/w4a16.h).

The library is built in-tree by ``python -m int4_weight_only_amd.build``.
Loading fails loudly when it is missing: there is no fallback path.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

# name -> (restype, argtypes); mirrors include/w4a16.h
SIGNATURES = {
    "w4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4_last_hip_error": (ctypes.c_int, []),
    "w4_version": (ctypes.c_char_p, []),
    "w4_quantize_pack": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "w4_fake_quant": (ctypes.c_int, [_p, _i64, _i64, _p, _p]),
    "w4_quantize_pack_asym": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _p]),
    "w4_fake_quant_asym": (ctypes.c_int, [_p, _i64, _i64, _p, _p]),
    "w4a16_gemm": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "w4a16_gemm_asym": (ctypes.c_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "w4_dequant": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p]),
    "w4_dequant_asym": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _p, _p]),
    "w4_pick_block_size": (_i32, [_i64, _i32, _i32]),
    "w4_moe_align_capacity": (_i64, [_i64, _i32, _i32, _i32]),
    "moe_align_block_size": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _p, _p, _p]),
    "w4a16_moe_gemm": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32,
                                      _i64, _i64, _i32, _i32, _p]),
    "w4a16_moe_gemm_swiglu": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32,
                                             _i64, _i64, _i32, _i32, _p]),
    "w4a16_moe_gemm_asym": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32,
                                           _i32, _i64, _i64, _i32, _i32, _p]),
    "w4a16_moe_gemm_swiglu_asym": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32,
                                                  _i32, _i64, _i64, _i32, _i32, _p]),
    "w4_silu_mul": (ctypes.c_int, [_p, _p, _i64, _i64, _p]),
    "w4_moe_sum": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i64, _p]),
    "w4_moe_route": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _p]),
    "w4_moe_combine_workspace_words": (_i64, [_i64, _i32, _i32, _i64, _i32]),
    "w4a16_moe_gemm_combine": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32,
                                              _i32, _i64, _i64, _i32, _i32, _p, _p]),
    "w4a16_moe_gemm_combine_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64,
                                                      _i32, _i32, _i64, _i64, _i32, _i32, _p]),
    "w4_dequant_t": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _p, _p]),
    "w4_bf16_gemm_nt": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "w4_repacked_words": (_i64, [_i64, _i64]),
    "w4_repack": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p]),
    "w4_restore": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p]),
    "w4_bf16_transpose": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p]),
    "w4_repacked_group_elems": (_i64, [_i64, _i64]),
    "w4_repack_groups": (ctypes.c_int, [_p, _i32, _i64, _i64, _i64, _p, _p]),
    "w4_restore_groups": (ctypes.c_int, [_p, _i32, _i64, _i64, _i64, _p, _p]),
    "w4a16_gemm_tiled": (ctypes.c_int, [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "w4a16_moe_gemm_tiled": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32,
                                            _i32, _i64, _i64, _i32, _i32, _p]),
    "w4a16_moe_gemm_swiglu_tiled": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32,
                                                   _i32, _i64, _i64, _i32, _i32, _p]),
}

_lib = None


def load():
    """Load libw4a16.so once and attach the prototypes.  Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m int4_weight_only_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class W4Error(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, fn, status):
        lib = load()
        msg = lib.w4_status_string(status).decode()
        if status == 5:
            msg += f" (hipError {lib.w4_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [status {status}]")
        self.status = status


def check(fn, status):
    if status != 0:
        raise W4Error(fn, status)
