"""INT4 weight-only quantization and W4A16 GEMMs on MI355X (gfx950).

Thin Python binding over the C ABI of ``libw4a16.so`` (include/w4a16.h).
Each function has the name of the C entry point it calls and does argument
marshalling only: shape/dtype/device checks, output allocation through
PyTorch, raw pointers and the current HIP stream.  Every step of the path
runs in the library's HIP kernels; nothing here computes.

Layouts (all row-major, contiguous, on one GPU):
  W       bf16  [N, K]        source / master weights
  Wq      int32 [N, K/8]      nibble j of word w holds the INT4 code of k = 8w + j
  S       bf16  [N, K/32]     one scale per 32 consecutive k
  X       bf16  [M, K]        activations;  Y bf16 [M, N]
  Z       uint8 [N, K/32]     zero points (the asymmetric variants)
  experts stacked on a leading axis: Wq [E, N, K/8], S [E, N, K/32], Z [E, N, K/32]
  Wt      int32 [E, w4_repacked_words(N, K)]  codes in the kernel-order layout
          (w4_repack / w4_restore)
  St, Zt  bf16 / uint8 [E, w4_repacked_group_elems(N, K)]  scales and zero
          points in kernel order (w4_repack_groups / w4_restore_groups);
          the *_tiled products read Wt, St and Zt and take N explicitly
"""

import torch

from . import _lib

__all__ = [
    "w4_quantize_pack", "w4_fake_quant", "w4_quantize_pack_asym", "w4_fake_quant_asym",
    "w4_dequant", "w4_dequant_asym", "w4_dequant_t", "w4_bf16_gemm_nt", "w4_bf16_transpose",
    "w4a16_gemm", "w4a16_gemm_asym", "w4_pick_block_size",
    "w4_moe_align_capacity", "moe_align_block_size", "w4a16_moe_gemm", "w4a16_moe_gemm_swiglu",
    "w4a16_moe_gemm_asym", "w4a16_moe_gemm_swiglu_asym",
    "w4_silu_mul", "w4_moe_sum", "w4_moe_route", "w4_moe_combine_workspace_words",
    "w4a16_moe_gemm_combine", "w4a16_moe_gemm_combine_noalloc", "library_path",
    "w4_repacked_words", "w4_repack", "w4_restore", "w4_repacked_group_elems",
    "w4_repack_groups", "w4_restore_groups", "w4a16_gemm_tiled",
    "w4a16_moe_gemm_tiled", "w4a16_moe_gemm_swiglu_tiled",
]


def library_path():
    return _lib.LIB_PATH


# The current stream's raw handle for a device index.  torch's private
# accessor costs ~0.1 us per call where torch.cuda.current_stream(...).cuda_stream
# costs ~3 us: at M = 1 a decode product runs ~8 us on the GPU, so the host
# side of a call must stay well below that.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return ctypes_void(torch.cuda.current_stream(t.device).cuda_stream)


def ctypes_void(v):
    return None if v is None else int(v)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def w4_quantize_pack(W, Wq=None, S=None):
    """bf16 W [N, K] -> (int32 Wq [N, K/8], bf16 S [N, K/32])."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    if S is None:
        S = torch.empty((N, K // 32), dtype=torch.bfloat16, device=W.device)
    _need(Wq, "Wq", torch.int32)
    _need(S, "S", torch.bfloat16)
    if Wq.numel() != N * (K // 8) or S.numel() != N * (K // 32):
        raise ValueError("Wq / S sizes do not match W")
    lib = _lib.load()
    _lib.check("w4_quantize_pack",
               lib.w4_quantize_pack(_ptr(W), N, K, _ptr(Wq), _ptr(S), _stream(W)))
    return Wq, S


def w4_fake_quant(W, out=None):
    """QAT forward: bf16 W [N, K] -> bf16 dequant(quantize(W)).  ``out`` may be W."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    _need(out, "out", torch.bfloat16)
    if out.numel() != W.numel():
        raise ValueError("out size does not match W")
    lib = _lib.load()
    _lib.check("w4_fake_quant", lib.w4_fake_quant(_ptr(W), N, K, _ptr(out), _stream(W)))
    return out


def w4_quantize_pack_asym(W, Wq=None, S=None, Z=None):
    """bf16 W [N, K] -> (Wq int32 [N, K/8] unsigned codes, S bf16 [N, K/32],
    Z uint8 [N, K/32] zero points): asymmetric INT4 on the grid [0, 15]."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    if S is None:
        S = torch.empty((N, K // 32), dtype=torch.bfloat16, device=W.device)
    if Z is None:
        Z = torch.empty((N, K // 32), dtype=torch.uint8, device=W.device)
    _need(Wq, "Wq", torch.int32)
    _need(S, "S", torch.bfloat16)
    _need(Z, "Z", torch.uint8)
    if Wq.numel() != N * (K // 8) or S.numel() != N * (K // 32) or Z.numel() != N * (K // 32):
        raise ValueError("output sizes do not match W")
    lib = _lib.load()
    _lib.check("w4_quantize_pack_asym", lib.w4_quantize_pack_asym(
        _ptr(W), N, K, _ptr(Wq), _ptr(S), _ptr(Z), _stream(W)))
    return Wq, S, Z


def w4_fake_quant_asym(W, out=None):
    """bf16 W [N, K] -> bf16 (q - z) * s on the asymmetric grid.  ``out`` may be W."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    if out is None:
        out = torch.empty_like(W)
    _need(out, "out", torch.bfloat16)
    if out.numel() != W.numel():
        raise ValueError("out size does not match W")
    lib = _lib.load()
    _lib.check("w4_fake_quant_asym", lib.w4_fake_quant_asym(_ptr(W), N, K, _ptr(out), _stream(W)))
    return out


def _dequant(name, Wq, S, Z, out):
    _need(Wq, "Wq", torch.int32, 2)
    _need(S, "S", torch.bfloat16, 2)
    N, kw = Wq.shape
    K = kw * 8
    if tuple(S.shape) != (N, K // 32):
        raise ValueError(f"S must be [{N}, {K // 32}], got {tuple(S.shape)}")
    if Z is not None:
        _need(Z, "Z", torch.uint8, 2)
        if tuple(Z.shape) != (N, K // 32):
            raise ValueError(f"Z must be [{N}, {K // 32}], got {tuple(Z.shape)}")
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=Wq.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != N * K:
        raise ValueError("out size does not match [N, K]")
    lib = _lib.load()
    head = (_ptr(Wq), _ptr(S)) + (() if Z is None else (_ptr(Z),))
    _lib.check(name, getattr(lib, name)(*head, N, K, _ptr(out), _stream(Wq)))
    return out


def w4_dequant(Wq, S, out=None):
    """Packed codes -> bf16 W [N, K] = bf16(q * s): the fake-quantized values."""
    return _dequant("w4_dequant", Wq, S, None, out)


def w4_dequant_asym(Wq, S, Z, out=None):
    """Zero-point codes -> bf16 W [N, K] = bf16((q - z) * s)."""
    return _dequant("w4_dequant_asym", Wq, S, Z, out)


def w4_dequant_t(Wq, S, Z=None, out=None):
    """Packed codes -> bf16 W'^T [K, N] (the dequantized weight, transposed;
    zero-point codes when Z uint8 [N, K/32] is given)."""
    _need(Wq, "Wq", torch.int32, 2)
    _need(S, "S", torch.bfloat16, 2)
    N, kw = Wq.shape
    K = kw * 8
    if tuple(S.shape) != (N, K // 32):
        raise ValueError(f"S must be [{N}, {K // 32}], got {tuple(S.shape)}")
    if Z is not None:
        _need(Z, "Z", torch.uint8, 2)
        if tuple(Z.shape) != (N, K // 32):
            raise ValueError(f"Z must be [{N}, {K // 32}], got {tuple(Z.shape)}")
    if out is None:
        out = torch.empty((K, N), dtype=torch.bfloat16, device=Wq.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != N * K:
        raise ValueError("out size does not match [K, N]")
    lib = _lib.load()
    _lib.check("w4_dequant_t", lib.w4_dequant_t(_ptr(Wq), _ptr(S), _ptr(Z), N, K, _ptr(out),
                                                _stream(Wq)))
    return out


def w4_bf16_transpose(A, rows_padded=None, out=None):
    """A bf16 [R, C] -> A^T [C, RP] with RP = rows_padded (>= R, default R)
    and zero columns R .. RP - 1."""
    _need(A, "A", torch.bfloat16, 2)
    R, C = A.shape
    RP = R if rows_padded is None else int(rows_padded)
    if RP < R:
        raise ValueError("rows_padded must be >= the rows of A")
    if out is None:
        out = torch.empty((C, RP), dtype=torch.bfloat16, device=A.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != C * RP:
        raise ValueError(f"out must hold [{C}, {RP}]")
    lib = _lib.load()
    _lib.check("w4_bf16_transpose", lib.w4_bf16_transpose(_ptr(A), R, C, RP, _ptr(out),
                                                          _stream(A)))
    return out


def w4_bf16_gemm_nt(A, B, out=None):
    """bf16 C [M, N] = A [M, K] * B [N, K]^T with fp32 accumulation (K % 8 == 0)."""
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)} B {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out size does not match [M, N]")
    lib = _lib.load()
    _lib.check("w4_bf16_gemm_nt", lib.w4_bf16_gemm_nt(_ptr(A), _ptr(B), _ptr(out), M, N, K,
                                                      _stream(A)))
    return out


def w4a16_gemm(X, Wq, S, out=None):
    """Y [M, N] = X [M, K] * dequant(Wq, S)^T, bf16 out, fp32 accumulation."""
    _need(X, "X", torch.bfloat16, 2)
    _need(Wq, "Wq", torch.int32, 2)
    _need(S, "S", torch.bfloat16, 2)
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] * 8 != K or tuple(S.shape) != (N, K // 32):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)} Wq {tuple(Wq.shape)} "
                         f"S {tuple(S.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out size does not match [M, N]")
    lib = _lib.load()
    _lib.check("w4a16_gemm", lib.w4a16_gemm(_ptr(X), _ptr(Wq), _ptr(S), _ptr(out),
                                            M, N, K, _stream(X)))
    return out


def w4a16_gemm_asym(X, Wq, S, Z, out=None):
    """Zero-point weights: Y [M, N] = X [M, K] * dequant_asym(Wq, S, Z)^T with
    w' = bf16((q - z) s), q the unsigned codes of Wq and Z uint8 [N, K/32]."""
    _need(X, "X", torch.bfloat16, 2)
    _need(Wq, "Wq", torch.int32, 2)
    _need(S, "S", torch.bfloat16, 2)
    _need(Z, "Z", torch.uint8, 2)
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] * 8 != K or tuple(S.shape) != (N, K // 32) or tuple(Z.shape) != (N, K // 32):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)} Wq {tuple(Wq.shape)} "
                         f"S {tuple(S.shape)} Z {tuple(Z.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out size does not match [M, N]")
    lib = _lib.load()
    _lib.check("w4a16_gemm_asym", lib.w4a16_gemm_asym(_ptr(X), _ptr(Wq), _ptr(S), _ptr(Z),
                                                      _ptr(out), M, N, K, _stream(X)))
    return out


def w4_pick_block_size(T, k, E):
    return int(_lib.load().w4_pick_block_size(T, k, E))


def w4_moe_align_capacity(T, k, E, B):
    return int(_lib.load().w4_moe_align_capacity(T, k, E, B))


def moe_align_block_size(topk_ids, E, B, sorted_token_ids=None, expert_ids=None,
                         num_tokens_post_padded=None):
    """int32 topk_ids [T, k] -> (sorted_token_ids [cap], expert_ids [cap/B], ntpp [1])."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    cap = w4_moe_align_capacity(T, k, E, B)
    if cap < 0:
        raise ValueError("invalid T, k, E or B")
    dev = topk_ids.device
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(cap // B, dtype=torch.int32, device=dev)
    if num_tokens_post_padded is None:
        num_tokens_post_padded = torch.empty(1, dtype=torch.int32, device=dev)
    for t, n, size in ((sorted_token_ids, "sorted_token_ids", cap),
                       (expert_ids, "expert_ids", cap // B),
                       (num_tokens_post_padded, "num_tokens_post_padded", 1)):
        _need(t, n, torch.int32)
        if t.numel() < size:
            raise ValueError(f"{n} needs {size} entries")
    lib = _lib.load()
    _lib.check("moe_align_block_size", lib.moe_align_block_size(
        _ptr(topk_ids), T, k, E, B, _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _stream(topk_ids)))
    return sorted_token_ids, expert_ids, num_tokens_post_padded


def _moe_args(X, Wq, S, Z, sorted_token_ids, expert_ids, num_tokens_post_padded, T, k, B,
              x_row_div):
    """Checks shared by the grouped products; returns (E, N, K)."""
    _need(X, "X", torch.bfloat16, 2)
    _need(Wq, "Wq", torch.int32, 3)
    _need(S, "S", torch.bfloat16, 3)
    E, N, kw = Wq.shape
    K = kw * 8
    if X.shape[1] != K or tuple(S.shape) != (E, N, K // 32):
        raise ValueError("shape mismatch between X, Wq and S")
    if Z is not None:
        _need(Z, "Z", torch.uint8, 3)
        if tuple(Z.shape) != (E, N, K // 32):
            raise ValueError("Z must be [E, N, K/32]")
    if X.shape[0] != (T * k) // x_row_div:
        raise ValueError("X must have T*k / x_row_div rows")
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (num_tokens_post_padded, "num_tokens_post_padded")):
        _need(t, n, torch.int32)
    cap = w4_moe_align_capacity(T, k, E, B)
    if sorted_token_ids.numel() < cap or expert_ids.numel() < cap // B:
        raise ValueError("alignment buffers are smaller than the capacity")
    return E, N, K


def _moe_gemm(name, X, Wq, S, Z, sorted_token_ids, expert_ids, num_tokens_post_padded, T, k, B,
              x_row_div, topk_weights, out):
    E, N, K = _moe_args(X, Wq, S, Z, sorted_token_ids, expert_ids, num_tokens_post_padded, T, k,
                        B, x_row_div)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32)
        if topk_weights.numel() != T * k:
            raise ValueError("topk_weights must have T*k entries")
    if out is None:
        out = torch.empty((T * k, N), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * k * N:
        raise ValueError("out must be [T*k, N]")
    lib = _lib.load()
    head = (_ptr(X), _ptr(Wq), _ptr(S)) + (() if Z is None else (_ptr(Z),))
    _lib.check(name, getattr(lib, name)(
        *head, _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded),
        _ptr(topk_weights), _ptr(out), T, k, E, N, K, B, x_row_div, _stream(X)))
    return out


def _moe_gemm_swiglu(name, X, Wq, S, Z, sorted_token_ids, expert_ids, num_tokens_post_padded, T,
                     k, B, x_row_div, out):
    E, N, K = _moe_args(X, Wq, S, Z, sorted_token_ids, expert_ids, num_tokens_post_padded, T, k,
                        B, x_row_div)
    if N % 2:
        raise ValueError("Wq must hold 2I rows per expert")
    I = N // 2
    if out is None:
        out = torch.empty((T * k, I), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * k * I:
        raise ValueError("out must be [T*k, I]")
    lib = _lib.load()
    head = (_ptr(X), _ptr(Wq), _ptr(S)) + (() if Z is None else (_ptr(Z),))
    _lib.check(name, getattr(lib, name)(
        *head, _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded),
        _ptr(out), T, k, E, I, K, B, x_row_div, _stream(X)))
    return out


def w4a16_moe_gemm(X, Wq, S, sorted_token_ids, expert_ids, num_tokens_post_padded,
                   T, k, B, x_row_div, topk_weights=None, out=None):
    """Grouped expert product over aligned blocks.

    Row f of ``out`` [T*k, N] = X[f // x_row_div] * dequant(Wq[e], S[e])^T
    (times topk_weights.flat[f] when given) for every valid slot f of every
    block b < ntpp / B with e = expert_ids[b].  Other rows are not written.
    """
    return _moe_gemm("w4a16_moe_gemm", X, Wq, S, None, sorted_token_ids, expert_ids,
                     num_tokens_post_padded, T, k, B, x_row_div, topk_weights, out)


def w4a16_moe_gemm_asym(X, Wq, S, Z, sorted_token_ids, expert_ids, num_tokens_post_padded,
                        T, k, B, x_row_div, topk_weights=None, out=None):
    """``w4a16_moe_gemm`` with zero-point experts: Z uint8 [E, N, K/32] and
    w' = bf16((q - z) s) from the unsigned codes of Wq."""
    return _moe_gemm("w4a16_moe_gemm_asym", X, Wq, S, Z, sorted_token_ids, expert_ids,
                     num_tokens_post_padded, T, k, B, x_row_div, topk_weights, out)


def w4a16_moe_gemm_swiglu(X, Wq, S, sorted_token_ids, expert_ids, num_tokens_post_padded,
                          T, k, B, x_row_div, out=None):
    """gate_up projection with the SwiGLU fused into its epilogue.

    Wq [E, 2I, K/8] / S [E, 2I, K/32] hold gate rows [0, I) and up rows
    [I, 2I).  Row f of ``out`` [T*k, I] = bf16(silu(g) * u) with g, u the
    bf16 gate and up products of X[f // x_row_div], i.e. exactly
    w4_silu_mul(w4a16_moe_gemm(...)).  Other rows are not written.
    """
    return _moe_gemm_swiglu("w4a16_moe_gemm_swiglu", X, Wq, S, None, sorted_token_ids,
                            expert_ids, num_tokens_post_padded, T, k, B, x_row_div, out)


def w4a16_moe_gemm_swiglu_asym(X, Wq, S, Z, sorted_token_ids, expert_ids,
                               num_tokens_post_padded, T, k, B, x_row_div, out=None):
    """``w4a16_moe_gemm_swiglu`` with zero-point experts (Z uint8 [E, 2I, K/32])."""
    return _moe_gemm_swiglu("w4a16_moe_gemm_swiglu_asym", X, Wq, S, Z, sorted_token_ids,
                            expert_ids, num_tokens_post_padded, T, k, B, x_row_div, out)


def w4_silu_mul(H1, out=None):
    """bf16 H1 [R, 2I] -> bf16 A [R, I] = silu(H1[:, :I]) * H1[:, I:]."""
    _need(H1, "H1", torch.bfloat16, 2)
    R, I2 = H1.shape
    I = I2 // 2
    if I2 % 2:
        raise ValueError("H1 must have an even number of columns")
    if out is None:
        out = torch.empty((R, I), dtype=torch.bfloat16, device=H1.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != R * I:
        raise ValueError("out must be [R, I]")
    lib = _lib.load()
    _lib.check("w4_silu_mul", lib.w4_silu_mul(_ptr(H1), _ptr(out), R, I, _stream(H1)))
    return out


def w4_moe_sum(H2, topk_weights, T, k, out=None):
    """bf16 H2 [T*k, H] -> bf16 Out [T, H] = sum_j w[t, j] * H2[t*k + j]."""
    _need(H2, "H2", torch.bfloat16, 2)
    H = H2.shape[1]
    if H2.shape[0] != T * k:
        raise ValueError("H2 must have T*k rows")
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32)
        if topk_weights.numel() != T * k:
            raise ValueError("topk_weights must have T*k entries")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=H2.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * H:
        raise ValueError("out must be [T, H]")
    lib = _lib.load()
    _lib.check("w4_moe_sum", lib.w4_moe_sum(_ptr(H2), _ptr(topk_weights), _ptr(out), T, k, H,
                                            _stream(H2)))
    return out


def w4_moe_route(logits, k, topk_ids=None, topk_weights=None):
    """fp32 logits [T, E] -> (int32 ids [T, k], fp32 weights [T, k])."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", torch.int32)
    _need(topk_weights, "topk_weights", torch.float32)
    if topk_ids.numel() != T * k or topk_weights.numel() != T * k:
        raise ValueError("outputs must be [T, k]")
    lib = _lib.load()
    _lib.check("w4_moe_route", lib.w4_moe_route(_ptr(logits), T, E, k, _ptr(topk_ids),
                                                _ptr(topk_weights), _stream(logits)))
    return topk_ids, topk_weights


# ------------------------------------------------------ kernel-order codes --

def w4_repacked_words(N, K):
    """int32 words of one [N, K] matrix in the kernel-order layout."""
    n = int(_lib.load().w4_repacked_words(N, K))
    if n < 0:
        raise ValueError("invalid N or K")
    return n


def w4_repack(Wq, out=None):
    """Canonical codes Wq [N, K/8] (or [E, N, K/8]) -> kernel order
    Wt int32 [E, w4_repacked_words(N, K)] (E = 1 for a 2-D Wq)."""
    _need(Wq, "Wq", torch.int32)
    if Wq.dim() not in (2, 3):
        raise ValueError("Wq must be [N, K/8] or [E, N, K/8]")
    E, N, kw = (1,) + tuple(Wq.shape) if Wq.dim() == 2 else tuple(Wq.shape)
    K = kw * 8
    words = w4_repacked_words(N, K)
    if out is None:
        out = torch.empty((E, words), dtype=torch.int32, device=Wq.device)
    _need(out, "out", torch.int32)
    if out.numel() != E * words:
        raise ValueError(f"out needs {E * words} words")
    lib = _lib.load()
    _lib.check("w4_repack", lib.w4_repack(_ptr(Wq), E, N, K, _ptr(out), _stream(Wq)))
    return out


def w4_restore(Wt, N, K, out=None):
    """Kernel-order codes Wt [E, words] -> canonical Wq [E, N, K/8] (the
    inverse of w4_repack; [N, K/8] when E = 1 and ``out`` is not given)."""
    _need(Wt, "Wt", torch.int32)
    words = w4_repacked_words(N, K)
    if Wt.numel() % max(words, 1) != 0:
        raise ValueError("Wt size is not a whole number of matrices")
    E = Wt.numel() // max(words, 1)
    if out is None:
        shape = (N, K // 8) if E == 1 else (E, N, K // 8)
        out = torch.empty(shape, dtype=torch.int32, device=Wt.device)
    _need(out, "out", torch.int32)
    if out.numel() != E * N * (K // 8):
        raise ValueError("out size does not match [E, N, K/8]")
    lib = _lib.load()
    _lib.check("w4_restore", lib.w4_restore(_ptr(Wt), E, N, K, _ptr(out), _stream(Wt)))
    return out


def w4_repacked_group_elems(N, K):
    """Elements of one [N, K/32] per-group array in the kernel-order layout."""
    n = int(_lib.load().w4_repacked_group_elems(N, K))
    if n < 0:
        raise ValueError("invalid N or K")
    return n


_GROUP_DTYPES = {torch.bfloat16: 2, torch.uint8: 1}


def w4_repack_groups(A, out=None):
    """Per-group scales (bf16) or zero points (uint8) A [N, K/32] (or
    [E, N, K/32]) -> kernel order [E, w4_repacked_group_elems(N, K)]."""
    if not isinstance(A, torch.Tensor) or A.dtype not in _GROUP_DTYPES:
        raise TypeError("A must be a bf16 or uint8 tensor")
    _need(A, "A", A.dtype)
    if A.dim() not in (2, 3):
        raise ValueError("A must be [N, K/32] or [E, N, K/32]")
    E, N, G = (1,) + tuple(A.shape) if A.dim() == 2 else tuple(A.shape)
    K = 32 * G
    elems = w4_repacked_group_elems(N, K)
    if out is None:
        out = torch.empty((E, elems), dtype=A.dtype, device=A.device)
    _need(out, "out", A.dtype)
    if out.numel() != E * elems:
        raise ValueError(f"out needs {E * elems} elements")
    lib = _lib.load()
    _lib.check("w4_repack_groups", lib.w4_repack_groups(
        _ptr(A), _GROUP_DTYPES[A.dtype], E, N, K, _ptr(out), _stream(A)))
    return out


def w4_restore_groups(At, N, K, out=None):
    """Kernel-order per-group values At [E, elems] -> canonical [E, N, K/32]
    (the inverse of w4_repack_groups; [N, K/32] when E = 1 and ``out`` is not
    given)."""
    if not isinstance(At, torch.Tensor) or At.dtype not in _GROUP_DTYPES:
        raise TypeError("At must be a bf16 or uint8 tensor")
    _need(At, "At", At.dtype)
    elems = w4_repacked_group_elems(N, K)
    if At.numel() % max(elems, 1) != 0:
        raise ValueError("At size is not a whole number of matrices")
    E = At.numel() // max(elems, 1)
    if out is None:
        shape = (N, K // 32) if E == 1 else (E, N, K // 32)
        out = torch.empty(shape, dtype=At.dtype, device=At.device)
    _need(out, "out", At.dtype)
    if out.numel() != E * N * (K // 32):
        raise ValueError("out size does not match [E, N, K/32]")
    lib = _lib.load()
    _lib.check("w4_restore_groups", lib.w4_restore_groups(
        _ptr(At), _GROUP_DTYPES[At.dtype], E, N, K, _ptr(out), _stream(At)))
    return out


def _tiled_experts(X, Wt, St, Z, N, E=None):
    """E (from Wt unless given) and K of kernel-order operands, checking
    their sizes."""
    _need(X, "X", torch.bfloat16, 2)
    _need(Wt, "Wt", torch.int32)
    _need(St, "St", torch.bfloat16)
    K = X.shape[1]
    words, elems = w4_repacked_words(N, K), w4_repacked_group_elems(N, K)
    if E is None:
        E = Wt.numel() // max(words, 1)
    if E < 1 or Wt.numel() != E * words or St.numel() != E * elems:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)} Wt {tuple(Wt.shape)} "
                         f"St {tuple(St.shape)} for N={N}")
    if Z is not None:
        _need(Z, "Z", torch.uint8)
        if Z.numel() != E * elems:
            raise ValueError("Z must hold w4_repacked_group_elems(N, K) values per matrix")
    return E, K


def w4a16_gemm_tiled(X, Wt, St, N, Z=None, out=None):
    """w4a16_gemm (Z None) / w4a16_gemm_asym on kernel-order operands: codes
    Wt [1, w4_repacked_words(N, K)], scales St and zero points Z
    [1, w4_repacked_group_elems(N, K)]; K from X."""
    _, K = _tiled_experts(X, Wt, St, Z, N, E=1)
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != M * N:
        raise ValueError("out size does not match [M, N]")
    lib = _lib.load()
    _lib.check("w4a16_gemm_tiled", lib.w4a16_gemm_tiled(
        _ptr(X), _ptr(Wt), _ptr(St), _ptr(Z), _ptr(out), M, N, K, _stream(X)))
    return out


def _moe_tiled_args(X, Wt, St, Z, N, T, k, x_row_div):
    E, K = _tiled_experts(X, Wt, St, Z, N)
    if X.shape[0] != (T * k) // x_row_div:
        raise ValueError("X must have T*k / x_row_div rows")
    return E, K


def w4a16_moe_gemm_tiled(X, Wt, St, N, sorted_token_ids, expert_ids, num_tokens_post_padded,
                         T, k, B, x_row_div, Z=None, topk_weights=None, out=None):
    """``w4a16_moe_gemm`` (Z None) / ``w4a16_moe_gemm_asym`` on kernel-order
    expert operands: Wt [E, w4_repacked_words(N, K)], St and Z
    [E, w4_repacked_group_elems(N, K)]; E from Wt, K from X."""
    E, K = _moe_tiled_args(X, Wt, St, Z, N, T, k, x_row_div)
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (num_tokens_post_padded, "num_tokens_post_padded")):
        _need(t, n, torch.int32)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32)
        if topk_weights.numel() != T * k:
            raise ValueError("topk_weights must have T*k entries")
    if out is None:
        out = torch.empty((T * k, N), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * k * N:
        raise ValueError("out must be [T*k, N]")
    lib = _lib.load()
    _lib.check("w4a16_moe_gemm_tiled", lib.w4a16_moe_gemm_tiled(
        _ptr(X), _ptr(Wt), _ptr(St), _ptr(Z), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(topk_weights), _ptr(out), T, k, E, N, K, B,
        x_row_div, _stream(X)))
    return out


def w4a16_moe_gemm_swiglu_tiled(X, Wt, St, N, sorted_token_ids, expert_ids,
                                num_tokens_post_padded, T, k, B, x_row_div, Z=None, out=None):
    """``w4a16_moe_gemm_swiglu`` (Z None) / ``..._asym`` on kernel-order
    expert operands of N = 2I rows (Wt, St, Z as ``w4a16_moe_gemm_tiled``)."""
    E, K = _moe_tiled_args(X, Wt, St, Z, N, T, k, x_row_div)
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (num_tokens_post_padded, "num_tokens_post_padded")):
        _need(t, n, torch.int32)
    if N % 2:
        raise ValueError("Wt must hold 2I rows per expert")
    I = N // 2
    if out is None:
        out = torch.empty((T * k, I), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * k * I:
        raise ValueError("out must be [T*k, I]")
    lib = _lib.load()
    _lib.check("w4a16_moe_gemm_swiglu_tiled", lib.w4a16_moe_gemm_swiglu_tiled(
        _ptr(X), _ptr(Wt), _ptr(St), _ptr(Z), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(out), T, k, E, I, K, B, x_row_div, _stream(X)))
    return out


# ---------------------------------------------- down product + top-k combine --

def w4_moe_combine_workspace_words(T, k, E, N, B):
    """int32 arrival counters ``w4a16_moe_gemm_combine`` needs."""
    n = int(_lib.load().w4_moe_combine_workspace_words(T, k, E, N, B))
    if n < 0:
        raise ValueError("invalid T, k, E, N or B")
    return n


def w4a16_moe_gemm_combine(A, Wq, S, sorted_token_ids, expert_ids, num_tokens_post_padded,
                           topk_ids, topk_weights, B, N=None, tiled=False, H2=None, out=None,
                           workspace=None):
    """The grouped down product with the top-k combine fused.

    A bf16 [T*k, K]; canonical experts Wq [E, N, K/8], S [E, N, K/32], or
    (``tiled``) kernel-order Wt / St with N given.  Returns (Out [T, N],
    H2 [T*k, N]); ``workspace`` int32 [w4_moe_combine_workspace_words(...)]
    holding zeros (allocated zeroed when omitted; every call leaves it zero).
    """
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    if tiled:
        if N is None:
            raise ValueError("kernel-order experts need N")
        E, K = _moe_tiled_args(A, Wq, S, None, N, T, k, 1)
        for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                     (num_tokens_post_padded, "num_tokens_post_padded")):
            _need(t, n, torch.int32)
    else:
        E, N, K = _moe_args(A, Wq, S, None, sorted_token_ids, expert_ids,
                            num_tokens_post_padded, T, k, B, 1)
    _need(topk_weights, "topk_weights", torch.float32)
    if topk_weights.numel() != T * k:
        raise ValueError("topk_weights must be [T, k]")
    dev = A.device
    if H2 is None:
        H2 = torch.empty((T * k, N), dtype=torch.bfloat16, device=dev)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    _need(H2, "H2", torch.bfloat16)
    _need(out, "out", torch.bfloat16)
    if H2.numel() != T * k * N or out.numel() != T * N:
        raise ValueError("H2 must be [T*k, N] and out [T, N]")
    words = w4_moe_combine_workspace_words(T, k, E, N, B)
    if workspace is None:
        workspace = torch.zeros(words, dtype=torch.int32, device=dev)
    _need(workspace, "workspace", torch.int32)
    if workspace.numel() < words:
        raise ValueError(f"workspace needs {words} int32 words")
    lib = _lib.load()
    _lib.check("w4a16_moe_gemm_combine", lib.w4a16_moe_gemm_combine(
        _ptr(A), _ptr(Wq), _ptr(S), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(topk_ids), _ptr(topk_weights), _ptr(H2), _ptr(out),
        T, k, E, N, K, B, 1 if tiled else 0, _ptr(workspace), _stream(A)))
    return out, H2


def w4a16_moe_gemm_combine_noalloc(A, Wq, S, sorted_token_ids, expert_ids,
                                   num_tokens_post_padded, topk_ids, topk_weights, B, H2, out,
                                   N=None, tiled=False):
    """``w4a16_moe_gemm_combine`` with the library's own counters: the call
    allocates nothing (H2 and out are given).  Returns (out, H2)."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    if tiled:
        if N is None:
            raise ValueError("kernel-order experts need N")
        E, K = _moe_tiled_args(A, Wq, S, None, N, T, k, 1)
    else:
        E, N, K = _moe_args(A, Wq, S, None, sorted_token_ids, expert_ids,
                            num_tokens_post_padded, T, k, B, 1)
    for t, n, dt in ((sorted_token_ids, "sorted_token_ids", torch.int32),
                     (expert_ids, "expert_ids", torch.int32),
                     (num_tokens_post_padded, "num_tokens_post_padded", torch.int32),
                     (topk_weights, "topk_weights", torch.float32),
                     (H2, "H2", torch.bfloat16), (out, "out", torch.bfloat16)):
        _need(t, n, dt)
    if H2.numel() != T * k * N or out.numel() != T * N or topk_weights.numel() != T * k:
        raise ValueError("H2 must be [T*k, N], out [T, N], topk_weights [T, k]")
    lib = _lib.load()
    _lib.check("w4a16_moe_gemm_combine_noalloc", lib.w4a16_moe_gemm_combine_noalloc(
        _ptr(A), _ptr(Wq), _ptr(S), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(topk_ids), _ptr(topk_weights), _ptr(H2), _ptr(out),
        T, k, E, N, K, B, 1 if tiled else 0, _stream(A)))
    return out, H2
