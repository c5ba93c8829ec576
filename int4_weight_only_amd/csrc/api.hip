// C ABI of libw4a16.so: argument validation and dispatch.
//
// Every entry point validates all of its arguments before enqueueing any
// work, so a nonzero status leaves the outputs untouched.  Nothing here
// allocates, synchronizes or reads device memory.
#include "w4a16.h"

#include "common.h"

namespace {

thread_local int g_last_hip_error = 0;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return W4_OK;
  g_last_hip_error = (int)e;
  return W4_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

constexpr int64_t kMaxI32 = 2147483647;

// The kernels address operands with 32-bit raw-buffer offsets and use
// offset 2^31 as "past the end" (reads zero): every buffer a kernel spans
// must stay below 2^31 bytes.
inline bool fits_buffer(int64_t bytes) { return bytes >= 0 && bytes < ((int64_t)1 << 31); }

// Decode path (M <= 32): per-workgroup weight buffers, X below 2^30 bytes.
inline bool use_decode(int64_t M, int64_t K) { return M <= 32 && K <= ((int64_t)1 << 24); }

// Tiled path: X [M, K] and the whole of Wq [N, K/8] in one buffer each,
// and a 1-D grid of tiles.
inline bool gemm_fits(int64_t M, int64_t N, int64_t K) {
  return fits_buffer(M * K * 2) && fits_buffer(N * (K / 2)) &&
         ((M + 127) / 128) * ((N + 255) / 256) < ((int64_t)1 << 31) - 8;
}

}  // namespace

namespace w4 {

// The launchers size their grids by it (decode tiles per workgroup, the
// bf16 product's tile shape).
int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace w4

extern "C" {

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_NULL: return "null pointer";
    case W4_ERR_SHAPE: return "bad shape";
    case W4_ERR_MISALIGNED: return "misaligned pointer";
    case W4_ERR_UNSUPPORTED: return "unsupported arguments";
    case W4_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int w4_last_hip_error(void) { return g_last_hip_error; }

const char* w4_version(void) { return "w4a16 gfx950 0.1"; }

int w4_quantize_pack(const uint16_t* W, int64_t N, int64_t K, int32_t* Wq, uint16_t* S,
                     void* stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (N == 0 || K == 0) return W4_OK;
  if (!W || !Wq || !S) return W4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(S, 2)) return W4_ERR_MISALIGNED;
  const int64_t words = N * (K / 8);
  if (words / (K / 8) != N || words > ((int64_t)1 << 38)) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_quantize(W, words, Wq, S, nullptr, nullptr, false, false,
                                        as_stream(stream)));
}

int w4_quantize_pack_asym(const uint16_t* W, int64_t N, int64_t K, int32_t* Wq, uint16_t* S,
                          uint8_t* Z, void* stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (N == 0 || K == 0) return W4_OK;
  if (!W || !Wq || !S || !Z) return W4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(Wq, 16) || !aligned(S, 2)) return W4_ERR_MISALIGNED;
  const int64_t words = N * (K / 8);
  if (words / (K / 8) != N || words > ((int64_t)1 << 38)) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_quantize(W, words, Wq, S, Z, nullptr, false, true,
                                        as_stream(stream)));
}

int w4_fake_quant_asym(const uint16_t* W, int64_t N, int64_t K, uint16_t* W_fq, void* stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (N == 0 || K == 0) return W4_OK;
  if (!W || !W_fq) return W4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(W_fq, 16)) return W4_ERR_MISALIGNED;
  const int64_t words = N * (K / 8);
  if (words / (K / 8) != N || words > ((int64_t)1 << 38)) return W4_ERR_UNSUPPORTED;
  const uintptr_t a = (uintptr_t)W, b = (uintptr_t)W_fq, len = (uintptr_t)(words * 16);
  if (a != b && a < b + len && b < a + len) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_quantize(W, words, nullptr, nullptr, nullptr, W_fq, true, true,
                                        as_stream(stream)));
}

int w4_fake_quant(const uint16_t* W, int64_t N, int64_t K, uint16_t* W_fq, void* stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (N == 0 || K == 0) return W4_OK;
  if (!W || !W_fq) return W4_ERR_NULL;
  if (!aligned(W, 16) || !aligned(W_fq, 16)) return W4_ERR_MISALIGNED;
  const int64_t words = N * (K / 8);
  if (words / (K / 8) != N || words > ((int64_t)1 << 38)) return W4_ERR_UNSUPPORTED;
  // in place is fine; partial overlap is not
  const uintptr_t a = (uintptr_t)W, b = (uintptr_t)W_fq, len = (uintptr_t)(words * 16);
  if (a != b && a < b + len && b < a + len) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_quantize(W, words, nullptr, nullptr, nullptr, W_fq, true, false,
                                        as_stream(stream)));
}

}  // extern "C"

namespace {

int dequant_checked(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, bool asym, int64_t N,
                    int64_t K, uint16_t* W, void* stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (N == 0 || K == 0) return W4_OK;
  if (!Wq || !S || !W || (asym && !Z)) return W4_ERR_NULL;
  if (!aligned(Wq, 4) || !aligned(S, 2) || !aligned(W, 16)) return W4_ERR_MISALIGNED;
  const int64_t words = N * (K / 8);
  if (words / (K / 8) != N || words > ((int64_t)1 << 38)) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_dequant(Wq, S, asym ? Z : nullptr, W, words, as_stream(stream)));
}

}  // namespace

extern "C" {

int w4_dequant(const int32_t* Wq, const uint16_t* S, int64_t N, int64_t K, uint16_t* W,
               void* stream) {
  return dequant_checked(Wq, S, nullptr, false, N, K, W, stream);
}

int w4_dequant_asym(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, int64_t N, int64_t K,
                    uint16_t* W, void* stream) {
  return dequant_checked(Wq, S, Z, true, N, K, W, stream);
}

int w4a16_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y, int64_t M,
               int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4_OK;
  if (!Y) return W4_ERR_NULL;
  if (!aligned(Y, 4)) return W4_ERR_MISALIGNED;
  if (M > kMaxI32 || N > kMaxI32 || K > kMaxI32 || M * N > ((int64_t)1 << 40) ||
      N * (K / 8) > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  if (K == 0) return hip_status(w4::launch_zero_bf16(Y, M * N, as_stream(stream)));
  if (!X || !Wq || !S) return W4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(S, 2)) return W4_ERR_MISALIGNED;
  if (use_decode(M, K))
    return hip_status(w4::launch_gemv(X, Wq, S, Y, M, N, K, as_stream(stream)));
  if (!gemm_fits(M, N, K)) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_gemm(X, Wq, S, Y, M, N, K, as_stream(stream)));
}

int w4a16_gemm_asym(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                    uint16_t* Y, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4_OK;
  if (!Y) return W4_ERR_NULL;
  if (!aligned(Y, 4)) return W4_ERR_MISALIGNED;
  if (M > kMaxI32 || N > kMaxI32 || K > kMaxI32 || M * N > ((int64_t)1 << 40) ||
      N * (K / 8) > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  if (!use_decode(M, K) && !gemm_fits(M, N, K)) return W4_ERR_UNSUPPORTED;
  if (K == 0) return hip_status(w4::launch_zero_bf16(Y, M * N, as_stream(stream)));
  if (!X || !Wq || !S || !Z) return W4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(S, 2)) return W4_ERR_MISALIGNED;
  if (use_decode(M, K))
    return hip_status(w4::launch_gemv_zp(X, Wq, S, Z, Y, M, N, K, as_stream(stream)));
  return hip_status(w4::launch_gemm_zp(X, Wq, S, Z, Y, M, N, K, as_stream(stream)));
}

int64_t w4_repacked_words(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % 32 != 0 || N > kMaxI32 || K > kMaxI32) return -1;
  return w4::tiled_words(N, K);
}

namespace {
int relayout_checked(const int32_t* src, int32_t* dst, int64_t E, int64_t N, int64_t K,
                     bool restore, void* stream) {
  if (E < 0 || N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (E == 0 || N == 0 || K == 0) return W4_OK;
  if (N > kMaxI32 || K > kMaxI32 || E * w4::tiled_words(N, K) > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  if (!src || !dst) return W4_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return W4_ERR_MISALIGNED;
  // the two buffers must not overlap
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  const uintptr_t la = (uintptr_t)(restore ? E * w4::tiled_words(N, K) : E * N * (K / 8)) * 4;
  const uintptr_t lb = (uintptr_t)(restore ? E * N * (K / 8) : E * w4::tiled_words(N, K)) * 4;
  if (a < b + lb && b < a + la) return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_relayout(src, dst, E, N, K, restore, as_stream(stream)));
}
}  // namespace

int w4_repack(const int32_t* Wq, int64_t E, int64_t N, int64_t K, int32_t* Wt, void* stream) {
  return relayout_checked(Wq, Wt, E, N, K, false, stream);
}

int w4_restore(const int32_t* Wt, int64_t E, int64_t N, int64_t K, int32_t* Wq, void* stream) {
  return relayout_checked(Wt, Wq, E, N, K, true, stream);
}

int64_t w4_repacked_group_elems(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % 32 != 0 || N > kMaxI32 || K > kMaxI32) return -1;
  return w4::tiled_group_elems(N, K);
}

namespace {
int relayout_groups_checked(const void* src, void* dst, int32_t elem_bytes, int64_t E, int64_t N,
                            int64_t K, bool restore, void* stream) {
  if (E < 0 || N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2) return W4_ERR_UNSUPPORTED;
  if (E == 0 || N == 0 || K == 0) return W4_OK;
  if (N > kMaxI32 || K > kMaxI32 || E * w4::tiled_group_elems(N, K) > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  if (!src || !dst) return W4_ERR_NULL;
  if (!aligned(src, elem_bytes) || !aligned(dst, elem_bytes)) return W4_ERR_MISALIGNED;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  const int64_t tiled = E * w4::tiled_group_elems(N, K), canon = E * N * (K / 32);
  const uintptr_t la = (uintptr_t)(restore ? tiled : canon) * elem_bytes;
  const uintptr_t lb = (uintptr_t)(restore ? canon : tiled) * elem_bytes;
  if (a < b + lb && b < a + la) return W4_ERR_UNSUPPORTED;
  return hip_status(
      w4::launch_relayout_groups(src, dst, elem_bytes, E, N, K, restore, as_stream(stream)));
}
}  // namespace

int w4_repack_groups(const void* A, int32_t elem_bytes, int64_t E, int64_t N, int64_t K, void* At,
                     void* stream) {
  return relayout_groups_checked(A, At, elem_bytes, E, N, K, false, stream);
}

int w4_restore_groups(const void* At, int32_t elem_bytes, int64_t E, int64_t N, int64_t K, void* A,
                      void* stream) {
  return relayout_groups_checked(At, A, elem_bytes, E, N, K, true, stream);
}

int w4a16_gemm_tiled(const uint16_t* X, const int32_t* Wt, const uint16_t* S, const uint8_t* Z,
                     uint16_t* Y, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4_OK;
  if (!Y) return W4_ERR_NULL;
  if (!aligned(Y, 4)) return W4_ERR_MISALIGNED;
  if (M > kMaxI32 || N > kMaxI32 || K > kMaxI32 || M * N > ((int64_t)1 << 40) ||
      N * (K / 8) > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  const bool decode = use_decode(M, K);
  if (!decode && !(fits_buffer(M * K * 2) && fits_buffer(w4::tiled_words(N, K) * 4) &&
                   ((M + 127) / 128) * ((N + 255) / 256) < ((int64_t)1 << 31) - 8))
    return W4_ERR_UNSUPPORTED;
  if (K == 0) return hip_status(w4::launch_zero_bf16(Y, M * N, as_stream(stream)));
  if (!X || !Wt || !S) return W4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Wt, 16) || !aligned(S, 2)) return W4_ERR_MISALIGNED;
  if (decode)
    return hip_status(w4::launch_gemv_any(X, Wt, S, Z, Y, M, N, K, true, as_stream(stream)));
  return hip_status(w4::launch_gemm_any(X, Wt, S, Z, Y, M, N, K, true, as_stream(stream)));
}

int w4_dequant_t(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, int64_t N, int64_t K,
                 uint16_t* WT, void* stream) {
  if (N < 0 || K < 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (N == 0 || K == 0) return W4_OK;
  if (!Wq || !S || !WT) return W4_ERR_NULL;
  if (!aligned(Wq, 4) || !aligned(S, 2) || !aligned(WT, 16)) return W4_ERR_MISALIGNED;
  if (N > kMaxI32 || K > kMaxI32 || N * K > ((int64_t)1 << 40) ||
      ((N + 63) / 64) * ((K + 127) / 128) >= kMaxI32)
    return W4_ERR_UNSUPPORTED;
  return hip_status(w4::launch_dequant_t(Wq, S, Z, WT, N, K, as_stream(stream)));
}

int w4_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N,
                    int64_t K, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 8 != 0) return W4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4_OK;
  if (!C) return W4_ERR_NULL;
  if (!aligned(C, 2)) return W4_ERR_MISALIGNED;
  if (!fits_buffer(M * K * 2) || !fits_buffer(N * K * 2) ||
      ((M + 127) / 128) * ((N + 127) / 128) >= kMaxI32 || M * N > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  if (K == 0) return hip_status(w4::launch_zero_bf16(C, M * N, as_stream(stream)));
  if (!A || !B) return W4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16)) return W4_ERR_MISALIGNED;
  return hip_status(w4::launch_bf16_gemm_nt(A, B, C, M, N, K, as_stream(stream)));
}

int w4_bf16_transpose(const uint16_t* A, int64_t R, int64_t C, int64_t RP, uint16_t* AT,
                      void* stream) {
  if (R < 0 || C < 0 || RP < R) return W4_ERR_SHAPE;
  if (RP == 0 || C == 0) return W4_OK;
  if (!AT || (R > 0 && !A)) return W4_ERR_NULL;
  if (!aligned(A, 2) || !aligned(AT, 2)) return W4_ERR_MISALIGNED;
  if (R > ((int64_t)1 << 40) / (C > 0 ? C : 1) || RP > ((int64_t)1 << 40) / C ||
      ((RP + 63) / 64) * ((C + 63) / 64) >= kMaxI32)
    return W4_ERR_UNSUPPORTED;
  const uintptr_t a = (uintptr_t)A, b = (uintptr_t)AT;
  const uintptr_t la = (uintptr_t)(R * C) * 2u, lb = (uintptr_t)(RP * C) * 2u;
  if (R > 0 && a < b + lb && b < a + la) return W4_ERR_UNSUPPORTED;   // overlapping buffers
  return hip_status(w4::launch_transpose_bf16(A, AT, R, C, RP, as_stream(stream)));
}

int32_t w4_pick_block_size(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const int64_t mean = (T * k + E - 1) / E;
  int64_t p = 1;
  while (p < mean) p *= 2;
  if (p < 16) p = 16;
  if (p > 64) p = 64;
  return (int32_t)p;
}

int64_t w4_moe_align_capacity(int64_t T, int32_t k, int32_t E, int32_t B) {
  if (T < 0 || k < 1 || E < 1 || B < 1) return -1;
  const int64_t n = T * k + (int64_t)E * (B - 1);
  return ((n + B - 1) / B) * B;
}

int moe_align_block_size(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t B,
                         int32_t* sorted_token_ids, int32_t* expert_ids,
                         int32_t* num_tokens_post_padded, void* stream) {
  if (T < 0 || k < 1 || E < 1 || B < 1) return W4_ERR_SHAPE;
  if (E > 1024 || B > 1024) return W4_ERR_UNSUPPORTED;
  if (T * k + (int64_t)E * B >= kMaxI32) return W4_ERR_UNSUPPORTED;
  if (!sorted_token_ids || !expert_ids || !num_tokens_post_padded) return W4_ERR_NULL;
  if (T > 0 && !topk_ids) return W4_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(sorted_token_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(num_tokens_post_padded, 4))
    return W4_ERR_MISALIGNED;
  const int64_t cap = w4_moe_align_capacity(T, k, E, B);
  return hip_status(w4::launch_align(topk_ids, T, k, E, B, cap, sorted_token_ids, expert_ids,
                                     num_tokens_post_padded, as_stream(stream)));
}

}  // extern "C"

namespace {

// Shared validation and dispatch of the grouped products (Z == nullptr:
// symmetric codes).  N is the weight rows per expert (2I with the SwiGLU).
// Checks shared by the grouped products; W4_OK, or -1 for a valid call with
// nothing to do (T == 0), or an error status.
int moe_gemm_validate(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                      bool asym, const int32_t* sorted_token_ids, const int32_t* expert_ids,
                      const int32_t* num_tokens_post_padded, const float* topk_weights,
                      uint16_t* Y, int64_t T, int32_t k, int32_t E, int64_t N, int64_t K,
                      int32_t B, int32_t x_row_div, bool swiglu, bool tiled) {
  if (T < 0 || k < 1 || E < 1 || N < 1 || K < 32 || K % 32 != 0 || B < 1) return W4_ERR_SHAPE;
  if (x_row_div != 1 && x_row_div != k) return W4_ERR_SHAPE;
  if (B > 1024 || E > 1024) return W4_ERR_UNSUPPORTED;
  if (T * k + (int64_t)E * B >= kMaxI32 || N > kMaxI32 || K > kMaxI32 ||
      (int64_t)E * N * (K / 8) > ((int64_t)1 << 40) || T * k * N > ((int64_t)1 << 40))
    return W4_ERR_UNSUPPORTED;
  // one buffer spans X's rows, one an expert's Wq
  if (!fits_buffer((T * k / x_row_div) * K * 2) ||
      !fits_buffer(tiled ? w4::tiled_words(N, K) * 4 : N * (K / 2)))
    return W4_ERR_UNSUPPORTED;
  if (T == 0) return -1;
  if (!X || !Wq || !S || !sorted_token_ids || !expert_ids || !num_tokens_post_padded || !Y ||
      (asym && !Z))
    return W4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Wq, 16) || !aligned(S, 2) || !aligned(Y, 4) ||
      !aligned(sorted_token_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(num_tokens_post_padded, 4) || !aligned(topk_weights, 4))
    return W4_ERR_MISALIGNED;
  if (w4::moe_gemm_workgroups(T, k, E, N, B, swiglu) >= kMaxI32) return W4_ERR_UNSUPPORTED;
  return W4_OK;
}

// Shared validation and dispatch of the grouped products (Z == nullptr:
// symmetric codes).  N is the weight rows per expert (2I with the SwiGLU).
int moe_gemm_checked(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                     bool asym, const int32_t* sorted_token_ids, const int32_t* expert_ids,
                     const int32_t* num_tokens_post_padded, const float* topk_weights,
                     uint16_t* Y, int64_t T, int32_t k, int32_t E, int64_t N, int64_t K,
                     int32_t B, int32_t x_row_div, bool swiglu, bool tiled, void* stream) {
  const int v = moe_gemm_validate(X, Wq, S, Z, asym, sorted_token_ids, expert_ids,
                                  num_tokens_post_padded, topk_weights, Y, T, k, E, N, K, B,
                                  x_row_div, swiglu, tiled);
  if (v != W4_OK) return v < 0 ? W4_OK : v;
  if (swiglu)
    return hip_status(w4::launch_moe_gemm_swiglu(X, Wq, S, asym ? Z : nullptr, sorted_token_ids,
                                                 expert_ids, num_tokens_post_padded, Y, T, k, E,
                                                 N / 2, K, B, x_row_div, tiled,
                                                 as_stream(stream)));
  return hip_status(w4::launch_moe_gemm(X, Wq, S, asym ? Z : nullptr, sorted_token_ids,
                                        expert_ids, num_tokens_post_padded, topk_weights, Y, T,
                                        k, E, N, K, B, x_row_div, tiled, as_stream(stream)));
}

}  // namespace

extern "C" {

int w4a16_moe_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded, const float* topk_weights, uint16_t* Y,
                   int64_t T, int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                   int32_t x_row_div, void* stream) {
  return moe_gemm_checked(X, Wq, S, nullptr, false, sorted_token_ids, expert_ids,
                          num_tokens_post_padded, topk_weights, Y, T, k, E, N, K, B, x_row_div,
                          false, false, stream);
}

int w4a16_moe_gemm_asym(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                        const int32_t* sorted_token_ids, const int32_t* expert_ids,
                        const int32_t* num_tokens_post_padded, const float* topk_weights,
                        uint16_t* Y, int64_t T, int32_t k, int32_t E, int64_t N, int64_t K,
                        int32_t B, int32_t x_row_div, void* stream) {
  return moe_gemm_checked(X, Wq, S, Z, true, sorted_token_ids, expert_ids,
                          num_tokens_post_padded, topk_weights, Y, T, k, E, N, K, B, x_row_div,
                          false, false, stream);
}

int w4a16_moe_gemm_swiglu(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const int32_t* sorted_token_ids, const int32_t* expert_ids,
                          const int32_t* num_tokens_post_padded, uint16_t* A, int64_t T,
                          int32_t k, int32_t E, int64_t I, int64_t K, int32_t B,
                          int32_t x_row_div, void* stream) {
  if (I < 1) return W4_ERR_SHAPE;
  const int64_t N = I > kMaxI32 ? kMaxI32 + 1 : 2 * I;   // past the limit: unsupported
  return moe_gemm_checked(X, Wq, S, nullptr, false, sorted_token_ids, expert_ids,
                          num_tokens_post_padded, nullptr, A, T, k, E, N, K, B, x_row_div,
                          true, false, stream);
}

int w4a16_moe_gemm_swiglu_asym(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                               const uint8_t* Z, const int32_t* sorted_token_ids,
                               const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                               uint16_t* A, int64_t T, int32_t k, int32_t E, int64_t I, int64_t K,
                               int32_t B, int32_t x_row_div, void* stream) {
  if (I < 1) return W4_ERR_SHAPE;
  const int64_t N = I > kMaxI32 ? kMaxI32 + 1 : 2 * I;   // past the limit: unsupported
  return moe_gemm_checked(X, Wq, S, Z, true, sorted_token_ids, expert_ids,
                          num_tokens_post_padded, nullptr, A, T, k, E, N, K, B, x_row_div,
                          true, false, stream);
}

int w4a16_moe_gemm_tiled(const uint16_t* X, const int32_t* Wt, const uint16_t* S,
                         const uint8_t* Z, const int32_t* sorted_token_ids,
                         const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                         const float* topk_weights, uint16_t* Y, int64_t T, int32_t k, int32_t E,
                         int64_t N, int64_t K, int32_t B, int32_t x_row_div, void* stream) {
  return moe_gemm_checked(X, Wt, S, Z, Z != nullptr, sorted_token_ids, expert_ids,
                          num_tokens_post_padded, topk_weights, Y, T, k, E, N, K, B, x_row_div,
                          false, true, stream);
}

int w4a16_moe_gemm_swiglu_tiled(const uint16_t* X, const int32_t* Wt, const uint16_t* S,
                                const uint8_t* Z, const int32_t* sorted_token_ids,
                                const int32_t* expert_ids,
                                const int32_t* num_tokens_post_padded, uint16_t* A, int64_t T,
                                int32_t k, int32_t E, int64_t I, int64_t K, int32_t B,
                                int32_t x_row_div, void* stream) {
  if (I < 1) return W4_ERR_SHAPE;
  const int64_t N = I > kMaxI32 ? kMaxI32 + 1 : 2 * I;   // past the limit: unsupported
  return moe_gemm_checked(X, Wt, S, Z, Z != nullptr, sorted_token_ids, expert_ids,
                          num_tokens_post_padded, nullptr, A, T, k, E, N, K, B, x_row_div,
                          true, true, stream);
}

int w4_silu_mul(const uint16_t* H1, uint16_t* A, int64_t R, int64_t I, void* stream) {
  if (R < 0 || I < 0 || I % 2 != 0) return W4_ERR_SHAPE;
  if (R == 0 || I == 0) return W4_OK;
  if (!H1 || !A) return W4_ERR_NULL;
  if (!aligned(H1, 4) || !aligned(A, 4)) return W4_ERR_MISALIGNED;
  return hip_status(w4::launch_silu_mul(H1, A, R, I, as_stream(stream)));
}

int w4_moe_sum(const uint16_t* H2, const float* topk_weights, uint16_t* Out, int64_t T, int32_t k,
               int64_t H, void* stream) {
  if (T < 0 || k < 1 || H < 0 || H % 2 != 0) return W4_ERR_SHAPE;
  if (T == 0 || H == 0) return W4_OK;
  if (!H2 || !Out) return W4_ERR_NULL;
  if (!aligned(H2, 4) || !aligned(Out, 4) || !aligned(topk_weights, 4)) return W4_ERR_MISALIGNED;
  return hip_status(w4::launch_moe_sum(H2, topk_weights, Out, T, k, H, as_stream(stream)));
}

int w4_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                 float* topk_weights, void* stream) {
  if (T < 0 || E < 1 || k < 1) return W4_ERR_SHAPE;
  if (E > 1024 || k > 16 || k > E || T > kMaxI32) return W4_ERR_UNSUPPORTED;
  if (T == 0) return W4_OK;
  if (!logits || !topk_ids || !topk_weights) return W4_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return W4_ERR_MISALIGNED;
  return hip_status(w4::launch_route(logits, T, E, k, topk_ids, topk_weights, as_stream(stream)));
}

int64_t w4_moe_combine_workspace_words(int64_t T, int32_t k, int32_t E, int64_t N, int32_t B) {
  if (T < 0 || k < 1 || E < 1 || N < 1 || B < 1) return -1;
  return w4::moe_combine_counters(T, k, E, N, B);
}

}  // extern "C"

namespace {

// Checks of the fused combine's operands other than the counters: W4_OK,
// -1 for a valid call with nothing to do (T == 0), or an error status.
int combine_validate(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                     const int32_t* sorted_token_ids, const int32_t* expert_ids,
                     const int32_t* num_tokens_post_padded, const int32_t* topk_ids,
                     const float* topk_weights, uint16_t* H2, uint16_t* Out, int64_t T,
                     int32_t k, int32_t E, int64_t N, int64_t K, int32_t B, int32_t tiled) {
  const int v = moe_gemm_validate(A, Wq, S, nullptr, false, sorted_token_ids, expert_ids,
                                  num_tokens_post_padded, topk_weights, H2, T, k, E, N, K, B, 1,
                                  false, tiled != 0);
  if (v != W4_OK) return v;
  if (T * N >= ((int64_t)1 << 40) || k > 16) return W4_ERR_UNSUPPORTED;
  if (!topk_ids || !topk_weights || !Out) return W4_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(Out, 2)) return W4_ERR_MISALIGNED;
  return W4_OK;
}

}  // namespace

extern "C" {

int w4a16_moe_gemm_combine(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                           const int32_t* sorted_token_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded, const int32_t* topk_ids,
                           const float* topk_weights, uint16_t* H2, uint16_t* Out, int64_t T,
                           int32_t k, int32_t E, int64_t N, int64_t K, int32_t B, int32_t tiled,
                           int32_t* workspace, void* stream) {
  const int v = combine_validate(A, Wq, S, sorted_token_ids, expert_ids, num_tokens_post_padded,
                                 topk_ids, topk_weights, H2, Out, T, k, E, N, K, B, tiled);
  if (v < 0) return W4_OK;
  if (v != W4_OK) return v;
  if (!workspace) return W4_ERR_NULL;
  if (!aligned(workspace, 4)) return W4_ERR_MISALIGNED;
  return hip_status(w4::launch_moe_gemm_combine(A, Wq, S, sorted_token_ids, expert_ids,
                                                num_tokens_post_padded, topk_ids, topk_weights,
                                                H2, Out, workspace, T, k, E, N, K, B, tiled != 0,
                                                as_stream(stream)));
}

int w4a16_moe_gemm_combine_noalloc(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                   const int32_t* num_tokens_post_padded,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   uint16_t* H2, uint16_t* Out, int64_t T, int32_t k, int32_t E,
                                   int64_t N, int64_t K, int32_t B, int32_t tiled,
                                   void* stream) {
  const int v = combine_validate(A, Wq, S, sorted_token_ids, expert_ids, num_tokens_post_padded,
                                 topk_ids, topk_weights, H2, Out, T, k, E, N, K, B, tiled);
  if (v < 0) return W4_OK;
  if (v != W4_OK) return v;
  if (w4::moe_combine_counters(T, k, E, N, B) > w4::kCombineScratchWords)
    return W4_ERR_UNSUPPORTED;
  int32_t* words = nullptr;
  const hipError_t e = w4::combine_scratch(&words);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(w4::launch_moe_gemm_combine(A, Wq, S, sorted_token_ids, expert_ids,
                                                num_tokens_post_padded, topk_ids, topk_weights,
                                                H2, Out, words, T, k, E, N, K, B, tiled != 0,
                                                as_stream(stream)));
}

}  // extern "C"
