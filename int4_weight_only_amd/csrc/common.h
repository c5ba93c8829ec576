// Internal device helpers shared by the HIP kernels of libw4a16.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, v_cvt_pk_bf16_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));

constexpr int kGroup = 32;   // elements per scale along K
constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 ----

// Two fp32 -> packed bf16 pair (lo = a, hi = b), round to nearest even,
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float a) {
  return (uint16_t)(pk_bf16(a, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// ------------------------------------------------------------- dequant ----

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Per-group constants of dequant8: s, -1032 s and -72 s.  Both products are
// exact in fp32 (an 8-bit-mantissa scale times a constant whose set bits
// span at most 8 places).
struct DeqScale {
  float s, c0, c1;
};
__device__ __forceinline__ DeqScale deq_scale(float s) { return {s, -1032.0f * s, -72.0f * s}; }

// Zero-point codes (unsigned q in [0, 15], w' = bf16((q - z) s)): the same
// operation without the nibble flip, with c0 = -(1024 + z) s and
// c1 = -(64 + z) s (exact: at most 11 and 7 significant bits times s).
__device__ __forceinline__ DeqScale deq_scale_zp(float s, float z) {
  return {s, -(1024.0f + z) * s, -(64.0f + z) * s};
}

// Eight INT4 codes of one packed word -> eight bf16 w' = bf16_rne(q * s),
// in k order (element j of the word -> bf16 j of the result: word x holds
// j = 0, 1, word y holds 2, 3, ...).
//   A nibble t (two's complement, q = t < 8 ? t : t - 16) sits in the
//   mantissa of an fp16 whose other bits are those of 1024.0 (nibble at
//   bits 0..3 of a half: mantissa unit 1) or of 64.0 (nibble at bits 4..7:
//   mantissa unit 1/16).  One v_bitop3 computes (w & mask) ^ magic for two
//   nibbles at once, the XOR flipping the nibble's top bit, so the fp16
//   values are 1024 + (q + 8) resp. 64 + (q + 8).  v_fma_mix_f32 widens
//   that fp16 exactly and computes (1024 + q + 8) s - 1032 s, resp.
//   (64 + q + 8) s - 72 s, i.e. q * s; it is exact (a 4-bit integer times
//   an 8-bit-mantissa scale fits in fp32), so the only rounding is the
//   final bf16 one.
// 17 VALU ops for 8 weights: one shift, four bitop3, eight fma_mix, four
// v_cvt_pk_bf16_f32.  UNSIGNED: zero-point codes, no flip (plain magics)
// and the constants of deq_scale_zp.
template <bool UNSIGNED = false>
__device__ __forceinline__ u32x4 dequant8(uint32_t w, const DeqScale& d) {
  constexpr uint32_t kLo = UNSIGNED ? 0x64006400u : 0x64086408u;   // 1024 (+ 8: flip)
  constexpr uint32_t kHi = UNSIGNED ? 0x54005400u : 0x54805480u;   // 64 (+ 8/16 units: flip)
  const uint32_t w8 = w >> 8;
  const f16x2 a = __builtin_bit_cast(f16x2, (w & 0x000F000Fu) ^ kLo);    // j = 0, 4
  const f16x2 b = __builtin_bit_cast(f16x2, (w & 0x00F000F0u) ^ kHi);    // j = 1, 5
  const f16x2 c = __builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) ^ kLo);   // j = 2, 6
  const f16x2 e = __builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) ^ kHi);   // j = 3, 7
  u32x4 r;
  r.x = pk_bf16(__builtin_fmaf((float)a.x, d.s, d.c0), __builtin_fmaf((float)b.x, d.s, d.c1));
  r.y = pk_bf16(__builtin_fmaf((float)c.x, d.s, d.c0), __builtin_fmaf((float)e.x, d.s, d.c1));
  r.z = pk_bf16(__builtin_fmaf((float)a.y, d.s, d.c0), __builtin_fmaf((float)b.y, d.s, d.c1));
  r.w = pk_bf16(__builtin_fmaf((float)c.y, d.s, d.c0), __builtin_fmaf((float)e.y, d.s, d.c1));
  return r;
}

// ---------------------------------------------------------------- MFMA ----

// D[16x16] += A[16x32] * B[32x16] (bf16 in, fp32 accumulate).
// Lane l supplies A row (l % 16) and B column (l % 16), 8 values each at
// K slots 8*(l/16) .. +7; it receives D[4*(l/16) + r][l % 16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D[32x32] += A[32x16] * B[16x32].  Lane l supplies A row (l % 32) and B
// column (l % 32), 8 values at K slots 8*(l/32) .. +7; it receives
// D[8*(v/4) + 4*(l/32) + (v%4)][l % 32] in element v = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ----------------------------------------------------------------- DPP ----

// SwiGLU of one element, fp32: silu(g) * u = g / (1 + e^-g) * u.  One
// definition for the standalone kernel and the fused GEMM epilogue, so both
// round identically.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Value from lane (l ^ 1) / (l ^ 2) inside each group of four lanes.
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

}  // namespace w4

// --------------------------------------------------- host-side launchers ----
// Implemented in the .hip files; called by api.hip after validation.
namespace w4 {
// compute units of the current device (cached per device; 256 if unknown)
int cu_count();
hipError_t launch_quantize(const uint16_t* W, int64_t words, int32_t* Wq, uint16_t* S,
                           uint8_t* Z, uint16_t* Wfq, bool fake, bool asym, hipStream_t st);
// packed codes -> bf16 weights (Z == nullptr: symmetric codes)
hipError_t launch_dequant(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, uint16_t* W,
                          int64_t words, hipStream_t st);
hipError_t launch_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st);
// zero-point weights (unsigned codes, Z uint8 [N, K/32])
hipError_t launch_gemm_zp(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st);
hipError_t launch_gemv_zp(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st);
// grouped products: Z == nullptr for symmetric codes, else Z [E, N, K/32]
hipError_t launch_moe_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* ntpp, const float* topk_w, uint16_t* Y, int64_t T,
                           int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                           int32_t x_row_div, bool tiled, hipStream_t st);
hipError_t launch_moe_gemm_swiglu(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                                  const uint8_t* Z, const int32_t* sorted_ids,
                                  const int32_t* expert_ids,
                                  const int32_t* ntpp, uint16_t* A, int64_t T, int32_t k,
                                  int32_t E, int64_t I, int64_t K, int32_t B, int32_t x_row_div,
                                  bool tiled, hipStream_t st);
// Slots of the grouped GEMM, and its workgroups (N-tiles x slots, a 1-D grid).
int64_t moe_gemm_slots(int64_t T, int32_t k, int32_t E, int32_t B);
int64_t moe_gemm_workgroups(int64_t T, int32_t k, int32_t E, int64_t N, int32_t B, bool swiglu);
hipError_t launch_moe_gemm_combine(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                                   const int32_t* sorted_ids, const int32_t* expert_ids,
                                   const int32_t* ntpp, const int32_t* topk_ids,
                                   const float* topk_w, uint16_t* H2, uint16_t* Out, int32_t* cnt,
                                   int64_t T, int32_t k, int32_t E, int64_t N, int64_t K,
                                   int32_t B, bool tiled, hipStream_t st);
int64_t moe_combine_counters(int64_t T, int32_t k, int32_t E, int64_t N, int32_t B);
// The library's own counters for the allocation-free fused combine: the
// current device's copy (looked up once per device).
constexpr int64_t kCombineScratchWords = (int64_t)1 << 18;
hipError_t combine_scratch(int32_t** words);
hipError_t launch_align(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t B,
                        int64_t cap, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                        hipStream_t st);
hipError_t launch_silu_mul(const uint16_t* H1, uint16_t* A, int64_t R, int64_t I, hipStream_t st);
hipError_t launch_moe_sum(const uint16_t* H2, const float* w, uint16_t* Out, int64_t T, int32_t k,
                          int64_t H, hipStream_t st);
hipError_t launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                        float* w, hipStream_t st);
hipError_t launch_zero_bf16(uint16_t* Y, int64_t n, hipStream_t st);
// kernel-order code layout: int32 words of one [N, K] matrix, and the
// conversion canonical -> kernel order (restore: back) of E stacked matrices
int64_t tiled_words(int64_t N, int64_t K);
hipError_t launch_relayout(const int32_t* src, int32_t* dst, int64_t E, int64_t N, int64_t K,
                           bool restore, hipStream_t st);
// kernel-order layout of per-group values (scales: 2 bytes, zero points: 1)
int64_t tiled_group_elems(int64_t N, int64_t K);
hipError_t launch_relayout_groups(const void* src, void* dst, int elem_bytes, int64_t E,
                                  int64_t N, int64_t K, bool restore, hipStream_t st);
// QAT input gradient: transposed dequant W'^T [K, N], and a bf16 NT GEMM
hipError_t launch_dequant_t(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, uint16_t* WT,
                            int64_t N, int64_t K, hipStream_t st);
// AT [C, RP] = A [R, C]^T, rows R .. RP - 1 of AT's columns zero
hipError_t launch_transpose_bf16(const uint16_t* A, uint16_t* AT, int64_t R, int64_t C,
                                 int64_t RP, hipStream_t st);
hipError_t launch_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, hipStream_t st);
// products on either layout (Z == nullptr: symmetric codes)
hipError_t launch_gemv_any(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                           bool tiled, hipStream_t st);
hipError_t launch_gemm_any(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                           bool tiled, hipStream_t st);
}  // namespace w4
