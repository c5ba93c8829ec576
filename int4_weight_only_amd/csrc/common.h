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

// Byte b of a 32-bit word as fp32 (v_cvt_f32_ubyteN).  Pure VALU op; the
// asm keeps the compiler from re-deriving each byte with a bitfield extract.
#define W4_CVT_UBYTE(N)                                                      \
  __device__ __forceinline__ float ubyte##N(uint32_t x) {                    \
    float r;                                                                 \
    asm("v_cvt_f32_ubyte" #N " %0, %1" : "=v"(r) : "v"(x));                  \
    return r;                                                                \
  }
W4_CVT_UBYTE(0)
W4_CVT_UBYTE(1)
W4_CVT_UBYTE(2)
W4_CVT_UBYTE(3)
#undef W4_CVT_UBYTE

// Eight INT4 codes of one packed word -> eight bf16 w' = bf16_rne(q * s),
// in k order (element j of the word -> bf16 j of the result: word x holds
// j = 0, 1, word y holds 2, 3, ...).
//   off = w ^ 0x88888888 turns each two's-complement nibble q into q + 8;
//   (q + 8) as fp32 comes from a byte convert; fma(q + 8, s, -8 s) = q * s
//   exactly (a 4-bit integer times an 8-bit-mantissa scale fits in fp32),
//   so the only rounding is the final bf16 one.
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s, float m8s) {
  const uint32_t off = w ^ 0x88888888u;
  const uint32_t lo = off & 0x0F0F0F0Fu;          // j = 0, 2, 4, 6
  const uint32_t hi = (off >> 4) & 0x0F0F0F0Fu;   // j = 1, 3, 5, 7
  u32x4 r;
  r.x = pk_bf16(__builtin_fmaf(ubyte0(lo), s, m8s), __builtin_fmaf(ubyte0(hi), s, m8s));
  r.y = pk_bf16(__builtin_fmaf(ubyte1(lo), s, m8s), __builtin_fmaf(ubyte1(hi), s, m8s));
  r.z = pk_bf16(__builtin_fmaf(ubyte2(lo), s, m8s), __builtin_fmaf(ubyte2(hi), s, m8s));
  r.w = pk_bf16(__builtin_fmaf(ubyte3(lo), s, m8s), __builtin_fmaf(ubyte3(hi), s, m8s));
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
hipError_t launch_quantize(const uint16_t* W, int64_t words, int32_t* Wq, uint16_t* S,
                           uint16_t* Wfq, bool fake, hipStream_t st);
hipError_t launch_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_moe_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* ntpp, const float* topk_w, uint16_t* Y, int64_t T,
                           int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                           int32_t x_row_div, hipStream_t st);
hipError_t launch_align(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t B,
                        int64_t cap, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                        hipStream_t st);
hipError_t launch_silu_mul(const uint16_t* H1, uint16_t* A, int64_t R, int64_t I, hipStream_t st);
hipError_t launch_moe_sum(const uint16_t* H2, const float* w, uint16_t* Out, int64_t T, int32_t k,
                          int64_t H, hipStream_t st);
hipError_t launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                        float* w, hipStream_t st);
hipError_t launch_zero_bf16(uint16_t* Y, int64_t n, hipStream_t st);
}  // namespace w4
