// Group-wise INT4 quantization (symmetric, and asymmetric with a zero
// point), packing and fake quantization.
//
// Method: "Quantization basics: from FP32 to INT4", §2.2 (z = 0,
// s = max|w| / q_max, q = clamp(round(w / s))) and §5 (round half to even,
// never a truncating cast); "Quantization-aware training" tag summary [11]
// (one scale per 1 x 32 group); "INT4 QAT end-to-end for RL" §3.2 (eight
// INT4 codes packed into one INT32) and §2.1 (fake quantization restores
// the weight to bf16 right after mapping it onto the INT4 grid).
//
// Mapping: one lane owns 8 consecutive elements (16 bytes in, one packed
// word out), four neighbouring lanes own one 32-element group.  The group
// maximum is combined across the quad with two DPP quad permutes, so every
// load and store is a contiguous, fully coalesced vector access and no LDS
// is used.  K % 32 == 0 makes groups tile the flattened [N*K] array, so the
// kernel works on flat word indices.
#include "common.h"

namespace w4 {

namespace {

// rint_half_even(w / s) for bf16 values w, s with s in [2^-110, 2^100],
// equal to rounding the IEEE fp32 quotient and then to an integer, in four
// VALU ops instead of a full IEEE division.  With r = rcp(s) (1 ulp):
//   y0 = w r  is w / s to ~2^-22 relative;
//   e  = w - y0 s  is exact (an fma; |e| needs ~11 bits on the grid of
//       y0 s, and that grid does not underflow for |w / s| >= 1/2 and
//       s >= 2^-110);
//   y1 = y0 + e r  is w / s to ~2^-42 absolute for |w / s| <= 16 (one
//       Newton correction of the quotient, as in Markstein's division).
// The rounded integer can only differ from that of the exact quotient where
// w / s is a half-integer or very close to one.  For bf16 operands w / s is
// either exactly a half-integer (a tie) or at least 2^-10 away from every
// half-integer (the distance is a nonzero integer over 4 * 2^8), so y1
// rounds to the tie exactly, rintf sends it to the even neighbour, and every
// other quotient rounds like the exact one.  Outside the range of s (and for
// s = 0) the callers divide.
__device__ __forceinline__ float rint_quot(float w, float s, float r) {
  const float y0 = w * r;
  const float e = __builtin_fmaf(-y0, s, w);
  return rintf(__builtin_fmaf(e, r, y0));
}

__device__ __forceinline__ bool quot_fast(float s) {
  return s >= 0x1p-110f && s <= 0x1p100f;
}

}  // namespace

// ASYM: "Quantization basics" §2.3 with the readings of the asymmetric
// oracle: unsigned grid [0, 15], range widened to contain 0,
// s = bf16(fp32(x_max - x_min) / 15), z = clamp(rint(-x_min / s), 0, 15),
// q = clamp(rint(w / s) + z, 0, 15), dequant bf16((q - z) s); z is one byte
// per group.  The scale is an IEEE fp32 division; every rint (half to even)
// of a quotient equals that of the IEEE fp32 quotient (rint_quot).
template <bool FAKE, bool ASYM>
__global__ __launch_bounds__(256) void k_quantize(const u32x4* __restrict__ W, int64_t words,
                                                  uint32_t* __restrict__ Wq,
                                                  uint16_t* __restrict__ S,
                                                  uint8_t* __restrict__ Z, u32x4* Wfq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // words % 4 == 0 and blocks start on multiples of 4, so a quad is either
  // entirely inside or entirely past the end: no DPP reads an exited lane.
  if (i >= words) return;
  const u32x4 v = W[i];
  const float w[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float s, zf = 0.0f, lo_g = 0.0f;
  uint16_t sb;
  if constexpr (!ASYM) {
    // For finite bf16, |w| orders like its 15-bit magnitude field.
    uint32_t a = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
    a = max(a, max(max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu), max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu)));
    a = max(a, quad_xor1(a));
    a = max(a, quad_xor2(a));
    const float amax = __uint_as_float(a << 16);
    sb = to_bf16(amax / 7.0f);                 // IEEE fp32 division, then RNE
    s = bf16f(sb);
  } else {
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      lo = fminf(lo, w[j]);
      hi = fmaxf(hi, w[j]);
    }
    lo = fminf(lo, __uint_as_float(quad_xor1(__float_as_uint(lo))));
    hi = fmaxf(hi, __uint_as_float(quad_xor1(__float_as_uint(hi))));
    lo = fminf(lo, __uint_as_float(quad_xor2(__float_as_uint(lo))));
    hi = fmaxf(hi, __uint_as_float(quad_xor2(__float_as_uint(hi))));
    lo = fminf(lo, 0.0f);                      // the grid always holds 0
    hi = fmaxf(hi, 0.0f);
    lo_g = lo;
    sb = to_bf16((hi - lo) / 15.0f);           // fp32 subtraction, IEEE division, RNE
    s = bf16f(sb);
  }
  // rint_even(w / s) for the group's elements (and the zero point's
  // rint_even(-lo / s)): the corrected reciprocal product where s allows,
  // else IEEE division
  float rq[8], rz = 0.0f;
  if (quot_fast(s)) {
    const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int j = 0; j < 8; ++j) rq[j] = rint_quot(w[j], s, r);
    if constexpr (ASYM) rz = rint_quot(0.0f - lo_g, s, r);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) rq[j] = rintf(w[j] / s);
    if constexpr (ASYM) rz = rintf((0.0f - lo_g) / s);
  }
  if constexpr (ASYM) zf = (s == 0.0f) ? 0.0f : fminf(fmaxf(rz, 0.0f), 15.0f);
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (!ASYM)
      q[j] = (s == 0.0f) ? 0.0f : fminf(fmaxf(rq[j], -8.0f), 7.0f);
    else
      q[j] = (s == 0.0f) ? 0.0f : fminf(fmaxf(rq[j] + zf, 0.0f), 15.0f);
  }
  if constexpr (!FAKE) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= ((uint32_t)(int)q[j] & 0xFu) << (4 * j);
    Wq[i] = word;
    if ((i & 3) == 0) {
      S[i >> 2] = sb;
      if constexpr (ASYM) Z[i >> 2] = (uint8_t)(int)zf;
    }
  } else {
    // (q - z) * s is exact in fp32; one rounding to bf16.  Adding +0 turns
    // the -0 that rintf gives for small negative w into the code's +0.
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = (q[j] - zf) + 0.0f;
    u32x4 o;
    o.x = pk_bf16(q[0] * s, q[1] * s);
    o.y = pk_bf16(q[2] * s, q[3] * s);
    o.z = pk_bf16(q[4] * s, q[5] * s);
    o.w = pk_bf16(q[6] * s, q[7] * s);
    Wfq[i] = o;
  }
}

hipError_t launch_quantize(const uint16_t* W, int64_t words, int32_t* Wq, uint16_t* S,
                           uint8_t* Z, uint16_t* Wfq, bool fake, bool asym, hipStream_t st) {
  const int64_t blocks = (words + 255) / 256;
  const dim3 g((unsigned)blocks), b(256);
  const u32x4* w = (const u32x4*)W;
  if (fake && asym)
    hipLaunchKernelGGL((k_quantize<true, true>), g, b, 0, st, w, words, nullptr, nullptr, nullptr,
                       (u32x4*)Wfq);
  else if (fake)
    hipLaunchKernelGGL((k_quantize<true, false>), g, b, 0, st, w, words, nullptr, nullptr,
                       nullptr, (u32x4*)Wfq);
  else if (asym)
    hipLaunchKernelGGL((k_quantize<false, true>), g, b, 0, st, w, words, (uint32_t*)Wq, S, Z,
                       nullptr);
  else
    hipLaunchKernelGGL((k_quantize<false, false>), g, b, 0, st, w, words, (uint32_t*)Wq, S,
                       nullptr, nullptr);
  return hipGetLastError();
}

// Packed codes back to bf16 weights, the values fake quantization gives:
// W'[n, k] = bf16(q s) (ASYM: bf16((q - z) s)), with the 17-op dequant of the
// W4A16 products (exact product, one rounding).  One lane per packed word:
// a 4-byte load, the group's scale (and zero point) shared by its four
// lanes, one 16-byte store.
// The 17-op step computes (1024 + n) s + c0 with c0 = -(1032 or 1024 + z) s,
// which overflows fp32 for s above about 3e35 (2^118); such groups take the
// direct product q * s (exact in fp32 as well).
template <bool ASYM>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ Wq,
                                                 const uint16_t* __restrict__ S,
                                                 const uint8_t* __restrict__ Z,
                                                 u32x4* __restrict__ W, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= words) return;
  const uint32_t w = Wq[i];
  const float s = bf16f(S[i >> 2]);
  const float z = ASYM ? (float)Z[i >> 2] : 0.0f;
  if (s <= 0x1p100f) {
    W[i] = dequant8<ASYM>(w, ASYM ? deq_scale_zp(s, z) : deq_scale(s));
  } else {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = ASYM ? (float)((w >> (4 * j)) & 0xFu) - z
                           : (float)((int32_t)(w << (28 - 4 * j)) >> 28);
      v[j] = q * s;
    }
    W[i] = u32x4{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]), pk_bf16(v[4], v[5]),
                 pk_bf16(v[6], v[7])};
  }
}

hipError_t launch_dequant(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, uint16_t* W,
                          int64_t words, hipStream_t st) {
  const dim3 g((unsigned)((words + 255) / 256)), b(256);
  if (Z != nullptr)
    hipLaunchKernelGGL(k_dequant<true>, g, b, 0, st, (const uint32_t*)Wq, S, Z, (u32x4*)W, words);
  else
    hipLaunchKernelGGL(k_dequant<false>, g, b, 0, st, (const uint32_t*)Wq, S, nullptr,
                       (u32x4*)W, words);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_bf16(uint16_t* __restrict__ Y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    Y[i] = 0;
}

hipError_t launch_zero_bf16(uint16_t* Y, int64_t n, hipStream_t st) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_zero_bf16, dim3((unsigned)blocks), dim3(256), 0, st, Y, n);
  return hipGetLastError();
}

}  // namespace w4
