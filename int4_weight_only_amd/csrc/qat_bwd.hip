// Kernels of the QAT linear layer's input gradient.
//
// Method: "INT4 QAT end-to-end for RL" §2.1 -- the forward multiplies the
// fake-quantized weight W' = bf16(q s) and the straight-through estimator
// passes the gradient through the rounding, so the input gradient is
// dX = dY W' (W' [N, K], dY [M, N]).  The library computes it in two calls
// on the packed codes: w4_dequant_t writes W'^T [K, N] (the dequantized
// weight, transposed, bit-exact with fake quantization), and
// w4_bf16_gemm_nt multiplies dY by it with fp32 accumulation.
#include "common.h"

namespace w4 {

namespace {

constexpr uint32_t kOOB = 0x80000000u;  // byte offset past any buffer: reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 8 bf16 of one packed word, as w4_dequant computes them (the 17-op step,
// or the direct product for scales above 2^100).
template <bool ASYM>
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, float s, float z) {
  if (s <= 0x1p100f) return dequant8<ASYM>(w, ASYM ? deq_scale_zp(s, z) : deq_scale(s));
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = ASYM ? (float)((w >> (4 * j)) & 0xFu) - z
                         : (float)((int32_t)(w << (28 - 4 * j)) >> 28);
    v[j] = q * s;
  }
  return u32x4{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]), pk_bf16(v[4], v[5]),
               pk_bf16(v[6], v[7])};
}

}  // namespace

// ------------------------------------------------------------ dequant_t --
// WT[k, n] = W'[n, k].  A workgroup of 256 threads takes 64 rows x 128
// columns of W': thread t dequantizes words (n0 + t % 64, w0 + t / 64 + 4 i),
// i = 0..3, into an LDS tile stored [k][n] (a wave writes 64 consecutive n
// of one k: one 128-byte LDS row), then writes 16-byte pieces of WT rows.
template <bool ASYM>
__global__ __launch_bounds__(256) void k_dequant_t(const uint32_t* __restrict__ Wq,
                                                   const uint16_t* __restrict__ S,
                                                   const uint8_t* __restrict__ Z,
                                                   uint16_t* __restrict__ WT, int64_t N,
                                                   int64_t K) {
  constexpr int TN = 64, TK = 128, PAD = 8;           // LDS row: 64 bf16 + pad
  __shared__ __attribute__((aligned(16))) uint16_t tile[TK][TN + PAD];
  const int tid = threadIdx.x;
  const int64_t ntn = (N + TN - 1) / TN;
  const int64_t n0 = (int64_t)(blockIdx.x % ntn) * TN;
  const int64_t k0 = (int64_t)(blockIdx.x / ntn) * TK;
  const int64_t kw = K / 8, G = K / 32;
  const int nl = tid % TN;
  const int64_t n = n0 + nl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int wl = tid / TN + 4 * i;                   // word of the tile row: 0..15
    const int64_t w = k0 / 8 + wl;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (n < N && w < kw) {
      const int64_t g = w / 4;
      v = dequant_word<ASYM>(Wq[n * kw + w], bf16f(S[n * G + g]),
                             ASYM ? (float)Z[n * G + g] : 0.0f);
    }
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[8 * wl + 2 * j][nl] = (uint16_t)(d[j] & 0xFFFFu);
      tile[8 * wl + 2 * j + 1][nl] = (uint16_t)(d[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kl = tid / 8 + 32 * i;                   // tile row 0..127
    const int c = tid % 8;                             // 8-column piece
    const int64_t k = k0 + kl;
    const int64_t nc = n0 + 8 * c;
    if (k >= K || nc >= N) continue;
    uint16_t* dst = WT + k * N + nc;
    const uint16_t* src = &tile[kl][8 * c];
    if (nc + 8 <= N && ((N & 7) == 0)) {
      *(u32x4*)dst = *(const u32x4*)src;
    } else {
      for (int j = 0; j < 8 && nc + j < N; ++j) dst[j] = src[j];
    }
  }
}

hipError_t launch_dequant_t(const int32_t* Wq, const uint16_t* S, const uint8_t* Z, uint16_t* WT,
                            int64_t N, int64_t K, hipStream_t st) {
  const int64_t blocks = ((N + 63) / 64) * ((K + 127) / 128);
  if (Z != nullptr)
    hipLaunchKernelGGL(k_dequant_t<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint32_t*)Wq, S, Z, WT, N, K);
  else
    hipLaunchKernelGGL(k_dequant_t<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint32_t*)Wq, S, nullptr, WT, N, K);
  return hipGetLastError();
}

// --------------------------------------------------------- bf16 NT GEMM --
// C[M, N] = bf16( sum_k A[m, k] B[n, k] ), fp32 accumulation in a fixed
// order (k ascending in 16-wide MFMA slices).  A workgroup of 4 waves takes
// 128 x 128 of C; wave (wm, wn) 64 x 64 as 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16.  Lane (r = l % 32, h = l / 32) loads the 16
// bytes k = 16 s + 8 h .. + 7 of its A row and B row straight into the
// operand registers (raw buffer loads; rows past the end and k past K read
// zero), the next 32-wide step's operands in flight while the MFMAs of the
// current one run.  K % 8 == 0 (16-byte rows pieces).
__global__ __launch_bounds__(256, 2) void k_bf16_gemm_nt(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ B,
                                                         uint16_t* __restrict__ C, int M, int N,
                                                         int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int ntn = (N + 127) / 128;
  const int tm = blockIdx.x / ntn, tn = blockIdx.x % ntn;
  const int m0 = tm * 128 + (wave >> 1) * 64;
  const int n0 = tn * 128 + (wave & 1) * 64;
  const __amdgpu_buffer_rsrc_t ar = rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(B, (uint32_t)N * (uint32_t)K * 2u);
  uint32_t arow[2], brow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 32 * i + l32, n = n0 + 32 * i + l32;
    arow[i] = m < M ? (uint32_t)m * (uint32_t)K * 2u : kOOB;
    brow[i] = n < N ? (uint32_t)n * (uint32_t)K * 2u : kOOB;
  }
  auto off = [&](uint32_t row, int k) { return (row != kOOB && k < K) ? row + 2u * k : kOOB; };
  auto load = [&](int step, u32x4 (&a)[2][2], u32x4 (&b)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = 32 * step + 16 * s + 8 * h;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[s][i] = __builtin_amdgcn_raw_buffer_load_b128(ar, off(arow[i], k), 0, 0);
        b[s][i] = __builtin_amdgcn_raw_buffer_load_b128(br, off(brow[i], k), 0, 0);
      }
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto mma = [&](const u32x4 (&a)[2][2], const u32x4 (&b)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[s][i], b[s][j], acc[i][j]);
  };
  const int nsteps = (K + 31) / 32;
  u32x4 a0[2][2], b0[2][2], a1[2][2], b1[2][2];
  load(0, a0, b0);
  for (int step = 0; step < nsteps; step += 2) {
    load(step + 1, a1, b1);            // past K: reads zero
    mma(a0, b0);
    if (step + 1 >= nsteps) break;
    load(step + 2, a0, b0);
    mma(a1, b1);
  }
  // lane holds D[8 (v / 4) + 4 h + v % 4][l32] of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * j + l32;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M) C[(int64_t)m * N + n] = to_bf16(acc[i][j][v]);
      }
    }
}

hipError_t launch_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, hipStream_t st) {
  const int64_t blocks = ((M + 127) / 128) * ((N + 127) / 128);
  hipLaunchKernelGGL(k_bf16_gemm_nt, dim3((unsigned)blocks), dim3(256), 0, st, A, B, C, (int)M,
                     (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace w4
