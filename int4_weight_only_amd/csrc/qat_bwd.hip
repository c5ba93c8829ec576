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
// order.  Tile (MI355X): a workgroup of 4 waves takes 128 rows of A x 256
// rows of B (one workgroup per CU); wave w owns B rows [64 w, 64 w + 64)
// and all 128 A rows, as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (128
// accumulator registers), so every operand read from LDS feeds 2 or 4
// MFMAs.  K advances 64 per step; both operands go straight from memory into
// LDS (16-byte buffer_load ... lds, three stages: two steps ahead, no staging
// registers), each 64-element row stored as eight 16-byte pieces
// XOR-swizzled by (row / 2) % 8 so that the MFMA operand reads of 32 rows
// spread over the banks.  Lane (r = l % 32, h = l / 32) reads elements
// 32 h + 8 j .. + 7 of its row for MFMA j of a step -- the same k
// permutation for A and B, which leaves each dot product's terms unchanged;
// the fp32 additions run step by step, MFMA j in order.  Rows past M or N
// and k past K read zero.  K % 8 == 0 (16-byte row pieces).
namespace {
constexpr int kNtBM = 128, kNtBN = 256, kNtK = 64, kNtStages = 3;
constexpr int kNtXA = kNtBM / 8 / 4;    // 1 KB loads per A stage per wave
constexpr int kNtXB = kNtBN / 8 / 4;    // ... per B stage per wave
}  // namespace

__global__ __launch_bounds__(256, 1) void k_bf16_gemm_nt(const uint16_t* __restrict__ A,
                                                         const uint16_t* __restrict__ B,
                                                         uint16_t* __restrict__ C, int M, int N,
                                                         int K) {
  // separately declared stages: each DMA target and each operand read names
  // one object
  __shared__ __attribute__((aligned(16))) uint16_t as0[kNtBM * kNtK];
  __shared__ __attribute__((aligned(16))) uint16_t as1[kNtBM * kNtK];
  __shared__ __attribute__((aligned(16))) uint16_t as2[kNtBM * kNtK];
  __shared__ __attribute__((aligned(16))) uint16_t bs0[kNtBN * kNtK];
  __shared__ __attribute__((aligned(16))) uint16_t bs1[kNtBN * kNtK];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[kNtBN * kNtK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  // tile order: the 1-D grid is dispatched round-robin over the 8 XCDs;
  // XCD x walks the contiguous tile range [x per, (x + 1) per) in groups of
  // 8 A row-blocks, so co-running workgroups share rows in its L2
  const int mt = (M + kNtBM - 1) / kNtBM, nt = (N + kNtBN - 1) / kNtBN;
  const int tiles = mt * nt;
  const int per = (tiles + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= tiles) return;
  const int group = t / (8 * nt);
  const int gm = min(8, mt - group * 8);
  const int in_group = t - group * (8 * nt);
  const int m0 = (group * 8 + in_group % gm) * kNtBM;
  const int n0 = (in_group / gm) * kNtBN;

  const __amdgpu_buffer_rsrc_t ar = rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(B, (uint32_t)N * (uint32_t)K * 2u);
  // Load i of this wave fills stage rows 8 (wave X + i) .. + 7: lane l
  // writes the 16 bytes at slot l, row r = 8 I + l / 8, stored piece l % 8,
  // which holds the row's piece (l % 8) ^ ((r / 2) % 8).  Byte offset of the
  // lane's piece at step 0, or OOB for rows past the end.
  auto row_off = [&](int first, int lim, int i) {
    const int r = 8 * i + (lane >> 3);
    const int pg = (lane & 7) ^ ((r >> 1) & 7);
    const int row = first + r;
    return row < lim ? ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)pg) * 2u : kOOB;
  };
  uint32_t aoff[kNtXA], boff[kNtXB];
  int acol[kNtXA], bcol[kNtXB];   // k of the lane's piece within a step
#pragma unroll
  for (int i = 0; i < kNtXA; ++i) {
    const int I = wave * kNtXA + i;
    aoff[i] = row_off(m0, M, I);
    acol[i] = 8 * ((lane & 7) ^ (((8 * I + (lane >> 3)) >> 1) & 7));
  }
#pragma unroll
  for (int i = 0; i < kNtXB; ++i) {
    const int I = wave * kNtXB + i;
    boff[i] = row_off(n0, N, I);
    bcol[i] = 8 * ((lane & 7) ^ (((8 * I + (lane >> 3)) >> 1) & 7));
  }
  auto load_stage = [&](int step, uint16_t* sa, uint16_t* sb) __attribute__((always_inline)) {
    const int k0 = step * kNtK;
#pragma unroll
    for (int i = 0; i < kNtXA; ++i) {
      const uint32_t off =
          (aoff[i] != kOOB && k0 + acol[i] < K) ? aoff[i] + (uint32_t)k0 * 2u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ar, (__attribute__((address_space(3))) void*)(sa + (wave * kNtXA + i) * 512), 16, off,
          0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kNtXB; ++i) {
      const uint32_t off =
          (boff[i] != kOOB && k0 + bcol[i] < K) ? boff[i] + (uint32_t)k0 * 2u : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          br, (__attribute__((address_space(3))) void*)(sb + (wave * kNtXB + i) * 512), 16, off,
          0, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ms][ns][v] = 0.0f;

  const int nsteps = (K + kNtK - 1) / kNtK;
  // One step: wait until this wave's loads of this step's stage have landed
  // (the next stage's loads may stay in flight), a bare s_barrier so that
  // every wave's part is visible and every wave is done with the stage the
  // new loads overwrite, start the stage two steps ahead, multiply.
  auto step_body = [&](int step, const uint16_t* sa, const uint16_t* sb, uint16_t* na,
                       uint16_t* nb) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kNtXA + kNtXB) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_stage(step + 2, na, nb);   // past K: reads zero
    if (step < nsteps) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 a[4], b[2];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const int R = ms * 32 + l32;
          a[ms] = *(const u32x4*)(sa + R * kNtK + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
        }
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const int R = wave * 64 + ns * 32 + l32;
          b[ns] = *(const u32x4*)(sb + R * kNtK + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
        }
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
          for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = mfma32(a[ms], b[ns], acc[ms][ns]);
      }
    }
  };
  load_stage(0, as0, bs0);
  load_stage(1, as1, bs1);
  for (int step = 0; step < nsteps; step += kNtStages) {
    step_body(step + 0, as0, bs0, as2, bs2);
    step_body(step + 1, as1, bs1, as0, bs0);
    step_body(step + 2, as2, bs2, as1, bs1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads past the end drained

  // lane holds D[8 (v / 4) + 4 h + v % 4][l32] of each 32 x 32 tile
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) {
    const int n = n0 + wave * 64 + ns * 32 + l32;
    if (n >= N) continue;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + ms * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M) C[(int64_t)m * N + n] = to_bf16(acc[ms][ns][v]);
      }
  }
}

hipError_t launch_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = ((M + kNtBM - 1) / kNtBM) * ((N + kNtBN - 1) / kNtBN);
  const int64_t blocks = (tiles + 7) / 8 * 8;   // whole rounds over the 8 XCDs
  hipLaunchKernelGGL(k_bf16_gemm_nt, dim3((unsigned)blocks), dim3(256), 0, st, A, B, C, (int)M,
                     (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace w4
