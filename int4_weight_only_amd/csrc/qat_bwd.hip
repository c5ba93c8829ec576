// Kernels of the QAT linear layer's gradients.
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

// ------------------------------------------------------------ transpose --
// AT[c, r] = A[r, c] for r < R, zero for R <= r < RP (A [R, C], AT [C, RP]).
// A workgroup of 256 threads moves a 64 x 64 tile through LDS (rows padded
// by 8 elements off the bank period).  VEC (C and RP multiples of 8, both
// buffers 16-byte aligned): 16-byte loads along A's rows and 16-byte stores
// along AT's rows; otherwise 2-byte accesses.
template <bool VEC>
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ A,
                                                        uint16_t* __restrict__ AT, int64_t R,
                                                        int64_t C, int64_t RP) {
  constexpr int TS = 64, PAD = 8;
  __shared__ __attribute__((aligned(16))) uint16_t tile[TS][TS + PAD];
  const int tid = threadIdx.x;
  const int64_t ntc = (C + TS - 1) / TS;
  const int64_t r0 = (int64_t)(blockIdx.x / ntc) * TS;
  const int64_t c0 = (int64_t)(blockIdx.x % ntc) * TS;
  if constexpr (VEC) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 32 * p + tid / 8, c = 8 * (tid % 8);
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (r0 + r < R && c0 + c < C) v = *(const u32x4*)(A + (r0 + r) * C + c0 + c);
      *(u32x4*)&tile[r][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = 32 * p + tid / 8, r = 8 * (tid % 8);
      if (c0 + c >= C || r0 + r >= RP) continue;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)tile[r + 2 * i][c] | ((uint32_t)tile[r + 2 * i + 1][c] << 16);
      *(u32x4*)(AT + (c0 + c) * RP + r0 + r) = u32x4{w[0], w[1], w[2], w[3]};
    }
  } else {
    for (int e = tid; e < TS * TS; e += 256) {
      const int r = e / TS, c = e % TS;
      tile[r][c] = (r0 + r < R && c0 + c < C) ? A[(r0 + r) * C + c0 + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int e = tid; e < TS * TS; e += 256) {
      const int c = e / TS, r = e % TS;
      if (c0 + c < C && r0 + r < RP) AT[(c0 + c) * RP + r0 + r] = tile[r][c];
    }
  }
}

hipError_t launch_transpose_bf16(const uint16_t* A, uint16_t* AT, int64_t R, int64_t C,
                                 int64_t RP, hipStream_t st) {
  const int64_t blocks = ((RP + 63) / 64) * ((C + 63) / 64);
  const bool vec = C % 8 == 0 && RP % 8 == 0 && (uintptr_t)A % 16 == 0 && (uintptr_t)AT % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(k_transpose_bf16<true>, dim3((unsigned)blocks), dim3(256), 0, st, A, AT, R,
                       C, RP);
  else
    hipLaunchKernelGGL(k_transpose_bf16<false>, dim3((unsigned)blocks), dim3(256), 0, st, A, AT,
                       R, C, RP);
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
// BM rows of A per workgroup, NWV waves as (BM / 128) x (NWV / (BM / 128))
// waves of 128 A rows x 64 B rows each, NST LDS stages.
template <int BM, int NWV, int NST>
__global__ __launch_bounds__(NWV * 64, 1) void k_bf16_gemm_nt(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ B,
                                                              uint16_t* __restrict__ C, int M,
                                                              int N, int K) {
  constexpr int KS = 64;                 // K per step
  constexpr int WA = BM / 128;           // waves along A
  constexpr int WB = NWV / WA;           // waves along B
  constexpr int BN = 64 * WB;
  constexpr int XA = BM / 8 / NWV;       // 1 KB loads per A stage per wave
  constexpr int XB = BN / 8 / NWV;       // ... per B stage per wave
  static_assert(NST == 2 || NST == 3, "stages");
  static_assert(XA * NWV * 8 == BM && XB * NWV * 8 == BN, "tile shape");
  // separately declared stages: each DMA target and each operand read names
  // one object
  __shared__ __attribute__((aligned(16))) uint16_t as0[BM * KS];
  __shared__ __attribute__((aligned(16))) uint16_t as1[BM * KS];
  __shared__ __attribute__((aligned(16))) uint16_t as2[NST > 2 ? BM * KS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t bs0[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t bs1[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[NST > 2 ? BN * KS : 8];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wa = wave / WB, wb = wave % WB;
  const int l32 = lane & 31, h = lane >> 5;
  // tile order: the 1-D grid is dispatched round-robin over the 8 XCDs;
  // XCD x walks the contiguous tile range [x per, (x + 1) per) in groups of
  // 8 A row-blocks, so co-running workgroups share rows in its L2
  const int mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  const int tiles = mt * nt;
  const int per = (tiles + 7) / 8;
  const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (t >= tiles) return;
  const int group = t / (8 * nt);
  const int gm = min(8, mt - group * 8);
  const int in_group = t - group * (8 * nt);
  const int m0 = (group * 8 + in_group % gm) * BM;
  const int n0 = (in_group / gm) * BN;

  const __amdgpu_buffer_rsrc_t ar = rsrc(A, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t br = rsrc(B, (uint32_t)N * (uint32_t)K * 2u);
  // Load I of a stage fills stage rows 8 I .. 8 I + 7: lane l writes the 16
  // bytes at slot l, row r = 8 I + l / 8, stored piece l % 8, which holds
  // the row's piece (l % 8) ^ ((r / 2) % 8).  Byte offset of the lane's
  // piece at step 0 (OOB for rows past the end) and its k within a step.
  auto row_off = [&](int first, int lim, int I) {
    const int r = 8 * I + (lane >> 3);
    const int pg = (lane & 7) ^ ((r >> 1) & 7);
    const int row = first + r;
    return row < lim ? ((uint32_t)row * (uint32_t)K + 8u * (uint32_t)pg) * 2u : kOOB;
  };
  auto piece_k = [&](int I) { return 8 * ((lane & 7) ^ (((8 * I + (lane >> 3)) >> 1) & 7)); };
  uint32_t aoff[XA], boff[XB];
#pragma unroll
  for (int i = 0; i < XA; ++i) aoff[i] = row_off(m0, M, wave * XA + i);
#pragma unroll
  for (int i = 0; i < XB; ++i) boff[i] = row_off(n0, N, wave * XB + i);
  auto load_stage = [&](int step, uint16_t* sa, uint16_t* sb) __attribute__((always_inline)) {
    const int k0 = step * KS;
#pragma unroll
    for (int i = 0; i < XA; ++i) {
      const uint32_t off = (aoff[i] != kOOB && k0 + piece_k(wave * XA + i) < K)
                               ? aoff[i] + (uint32_t)k0 * 2u
                               : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ar, (__attribute__((address_space(3))) void*)(sa + (wave * XA + i) * 512), 16, off, 0,
          0, 0);
    }
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const uint32_t off = (boff[i] != kOOB && k0 + piece_k(wave * XB + i) < K)
                               ? boff[i] + (uint32_t)k0 * 2u
                               : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          br, (__attribute__((address_space(3))) void*)(sb + (wave * XB + i) * 512), 16, off, 0,
          0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ms][ns][v] = 0.0f;

  const int nsteps = (K + KS - 1) / KS;
  // One step: wait until this wave's loads of this step's stage have landed
  // (the later stages' loads may stay in flight), a bare s_barrier so that
  // every wave's part is visible and every wave is done with the stage the
  // new loads overwrite, start the stage NST - 1 steps ahead, multiply.
  auto step_body = [&](int step, const uint16_t* sa, const uint16_t* sb, uint16_t* na,
                       uint16_t* nb) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NST - 2) * (XA + XB)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_stage(step + NST - 1, na, nb);   // past K: reads zero
    if (step < nsteps) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 a[4], b[2];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          const int R = wa * 128 + ms * 32 + l32;
          a[ms] = *(const u32x4*)(sa + R * KS + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
        }
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const int R = wb * 64 + ns * 32 + l32;
          b[ns] = *(const u32x4*)(sb + R * KS + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
        }
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
          for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = mfma32(a[ms], b[ns], acc[ms][ns]);
      }
    }
  };
  load_stage(0, as0, bs0);
  if constexpr (NST == 3) {
    load_stage(1, as1, bs1);
    for (int step = 0; step < nsteps; step += 3) {
      step_body(step + 0, as0, bs0, as2, bs2);
      step_body(step + 1, as1, bs1, as0, bs0);
      step_body(step + 2, as2, bs2, as1, bs1);
    }
  } else {
    for (int step = 0; step < nsteps; step += 2) {
      step_body(step + 0, as0, bs0, as1, bs1);
      step_body(step + 1, as1, bs1, as0, bs0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads past the end drained

  // lane holds D[8 (v / 4) + 4 h + v % 4][l32] of each 32 x 32 tile
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) {
    const int n = n0 + wb * 64 + ns * 32 + l32;
    if (n >= N) continue;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wa * 128 + ms * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < M) C[(int64_t)m * N + n] = to_bf16(acc[ms][ns][v]);
      }
  }
}

namespace {
template <int BM, int NWV, int NST>
hipError_t launch_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N,
                     int64_t K, hipStream_t st) {
  constexpr int BN = 64 * (NWV / (BM / 128));
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t blocks = (tiles + 7) / 8 * 8;   // whole rounds over the 8 XCDs
  hipLaunchKernelGGL((k_bf16_gemm_nt<BM, NWV, NST>), dim3((unsigned)blocks), dim3(NWV * 64), 0,
                     st, A, B, C, (int)M, (int)N, (int)K);
  return hipGetLastError();
}
}  // namespace

// 256 x 256 tiles of 8 waves (two per SIMD, two stages) when they fill
// every CU at least once: 440 -> 382 us on dY [4096, 14336] x W'^T
// [4096, 14336]; smaller products keep the 128 x 256 tile of 4 waves
// (three stages), which spreads them over more CUs.  Both sum each output
// in the same order, so the choice does not change a bit.
hipError_t launch_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                               int64_t N, int64_t K, hipStream_t st) {
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= cu_count()) return launch_nt<256, 8, 2>(A, B, C, M, N, K, st);
  return launch_nt<128, 4, 3>(A, B, C, M, N, K, st);
}

}  // namespace w4
