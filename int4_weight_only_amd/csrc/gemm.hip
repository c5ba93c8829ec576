// W4A16 product for large M (prefill) and the grouped MoE expert GEMM.
//
// Method: "INT4 QAT end-to-end for RL" §4 -- INT4 weights dequantized in
// registers and fed to BF16 matrix units (the write-up's GPUs lack INT4
// tensor cores; so does this path: MI355X bf16 MFMA), fp32 accumulation
// ("Quantization basics: from FP32 to INT4" §5 (3): the accumulator must
// be wide); and the fused MoE of the same section, where the rows of one
// expert, gathered by moe_align_block_size, share one weight tile.
//
// Tile (MI355X): a workgroup of NW waves computes BM activation rows x
// NW*WN weight rows.  Each wave owns WN weight rows and all BM activation
// rows, so every weight is loaded from HBM and dequantized exactly once
// per workgroup, straight into the MFMA B operand (no LDS round trip),
// and the VALU cost of dequantization (about 3 ops per weight) is spread
// over BM rows of MFMA work.  Activations are staged through LDS, double
// buffered, rows padded to 144 bytes so 16-byte reads of eight
// consecutive rows hit distinct banks.  K advances 64 per step: lane
// (n = l % 32, h = l / 32) loads the whole 32-element group 2c + h of
// weight row n (16 bytes, one scale) and word j of it feeds MFMA j
// (v_mfma_f32_32x32x16_bf16); the activation operand is read with the
// same K permutation, which leaves the sum unchanged.
#include "common.h"

namespace w4 {

namespace {

constexpr int kStepK = 64;            // K per pipeline step (two groups)
constexpr int kRowPad = kStepK + 8;   // LDS row length in bf16 (144 bytes)
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past any buffer: reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

}  // namespace

// MOE = false: dense.  Rows r of the tile are activation rows m0 + r.
// MOE = true: the workgroup leads a run of alignment blocks of one expert;
// row r of the run is pair f = sorted_ids[row0 + r] (valid if f < n_pairs),
// activation row f / x_row_div, output row f.
template <int BM, int WN, int NW, bool MOE>
__global__ __launch_bounds__(NW * 64, 2) void k_gemm(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Wq, const uint16_t* __restrict__ S,
    uint16_t* __restrict__ Y, int M, int N, int K, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ ntpp,
    const float* __restrict__ topk_w, int n_pairs, int B, int x_row_div, int E) {
  constexpr int NT = NW * 64;
  constexpr int MS = BM / 32;          // 32-row MFMA tiles along M
  constexpr int NS = WN / 32;          // 32-col MFMA tiles along N per wave
  constexpr int PIECES = BM * (kStepK / 8) / NT;   // 16-byte X pieces per thread per step
  static_assert(BM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert((BM * (kStepK / 8)) % NT == 0, "X staging must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][kRowPad];
  __shared__ int xrow[BM];     // activation row of each tile row (-1: none)
  __shared__ int orow[BM];     // output row of each tile row (-1: none)
  __shared__ int run_info[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int n_base = blockIdx.x * (NW * WN) + wave * WN;
  const int G = K >> 5;
  const int kw = K >> 3;

  int rows_total;              // rows handled by this workgroup (all passes)
  int row0 = 0;                // MoE: first sorted slot of the run
  int expert = 0;
  if constexpr (MOE) {
    if (tid == 0) {
      const int b = blockIdx.y;
      const int nblk = ntpp[0] / B;
      int lead = 0, first = 0, last = 0, e = -1;
      if (b < nblk) {
        e = expert_ids[b];
        // expert_ids[0, nblk) is non-decreasing: binary search the run
        int lo = 0, hi = b;                  // first index with id == e
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (expert_ids[mid] < e) lo = mid + 1; else hi = mid;
        }
        first = lo;
        lo = b; hi = nblk;                   // first index with id > e
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (expert_ids[mid] <= e) lo = mid + 1; else hi = mid;
        }
        const int blocks_per_wg = BM >= B ? BM / B : 1;
        if (e >= 0 && e < E && ((b - first) % blocks_per_wg) == 0) {
          lead = 1;
          last = min(lo, b + blocks_per_wg);
        }
      }
      run_info[0] = lead;
      run_info[1] = e;
      run_info[2] = b * B;
      run_info[3] = lead ? (last - b) * B : 0;
    }
    __syncthreads();
    if (!run_info[0]) return;
    expert = run_info[1];
    row0 = run_info[2];
    rows_total = run_info[3];
  } else {
    rows_total = min(BM, M - (int)blockIdx.y * BM);
  }

  const uint32_t* Wbase = Wq + (int64_t)expert * N * kw;
  const uint16_t* Sbase = S + (int64_t)expert * N * G;
  const int nsteps = (K + kStepK - 1) / kStepK;
  // raw buffer views: lanes whose offset lies past the end read zero, so
  // no load needs a branch (a branch around a load makes the compiler wait
  // for it inside the branch, serialising the loads)
  const int x_rows = MOE ? n_pairs / x_row_div : M;
  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)x_rows * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wr = rsrc(Wbase, (uint32_t)N * (uint32_t)kw * 4u);
  const __amdgpu_buffer_rsrc_t sr = rsrc(Sbase, (uint32_t)N * (uint32_t)G * 2u);

  for (int pass0 = 0; pass0 < rows_total; pass0 += BM) {
    const int rows = min(BM, rows_total - pass0);
    // ---- row tables for this pass
    for (int r = tid; r < BM; r += NT) {
      int xr = -1, yr = -1;
      if (r < rows) {
        if constexpr (MOE) {
          const int f = sorted_ids[row0 + pass0 + r];
          if (f < n_pairs) { xr = f / x_row_div; yr = f; }
        } else {
          const int m = blockIdx.y * BM + pass0 + r;
          xr = m; yr = m;
        }
      }
      xrow[r] = xr;
      orow[r] = yr;
    }
    __syncthreads();
    const int ms_valid = (rows + 31) >> 5;

    f32x16 acc[MS][NS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ms][ns][v] = 0.0f;

    // ---- staging helpers
    u32x4 xstage[PIECES];
    auto load_x = [&](int step) {
#pragma unroll
      for (int p = 0; p < PIECES; ++p) {
        const int piece = tid + p * NT;
        const int r = piece >> 3;
        const int col = (piece & 7) * 8 + step * kStepK;
        const int xr_ = xrow[r];
        const uint32_t off =
            (xr_ >= 0 && col < K) ? ((uint32_t)xr_ * (uint32_t)K + (uint32_t)col) * 2u : kOOB;
        xstage[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
      }
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int p = 0; p < PIECES; ++p) {
        const int piece = tid + p * NT;
        const int r = piece >> 3;
        *(u32x4*)&xs[buf][r][(piece & 7) * 8] = xstage[p];
      }
    };
    u32x4 wreg[NS];
    uint32_t sreg[NS];             // bf16 scale of this lane's group (low half)
    auto load_w = [&](int step) {
      const int g = 2 * step + h;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const uint32_t n = (uint32_t)(n_base + ns * 32 + l32);
        // rows past N lie past the buffer's end; a group past K reads zero
        const uint32_t woff = (g < G) ? (n * (uint32_t)kw + 4u * (uint32_t)g) * 4u : kOOB;
        wreg[ns] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, 0, 0);
        const uint32_t soff = (g < G) ? (n * (uint32_t)G + (uint32_t)g) * 2u : kOOB;
        sreg[ns] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
      }
    };

    load_x(0);
    load_w(0);
    store_x(0);
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
      const int buf = step & 1;
      // dequantize this step's weights into B operands
      u32x4 bop[NS][4];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const float s = bf16_lo(sreg[ns]);
        const float m8s = -8.0f * s;
        bop[ns][0] = dequant8(wreg[ns].x, s, m8s);
        bop[ns][1] = dequant8(wreg[ns].y, s, m8s);
        bop[ns][2] = dequant8(wreg[ns].z, s, m8s);
        bop[ns][3] = dequant8(wreg[ns].w, s, m8s);
      }
      const bool more = step + 1 < nsteps;
      if (more) {
        load_x(step + 1);
        load_w(step + 1);
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        if (ms < ms_valid) {
          const uint16_t* xp = &xs[buf][ms * 32 + l32][32 * h];
          const u32x4 a0 = *(const u32x4*)(xp + 0);
          const u32x4 a1 = *(const u32x4*)(xp + 8);
          const u32x4 a2 = *(const u32x4*)(xp + 16);
          const u32x4 a3 = *(const u32x4*)(xp + 24);
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            acc[ms][ns] = mfma32(a0, bop[ns][0], acc[ms][ns]);
            acc[ms][ns] = mfma32(a1, bop[ns][1], acc[ms][ns]);
            acc[ms][ns] = mfma32(a2, bop[ns][2], acc[ms][ns]);
            acc[ms][ns] = mfma32(a3, bop[ns][3], acc[ms][ns]);
          }
        }
      }
      if (more) store_x(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: lane holds D[8*(v/4) + 4*h + v%4][l32] of each tile
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      if (ms < ms_valid) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ms * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          const int yr = orow[r];
          if (yr < 0) continue;
          float wgt = 1.0f;
          if constexpr (MOE) {
            if (topk_w != nullptr) wgt = topk_w[yr];
          }
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            const int n = n_base + ns * 32 + l32;
            if (n < N) {
              float y = acc[ms][ns][v];
              if constexpr (MOE) y *= wgt;
              Y[(int64_t)yr * N + n] = to_bf16(y);
            }
          }
        }
      }
    }
    __syncthreads();   // row tables are rewritten by the next pass
  }
}

namespace {
constexpr int kBM = 128;
constexpr int kWN = 64;
constexpr int kNW = 4;
}  // namespace

hipError_t launch_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const dim3 grid((unsigned)((N + kNW * kWN - 1) / (kNW * kWN)), (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL((k_gemm<kBM, kWN, kNW, false>), grid, dim3(kNW * 64), 0, st, X,
                     (const uint32_t*)Wq, S, Y, (int)M, (int)N, (int)K, nullptr, nullptr, nullptr,
                     nullptr, 0, 1, 1, 0);
  return hipGetLastError();
}

hipError_t launch_moe_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* ntpp, const float* topk_w, uint16_t* Y, int64_t T,
                           int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                           int32_t x_row_div, hipStream_t st) {
  const int64_t n_pairs = T * k;
  const int64_t cap = ((n_pairs + (int64_t)E * (B - 1) + B - 1) / B) * B;
  const dim3 grid((unsigned)((N + kNW * kWN - 1) / (kNW * kWN)), (unsigned)(cap / B));
  hipLaunchKernelGGL((k_gemm<kBM, kWN, kNW, true>), grid, dim3(kNW * 64), 0, st, X,
                     (const uint32_t*)Wq, S, Y, 0, (int)N, (int)K, sorted_ids, expert_ids, ntpp,
                     topk_w, (int)n_pairs, (int)B, (int)x_row_div, (int)E);
  return hipGetLastError();
}

}  // namespace w4
