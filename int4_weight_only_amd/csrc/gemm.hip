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
// and the VALU cost of dequantization (17 ops per 8 weights) is spread
// over BM rows of MFMA work.  K advances 64 per step: lane (n = l % 32,
// h = l / 32) loads the whole 32-element group 2c + h of weight row n (16
// bytes, one scale) and word j of it feeds MFMA j
// (v_mfma_f32_32x32x16_bf16); the activation operand is read with the
// same K permutation, which leaves the sum unchanged.
//
// Pipeline: activations go straight from HBM into LDS (16-byte
// buffer_load ... lds, three stages, no staging registers); codes and
// scales go to registers two steps ahead (two register sets).  The K loop
// is unrolled by six so that each step names its LDS stages statically.
// In LDS a 64-element activation row is 128 bytes; its eight 16-byte
// pieces are stored XOR-swizzled by (row / 2) % 8 so that the MFMA
// operand reads of 32 consecutive rows spread over the banks.  Every load
// is a raw buffer load whose out-of-range lanes read zero (rows past the
// end, K past the end, the padding steps of the unrolled loop), so no
// load is conditional.
#include <type_traits>

#include "common.h"

namespace w4 {

namespace {

constexpr int kStepK = 64;            // K per pipeline step (two groups)
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
__global__ __launch_bounds__(NW * 64, BM >= 256 ? 1 : 2) void k_gemm(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Wq, const uint16_t* __restrict__ S,
    uint16_t* __restrict__ Y, int M, int N, int K, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ ntpp,
    const float* __restrict__ topk_w, int n_pairs, int B, int x_row_div, int E) {
  constexpr int NT = NW * 64;
  constexpr int MS = BM / 32;          // 32-row MFMA tiles along M
  constexpr int NS = WN / 32;          // 32-col MFMA tiles along N per wave
  constexpr int XI = BM / 8;           // 1 KB direct-to-LDS loads per activation stage
  constexpr int XPW = XI / NW;         // ... issued by each wave
  constexpr int STAGE = BM * kStepK;   // bf16 elements per activation stage (three stages)
  static_assert(BM % 32 == 0 && WN % 32 == 0 && XI % NW == 0 && BM <= NT, "tile shape");

  // three separately declared stages: each DMA target and each operand
  // read names one object, so the compiler can tell that reading stage s
  // does not wait on the DMA still filling stage s + 2
  __shared__ __attribute__((aligned(16))) uint16_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[STAGE];
  __shared__ int xrow[BM];     // activation row of each tile row (-1: none)
  __shared__ int orow[BM];     // output row of each tile row (-1: none)
  __shared__ int run_info[4];
  __shared__ int wave_end[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  // Tile of this workgroup.  MoE: (blockIdx.x = weight-row tile,
  // blockIdx.y = alignment block).  Dense: a 1-D grid; workgroups are
  // dispatched round-robin over the 8 XCDs (each with its own L2), so XCD x
  // takes the contiguous tile range [x * per, (x + 1) * per), walked in
  // groups of GM activation row-blocks: the workgroups running together on
  // one XCD share activation rows and weight rows in that XCD's L2.
  int tile_n, tile_m;
  if constexpr (MOE) {
    tile_n = blockIdx.x;
    tile_m = 0;
  } else {
    constexpr int kXcds = 8, GM = 8;
    const int mt = (M + BM - 1) / BM, nt = (N + NW * WN - 1) / (NW * WN);
    const int tiles = mt * nt;
    const int per = (tiles + kXcds - 1) / kXcds;
    const int pid = blockIdx.x;
    const int t = (pid % kXcds) * per + pid / kXcds;
    if (t >= tiles) return;
    const int group = t / (GM * nt);
    const int first_m = group * GM;
    const int gm = min(GM, mt - first_m);
    const int in_group = t - group * (GM * nt);
    tile_m = first_m + in_group % gm;
    tile_n = in_group / gm;
  }
  const int n_base = tile_n * (NW * WN) + wave * WN;
  const int G = K >> 5;
  const int kw = K >> 3;

  int rows_total;              // rows handled by this workgroup (all passes)
  int row0 = 0;                // MoE: first sorted slot of the run
  int expert = 0;
  if constexpr (MOE) {
    // Find this block's run of one expert with wave 0: expert_ids[0, nblk)
    // is non-decreasing, so the blocks of expert e are contiguous.  Lanes
    // read the 64 ids ending at b and the 64 ids starting at b in two
    // parallel loads; ballots give the distance to the run's first block
    // (a longer run walks back 64 blocks at a time) and its end.
    if (wave == 0) {
      const int b = blockIdx.y;
      const int nblk = ntpp[0] / B;
      int lead = 0, e = -1, last = 0;
      if (b < nblk) {
        e = expert_ids[b];
        const int bpw = BM >= B ? BM / B : 1;
        // backwards: first block of the run
        int first = b;
        for (int base = b;; base -= 64) {
          const int idx = base - lane;                       // lane 0 = base
          const int id = idx >= 0 ? expert_ids[idx] : -2;
          const uint64_t same = __ballot(id == e);           // contiguous from lane 0
          const int run = __popcll(same);
          first = base - run + 1;
          if (run < 64 || base - 64 < 0) break;
        }
        // forwards: end of the run, capped at bpw blocks from b
        const int fidx = b + lane;
        const int fid = (fidx < nblk && lane < bpw) ? expert_ids[fidx] : -2;
        const int fwd = __popcll(__ballot(fid == e));      // blocks of the run in [b, b + bpw)
        if (e >= 0 && e < E && ((b - first) % bpw) == 0) {
          lead = 1;
          last = b + fwd;
        }
      }
      if (lane == 0) {
        run_info[0] = lead;
        run_info[1] = e;
        run_info[2] = b * B;
        run_info[3] = lead ? (last - b) * B : 0;
      }
    }
    __syncthreads();
    if (!run_info[0]) return;
    expert = run_info[1];
    row0 = run_info[2];
    rows_total = run_info[3];
  } else {
    rows_total = min(BM, M - tile_m * BM);
  }

  const uint32_t* Wbase = Wq + (int64_t)expert * N * kw;
  const uint16_t* Sbase = S + (int64_t)expert * N * G;
  const int nsteps = (K + kStepK - 1) / kStepK;
  const int nsteps6 = (nsteps + 5) / 6 * 6;  // padded to the unroll; pad steps load zeros, skip MFMAs
  const int x_rows = MOE ? n_pairs / x_row_div : M;
  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)x_rows * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wr = rsrc(Wbase, (uint32_t)N * (uint32_t)kw * 4u);
  const __amdgpu_buffer_rsrc_t sr = rsrc(Sbase, (uint32_t)N * (uint32_t)G * 2u);

  for (int pass0 = 0; pass0 < rows_total; pass0 += BM) {
    const int rows = min(BM, rows_total - pass0);
    // ---- row tables for this pass (thread r < BM fills row r)
    {
      int xr_ = -1, yr = -1;
      if (tid < rows) {
        if constexpr (MOE) {
          const int f = sorted_ids[row0 + pass0 + tid];
          if (f < n_pairs) { xr_ = f / x_row_div; yr = f; }
        } else {
          const int m = tile_m * BM + pass0 + tid;
          xr_ = m; yr = m;
        }
      }
      if (tid < BM) {
        xrow[tid] = xr_;
        orow[tid] = yr;
      }
      if constexpr (MOE) {
        // one past the last valid row of each wave's 64 rows: padding
        // slots (sentinel ids) at the end of a run need no MFMA tile
        const uint64_t v = __ballot(xr_ >= 0);
        if (lane == 0) wave_end[wave] = v ? wave * 64 + 64 - (int)__clzll(v) : 0;
      }
    }
    __syncthreads();
    int ms_valid = (rows + 31) >> 5;
    if constexpr (MOE) {
      int end = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) end = max(end, wave_end[w]);
      ms_valid = (end + 31) >> 5;
      if (ms_valid == 0) {   // a pass of padding only (blocks larger than the tile)
        __syncthreads();     // wave_end is rewritten by the next pass
        continue;
      }
    }

    // Direct-to-LDS activation loads.  Instruction i of this wave fills
    // tile rows 8 (wave*XPW + i) .. +7; lane l writes the 16 bytes at
    // slot l, i.e. row r = 8 I + l / 8, stored piece l % 8, which holds
    // global piece (l % 8) ^ ((r / 2) % 8) of that row.
    uint32_t xoff[XPW];        // byte offset of this lane's piece at step 0 (or OOB)
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      const int r = 8 * (wave * XPW + i) + (lane >> 3);
      const int pg = (lane & 7) ^ ((r >> 1) & 7);
      const int xr_ = xrow[r];
      xoff[i] = xr_ >= 0 ? ((uint32_t)xr_ * (uint32_t)K + 8u * (uint32_t)pg) * 2u : kOOB;
    }
    auto load_x = [&](int step, uint16_t* st) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < XPW; ++i) {
        const int col = step * kStepK + 8 * ((lane & 7) ^ (((8 * (wave * XPW + i) + (lane >> 3)) >> 1) & 7));
        const uint32_t off = (xoff[i] != kOOB && col < K) ? xoff[i] + (uint32_t)step * (kStepK * 2) : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void*)(st + (wave * XPW + i) * 512), 16, off, 0,
            0, 0);
      }
    };
    // codes + scales of one step into a register set
    auto load_w = [&](int step, u32x4 (&wreg)[NS], uint32_t (&sreg)[NS])
        __attribute__((always_inline)) {
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

    f32x16 acc[MS][NS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ms][ns][v] = 0.0f;

    // one step: wait for this step's activations, make them visible, start
    // the stage two ahead, dequantize, multiply, start the codes two ahead.
    // MSE activation tiles are multiplied (rows past the pass read zero).
    // Per 16-wide K slice j all operand reads are issued first and the
    // MSE x NS MFMAs that follow are independent (no accumulator chain).
    auto step_body = [&](auto mse, int step, const uint16_t* st, uint16_t* st_next2,
                         u32x4 (&wreg)[NS], uint32_t (&sreg)[NS]) __attribute__((always_inline)) {
      constexpr int MSE = decltype(mse)::value;
      // loads issued after this step's activations: its codes and scales
      // (2 NS), the next step's activations (XPW) and codes (2 NS)
      static_assert(XPW + 4 * NS <= 63, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(XPW + 4 * NS) : "memory");
      __syncthreads();
      load_x(step + 2, st_next2);
      if (step < nsteps) {
        u32x4 bop[NS][4];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const DeqScale d = deq_scale(bf16_lo(sreg[ns]));
          bop[ns][0] = dequant8(wreg[ns].x, d);
          bop[ns][1] = dequant8(wreg[ns].y, d);
          bop[ns][2] = dequant8(wreg[ns].z, d);
          bop[ns][3] = dequant8(wreg[ns].w, d);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 a[MSE];
#pragma unroll
          for (int ms = 0; ms < MSE; ++ms) {
            const int R = ms * 32 + l32;
            a[ms] = *(const u32x4*)(st + R * kStepK + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
          }
#pragma unroll
          for (int ms = 0; ms < MSE; ++ms)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) acc[ms][ns] = mfma32(a[ms], bop[ns][j], acc[ms][ns]);
        }
      }
      load_w(step + 2, wreg, sreg);
    };

    u32x4 wa[NS], wb[NS];
    uint32_t sa[NS], sb[NS];
    load_x(0, xs0);
    load_w(0, wa, sa);
    load_x(1, xs1);
    load_w(1, wb, sb);
    auto run_steps = [&](auto mse) __attribute__((always_inline)) {
      for (int step = 0; step < nsteps6; step += 6) {
        step_body(mse, step + 0, xs0, xs2, wa, sa);
        step_body(mse, step + 1, xs1, xs0, wb, sb);
        step_body(mse, step + 2, xs2, xs1, wa, sa);
        step_body(mse, step + 3, xs0, xs2, wb, sb);
        step_body(mse, step + 4, xs1, xs0, wa, sa);
        step_body(mse, step + 5, xs2, xs1, wb, sb);
      }
    };
    if constexpr (MOE) {
      // MFMA row tiles that hold valid rows (a run of one expert is often
      // a single 32-row tile; a run of 85 rows padded to 128 needs three)
      static_assert(MS == 4, "one instantiation per row-tile count");
      if (ms_valid == 1)
        run_steps(std::integral_constant<int, 1>{});
      else if (ms_valid == 2)
        run_steps(std::integral_constant<int, 2>{});
      else if (ms_valid == 3)
        run_steps(std::integral_constant<int, 3>{});
      else
        run_steps(std::integral_constant<int, 4>{});
    } else {
      run_steps(std::integral_constant<int, MS>{});
    }
    // drain the loads of the padding steps before LDS is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
    __syncthreads();   // row tables and LDS stages are rewritten by the next pass
  }
}

namespace {
constexpr int kWN = 64;
constexpr int kNW = 4;
constexpr int kBMDense = 128;   // dense prefill tile rows (two workgroups per CU)
constexpr int kBMMoe = 128;     // expert blocks are 16..64 rows: a smaller tile pads less
}  // namespace

hipError_t launch_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = ((N + kNW * kWN - 1) / (kNW * kWN)) * ((M + kBMDense - 1) / kBMDense);
  const dim3 grid((unsigned)(((tiles + 7) / 8) * 8));   // whole rounds over the 8 XCDs
  hipLaunchKernelGGL((k_gemm<kBMDense, kWN, kNW, false>), grid, dim3(kNW * 64), 0, st, X,
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
  hipLaunchKernelGGL((k_gemm<kBMMoe, kWN, kNW, true>), grid, dim3(kNW * 64), 0, st, X,
                     (const uint32_t*)Wq, S, Y, 0, (int)N, (int)K, sorted_ids, expert_ids, ntpp,
                     topk_w, (int)n_pairs, (int)B, (int)x_row_div, (int)E);
  return hipGetLastError();
}

}  // namespace w4
