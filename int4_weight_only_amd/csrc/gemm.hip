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
// Code layouts (TL).  Canonical: Wq [N, K/8] row-major, so the 16-byte
// pieces one step of a wave loads (group 2 c + h of 32 rows) lie 32 bytes
// per row, K/2 bytes apart.  Kernel order (w4_repack): 32-row x 64-k blocks
// of 1 KB, block (r, c) at byte 1024 (r ceil(K/64) + c), and inside it the
// 16-byte unit 32 h + (n % 32) = group 2 c + h of row 32 r + n % 32 -- the
// order in which the lanes of one load read them, so each load instruction
// reads 1 KB of contiguous memory and a run of steps is one contiguous
// stream (the weight-layout conversion the RL write-up's section 4 applies
// before its inference kernel).  Scales and zero points come in kernel
// order too (w4_repack_groups): 16-row x 8-group blocks of 128 values, so
// the 8 values of a window that lanes n .. n + 15 load are 256 contiguous
// bytes (128 for zero points) instead of 16 pieces one row apart.  The
// arithmetic is identical.
//
// Pipeline: activations go straight from HBM into LDS (16-byte
// buffer_load ... lds, four stages: three steps ahead, no staging
// registers); codes go to registers two steps ahead (two register sets;
// four for the 32-row tile, whose few MFMAs per step leave the weight
// stream latency-bound), scales in 8-step windows.  The K loop is unrolled
// by four (the stage rotation, or the register-set rotation if longer) so
// that each step names its LDS stage and register set statically.
// In LDS a 64-element activation row is 128 bytes; its eight 16-byte
// pieces are stored XOR-swizzled by (row / 2) % 8 so that the MFMA
// operand reads of 32 consecutive rows spread over the banks.  Every load
// is a raw buffer load whose out-of-range lanes read zero (rows past the
// end, K past the end, the padding steps of the unrolled loop), so no
// load is conditional.
#include <mutex>
#include <type_traits>

#include "common.h"

namespace w4 {

namespace {

constexpr int kStepK = 64;            // K per pipeline step (two groups)
constexpr int kXS = 4;                // LDS activation stages (three steps ahead)
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
// SA: K is a multiple of 256, so a row's scales start 16-byte aligned and
// eight of them are one 16-byte load, and every step lies inside K: the
// loads carry no per-lane range checks.  Loads issued ahead past the last
// step read the next rows' bytes, which no step uses; the 32-row tile,
// which issues codes up to eight steps ahead, sends them to an empty buffer
// instead (a uniform choice: they read zero without touching memory).
// SWI (MoE only): N = 2I weight rows, gate [0, I) and up [I, 2I); waves 0, 1
// take gate rows [c, c + 2 WN) and waves 2, 3 the matching up rows, and the
// epilogue writes A = bf16(silu(bf16(gate)) * bf16(up)) [rows, I].
// ZP: zero-point weights, unsigned codes and one zero point byte per group
// in Z [N, K/32] (grouped: Z [E, N, K/32]); w' = bf16((q - z) s).
// BM = 32 (one MFMA row tile, few rows per expert): eight code register
// sets filled four steps at a time (a row's 128-byte code line is requested
// in four back-to-back loads instead of across four steps, when L2 may have
// dropped it) and four workgroups per CU keep weight bytes in flight, and
// workgroups index runs rather than blocks.
// CMB (grouped down product only): the workgroup stores its rows of Y (the
// unweighted bf16 products) with agent-coherent stores (written through the
// XCD's L2), waits until they are done, and counts each row's token in on
// cnt[token * ntn + tile_n] (one counter per token and weight-row tile,
// device-scope atomics); the workgroup whose count completes a token (its
// pairs routed to experts in [0, E) all stored) reads those rows back with
// agent-coherent loads and writes Out[token, tile columns] = bf16(sum over j
// in order of cw[t k + j] * Y[t k + j, column]) -- the same fp32 operations
// in the same order as the separate combine -- and sets the counter back
// to 0.  Coherent accesses replace an L2 write-back per workgroup and an L2
// invalidate per completing workgroup, which measured 2.5x slower.  Pairs
// whose expert lies outside [0, E) take no part.
template <int BM, int WN, int NW, bool MOE, bool SA, bool SWI, bool ZP = false, bool TL = false,
          bool CMB = false>
__global__ __launch_bounds__(NW * 64, BM >= 256 ? 1 : (BM <= 32 ? 4 : 2)) void k_gemm(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ Wq, const uint16_t* __restrict__ S,
    const uint8_t* __restrict__ Z, uint16_t* __restrict__ Y, int M, int N, int K,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ expert_ids,
    const int32_t* __restrict__ ntpp, const float* __restrict__ topk_w, int n_pairs, int B,
    int x_row_div, int E, uint16_t* __restrict__ Out, int32_t* __restrict__ cnt,
    const int32_t* __restrict__ topk_ids, const float* __restrict__ cw, int topk) {
  constexpr int NT = NW * 64;
  constexpr int MS = BM / 32;          // 32-row MFMA tiles along M
  constexpr int NS = WN / 32;          // 32-col MFMA tiles along N per wave
  constexpr int XI = BM / 8;           // 1 KB direct-to-LDS loads per activation stage
  constexpr int XPW = XI / NW;         // ... issued by each wave
  constexpr int STAGE = BM * kStepK;   // bf16 elements per activation stage
  // 32-row tile: eight code register sets filled four at a time (steps
  // 4u + 8 .. 4u + 11 after step 4u + 3), so the four 32-byte pieces of a
  // row's 128-byte code line are requested back to back
  constexpr bool kGroupW = BM <= 32;
  constexpr int kWS = kGroupW ? 8 : 2;   // code register sets (steps ahead)
  constexpr int kU = kWS > kXS ? kWS : kXS;   // K-loop unroll: stage and set named statically
  constexpr bool kRunSlots = MOE && BM <= 32;  // grouped product: slots index runs
  constexpr bool kNullPast = SA && kGroupW;      // loads past the last step read the empty buffer
  constexpr bool kPipe = !MOE;                   // dequant of slice j + 1 under slice j's MFMAs
  static_assert(kU % kXS == 0 && kU % kWS == 0, "unroll");
  static_assert(BM % 32 == 0 && WN % 32 == 0 && XI % NW == 0 && BM <= NT, "tile shape");

  // separately declared stages: each DMA target and each operand read names
  // one object, so the compiler can tell that reading stage s does not wait
  // on the DMA still filling a later stage
  __shared__ __attribute__((aligned(16))) uint16_t xs0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t xs3[STAGE];
  __shared__ int xrow[BM];     // activation row of each tile row (-1: none)
  __shared__ int orow[BM];     // output row of each tile row (-1: none)
  __shared__ int run_info[4];
  __shared__ int wave_end[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, so the LDS addresses of the direct-to-LDS loads are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  // Tile of this workgroup.  MoE: a slot of at most BM rows (an alignment
  // block, or one BM-row part of a block larger than BM) and a weight-row
  // tile; the workgroup leads a run of consecutive slots of one expert,
  // at most BM rows.  Dense: a 1-D grid; workgroups are
  // dispatched round-robin over the 8 XCDs (each with its own L2), so XCD x
  // takes the contiguous tile range [x * per, (x + 1) * per), walked in
  // groups of GM activation row-blocks: the workgroups running together on
  // one XCD share activation rows and weight rows in that XCD's L2.
  int tile_n, tile_m;
  int slot = 0;
  const int bpw = BM >= B ? BM / B : 1;               // MoE: blocks per run (at most)
  const int ppb = B > BM ? (B + BM - 1) / BM : 1;      // MoE: slots per block
  if constexpr (MOE) {
    // XCD-aware: slots go round-robin over the XCDs, all N-tiles of a slot
    // on one XCD, which share its rows.  32-row tile: a slot is a run
    // (below).  128-row tile: a slot is a block part, and groups of bpw
    // slots (one run's worth of blocks) go to one XCD, which measured
    // faster there than single slots.
    // N-tiles: 2 WN gate rows (+ the matching up rows) per workgroup with
    // SWI, else NW WN weight rows; a 1-D grid of N-tiles x slots
    const int ntn = SWI ? ((N >> 1) + 2 * WN - 1) / (2 * WN) : (N + NW * WN - 1) / (NW * WN);
    const int pid = blockIdx.x;                      // dispatch order
    const int xcd = pid & 7, j = pid >> 3;
    tile_n = j % ntn;
    const int q = j / ntn;
    slot = kRunSlots ? xcd + 8 * q : (xcd + 8 * (q / bpw)) * bpw + q % bpw;
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
  static_assert(!SWI || (MOE && NW == 4), "fused SwiGLU: grouped product, four waves");
  static_assert(!CMB || (MOE && !SWI), "fused combine: grouped down product");
  const int n_base = SWI ? (wave >> 1) * (N >> 1) + tile_n * (2 * WN) + (wave & 1) * WN
                         : tile_n * (NW * WN) + wave * WN;
  const int G = K >> 5;
  const int kw = K >> 3;

  int rows;                    // rows of this workgroup's tile (<= BM)
  int row0 = 0;                // MoE: first sorted position of the run
  int expert = 0;
  if constexpr (MOE) {
    // Find this slot's run of one expert with wave 0: expert_ids[0, nblk)
    // is non-decreasing, so the blocks of expert e are contiguous.
    if (wave == 0) {
      const int nblk = ntpp[0] / B;
      int lead = 0, e = -1, last = 0, b = 0, part = 0;
      if (kRunSlots && bpw > 1) {
        // Runs of up to bpw blocks start wherever an expert's blocks do, so
        // slot r is the r-th run: count run starts over expert_ids, 64
        // blocks per step with sixteen steps' ids loaded at once.  A ballot of
        // expert starts (id differs from the previous block's) gives each
        // block its expert's first block; a second ballot marks the blocks
        // that start a run.  Indexing slots by run spreads the runs evenly
        // over the XCDs and launches no workgroup for a run's later blocks.
        const int r = slot;
        int count = 0, carry_e = -3, carry_first = 0;
        b = -1;
        const uint64_t below = (1ull << lane) - 1ull;     // lanes < lane
        constexpr int kScan = 16;
        for (int cb = 0; cb < nblk && b < 0; cb += 64 * kScan) {
          int ev[kScan];
#pragma unroll
          for (int u = 0; u < kScan; ++u) {
            const int bb = cb + 64 * u + lane;
            ev[u] = bb < nblk ? expert_ids[bb] : -2;
          }
#pragma unroll
          for (int u = 0; u < kScan; ++u) {
            const int c0 = cb + 64 * u;
            if (c0 >= nblk || b >= 0) break;
            const int bb = c0 + lane;
            const bool valid = bb < nblk;
            const int eb = ev[u];
            int prev = __shfl_up(eb, 1);
            if (lane == 0) prev = carry_e;
            const uint64_t starts = __ballot(valid && eb != prev);
            const uint64_t upto = starts & (below | (1ull << lane));
            const int first = upto ? c0 + 63 - (int)__clzll(upto) : carry_first;
            const bool is_lead = valid && eb >= 0 && eb < E && ((bb - first) % bpw) == 0;
            const uint64_t leads = __ballot(is_lead);
            const int n = __popcll(leads);
            if (r < count + n) {
              const uint64_t hit = __ballot(is_lead && __popcll(leads & below) == r - count);
              const int ln = __ffsll((long long)hit) - 1;
              b = c0 + ln;
              e = __shfl(eb, ln);
            } else {
              count += n;
              carry_e = __shfl(eb, 63);
              carry_first = __shfl(first, 63);
            }
          }
        }
        if (b >= 0) {
          // blocks of the run: the expert's blocks in [b, b + bpw)
          const int fidx = b + lane;
          const int fid = (fidx < nblk && lane < bpw) ? expert_ids[fidx] : -2;
          lead = 1;
          last = b + __popcll(__ballot(fid == e));
        } else {
          b = 0;
        }
      } else if ((b = slot / ppb) < nblk) {
        // slot = block part: this block's run, led by it if it lies a
        // multiple of bpw blocks after its expert's first block.
        part = slot - b * ppb;
        e = expert_ids[b];
        // The expert's first block: expert_ids is non-decreasing, so the ids
        // below e form a prefix of [0, b]; 64 lanes sample [lo, hi] evenly and
        // a ballot narrows it 64-fold per step (three steps for 262144 blocks).
        int lo = 0, hi = b;
        while (lo < hi) {
          const int step = (hi - lo + 63) / 64;
          const int p = lo + lane * step;
          const int id = expert_ids[min(p, hi)];             // hi <= b < nblk: in bounds
          const int c = __popcll(__ballot(p < hi && id < e));
          if (c == 0) break;                                 // expert_ids[lo] == e
          const int nhi = min(hi, lo + c * step);
          lo = lo + (c - 1) * step + 1;
          hi = nhi;
        }
        const int first = lo;
        if (e >= 0 && e < E && ((b - first) % bpw) == 0) {
          // blocks of the run: the expert's blocks in [b, b + bpw), counted
          // 64 per ballot (bpw reaches 128 at B = 1)
          int fwd = 0;
          for (int off = 0; off < bpw; off += 64) {
            const int fidx = b + off + lane;
            const int fid = (fidx < nblk && off + lane < bpw) ? expert_ids[fidx] : -2;
            const int cnt = __popcll(__ballot(fid == e));
            fwd += cnt;
            if (cnt < 64) break;
          }
          lead = 1;
          last = b + fwd;
        }
      }
      if (lane == 0) {
        run_info[0] = lead;
        run_info[1] = e;
        run_info[2] = b * B + part * BM;
        run_info[3] = lead ? min(BM, (last - b) * B - part * BM) : 0;
      }
    }
    __syncthreads();
    if (!run_info[0]) return;
    expert = run_info[1];
    row0 = run_info[2];
    rows = run_info[3];
  } else {
    rows = min(BM, M - tile_m * BM);
  }

  // tiled: each expert holds ceil(N/32) x ceil(K/64) blocks of 1 KB
  const int64_t tl_words = (int64_t)((N + 31) >> 5) * ((K + kStepK - 1) / kStepK) * 256;
  const uint32_t* Wbase = Wq + (int64_t)expert * (TL ? tl_words : (int64_t)N * kw);
  // kernel-order scales and zero points: each expert holds ceil(N/16) x
  // ceil(G/8) blocks of 128 values (value 8 i + j of block (r, c) = row
  // 16 r + i, group 8 c + j)
  const uint32_t gblk = (uint32_t)(G + 7) >> 3;
  const int64_t grp_elems = TL ? (int64_t)((N + 15) >> 4) * gblk * 128 : (int64_t)N * G;
  const uint16_t* Sbase = S + (int64_t)expert * grp_elems;
  const int nsteps = (K + kStepK - 1) / kStepK;
  const int nstepsp = (nsteps + kU - 1) / kU * kU;  // padded to the unroll; pad steps load zeros, skip MFMAs
  const int x_rows = MOE ? n_pairs / x_row_div : M;
  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)x_rows * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wr =
      rsrc(Wbase, TL ? (uint32_t)tl_words * 4u : (uint32_t)N * (uint32_t)kw * 4u);
  const __amdgpu_buffer_rsrc_t sr = rsrc(Sbase, (uint32_t)grp_elems * 2u);
  const uint8_t* Zbase = ZP ? Z + (int64_t)expert * grp_elems : nullptr;
  const __amdgpu_buffer_rsrc_t zr = rsrc(Zbase, ZP ? (uint32_t)grp_elems : 0u);
  const __amdgpu_buffer_rsrc_t rnull = rsrc(nullptr, 0u);   // every load reads zero

  {
    // ---- row tables (thread r < BM fills row r)
    {
      int xr_ = -1, yr = -1;
      if (tid < rows) {
        if constexpr (MOE) {
          const int f = sorted_ids[row0 + tid];
          if (f < n_pairs) { xr_ = f / x_row_div; yr = f; }
        } else {
          const int m = tile_m * BM + tid;
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
      if (ms_valid == 0) return;   // a slot of padding only (blocks larger than the tile)
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
        // (an OOB row's offset stays past the buffer: X is below 2 GiB)
        const uint32_t off = (SA || (xoff[i] != kOOB && col < K))
                                 ? xoff[i] + (uint32_t)step * (kStepK * 2)
                                 : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            (kNullPast && step >= nsteps) ? rnull : xr,
            (__attribute__((address_space(3))) void*)(st + (wave * XPW + i) * 512), 16, off, 0, 0,
            0);
      }
    };
    // codes of one step into a register set
    auto load_w = [&](int step, u32x4 (&wreg)[NS]) __attribute__((always_inline)) {
      const int g = 2 * step + h;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const uint32_t n = (uint32_t)(n_base + ns * 32 + l32);
        // rows past N lie past the buffer's end (or in the zero padding of
        // the last 32-row block); a group past K reads zero
        uint32_t woff;
        if constexpr (TL)
          woff = (SA || g < G) ? (((n >> 5) * (uint32_t)nsteps + (uint32_t)step) * 64u + (uint32_t)h * 32u +
                            (n & 31u)) * 16u
                         : kOOB;
        else
          woff = (SA || g < G) ? (n * (uint32_t)kw + 4u * (uint32_t)g) * 4u : kOOB;
        wreg[ns] = __builtin_amdgcn_raw_buffer_load_b128((kNullPast && step >= nsteps) ? rnull : wr, woff,
                                                         0, 0);
      }
    };
    // Scales come in windows of 8 steps (16 groups): lane (n, h) loads the
    // 8 scales of groups 16 u + 8 h .. + 7 of its row, so a scale row is
    // read in 32-byte pieces, each once (scattered 2-byte loads per step
    // would need each 128-byte scale line to stay in L2 for 32 steps).
    // SA: windows past K read the next rows' values, which no step uses
    // (the 32-row tile sends a window wholly past K to the empty buffer).
    auto load_s = [&](int u, u32x4 (&raw)[NS]) __attribute__((always_inline)) {
      const int g0 = 16 * u + 8 * h;
      const __amdgpu_buffer_rsrc_t srs = (kNullPast && 16 * u >= G) ? rnull : sr;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const uint32_t n = (uint32_t)(n_base + ns * 32 + l32);
        if constexpr (TL) {
          // rows past N fall in the zero padding or past the expert's blocks
          const uint32_t e = ((n >> 4) * gblk + ((uint32_t)g0 >> 3)) * 128u + 8u * (n & 15u);
          raw[ns] = __builtin_amdgcn_raw_buffer_load_b128(srs, (SA || g0 < G) ? e * 2u : kOOB, 0, 0);
        } else if constexpr (SA) {
          raw[ns] = __builtin_amdgcn_raw_buffer_load_b128(srs, (n * (uint32_t)G + (uint32_t)g0) * 2u,
                                                          0, 0);
        } else {
          uint32_t hw[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int g = g0 + j;
            const uint32_t soff = (g < G) ? (n * (uint32_t)G + (uint32_t)g) * 2u : kOOB;
            hw[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
          }
          raw[ns] = u32x4{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16),
                          hw[6] | (hw[7] << 16)};
        }
      }
    };
    // Zero points in the same windows: lane (n, h) loads the 8 bytes of
    // groups 16 u + 8 h .. + 7 (one 8-byte load when rows are 8-byte
    // aligned, K % 256 == 0).
    auto load_z = [&](int u, u32x2 (&raw)[NS]) __attribute__((always_inline)) {
      const int g0 = 16 * u + 8 * h;
      const __amdgpu_buffer_rsrc_t zrs = (kNullPast && 16 * u >= G) ? rnull : zr;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const uint32_t n = (uint32_t)(n_base + ns * 32 + l32);
        if constexpr (TL) {
          const uint32_t e = ((n >> 4) * gblk + ((uint32_t)g0 >> 3)) * 128u + 8u * (n & 15u);
          raw[ns] = __builtin_amdgcn_raw_buffer_load_b64(zrs, (SA || g0 < G) ? e : kOOB, 0, 0);
        } else if constexpr (SA) {
          raw[ns] = __builtin_amdgcn_raw_buffer_load_b64(zrs, n * (uint32_t)G + (uint32_t)g0, 0, 0);
        } else {
          uint32_t b[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int g = g0 + j;
            const uint32_t zoff = (g < G) ? n * (uint32_t)G + (uint32_t)g : kOOB;
            b[j] = __builtin_amdgcn_raw_buffer_load_b8(zr, zoff, 0, 0);
          }
          raw[ns] = u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                          b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
        }
      }
    };
    // Step t of the window uses group 2 t + h.  v_permlane32_swap hands each
    // lane its partner's (other h) raw dwords; v_perm keeps half h of both:
    // scw[ns][k] = (scale of step k, scale of step k + 4) as a bf16 pair.
    const uint32_t half_sel = h ? 0x07060302u : 0x05040100u;
    auto unpack_s = [&](const u32x4 (&raw)[NS], uint32_t (&scw)[NS][4])
        __attribute__((always_inline)) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const uint32_t r[4] = {raw[ns].x, raw[ns].y, raw[ns].z, raw[ns].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const auto pr = __builtin_amdgcn_permlane32_swap(r[k], r[k], false, false);
          // pr[0]: the h = 0 lane's dword (groups 2k, 2k + 1 of the window)
          // pr[1]: the h = 1 lane's dword (groups 8 + 2k, 8 + 2k + 1)
          scw[ns][k] = __builtin_amdgcn_perm(pr[1], pr[0], half_sel);
        }
      }
    };
    // zero points: steps 0..3 take bytes h, 2 + h, 4 + h, 6 + h of the
    // h = 0 lane's 8 bytes, steps 4..7 the same bytes of the h = 1 lane's:
    // zw[ns][t / 4] byte t % 4 = zero point of step t
    const uint32_t byte_sel = h ? 0x07050301u : 0x06040200u;
    auto unpack_z = [&](const u32x2 (&raw)[NS], uint32_t (&zw)[NS][2])
        __attribute__((always_inline)) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const auto p0 = __builtin_amdgcn_permlane32_swap(raw[ns].x, raw[ns].x, false, false);
        const auto p1 = __builtin_amdgcn_permlane32_swap(raw[ns].y, raw[ns].y, false, false);
        zw[ns][0] = __builtin_amdgcn_perm(p1[0], p0[0], byte_sel);
        zw[ns][1] = __builtin_amdgcn_perm(p1[1], p0[1], byte_sel);
      }
    };

    // One step: wait for this step's activations and make them visible,
    // start the stage three ahead, dequantize, multiply, start the codes two
    // ahead.  MSE activation tiles are multiplied (rows past the tile read
    // zero).  Per 16-wide K slice j all operand reads are issued first and
    // the MSE x NS MFMAs that follow are independent (no accumulator chain).
    u32x4 wset[kWS][NS];       // code register sets: step t uses set t % kWS
    u32x4 sraw[NS];            // scale window in flight
    uint32_t scw[NS][4];       // scale window in use
    u32x2 zraw[NS];            // zero-point window in flight (ZP)
    uint32_t zw[NS][2];        // zero-point window in use (ZP)
    auto step_body = [&](auto mse, auto pos, int step, const uint16_t* st, uint16_t* st_next,
                         u32x4 (&wreg)[NS], f32x16 (&acc)[decltype(mse)::value][NS])
        __attribute__((always_inline)) {
      constexpr int MSE = decltype(mse)::value;
      // Wait until this wave's activations of this step have landed.  They
      // were issued three steps ago; after them came, in steady state, three
      // code sets (NS loads each: steps step + kWS - 3 .. step + kWS - 1)
      // and the activations of steps step + 1, step + 2 (XPW each).  With
      // two register sets the prologue has one code set fewer in the first
      // steps, so 2 XPW + 2 NS loads may stay in flight (in steady state
      // this also waits for the codes of step - 1, which that step
      // consumed).  The 32-row tile issues its codes four steps at a time,
      // at the end of each step 4u + 3 (steps 4u + 8 .. 4u + 11, before
      // their activations), so after the activations of step s come those
      // of s + 1 and s + 2 and, unless s % 4 == 3, one group of four code
      // sets: 2 XPW + 4 NS loads may stay in flight (2 XPW when
      // s % 4 == 3); its prologue issues in the same order.  Scale and
      // zero-point windows add loads, which only makes the wait stricter.
      // Then
      // a bare s_barrier: __syncthreads' release fence would also wait for
      // the later stages' DMA, which nothing reads yet.  The empty asm
      // statements keep LDS accesses on their side of the barrier.
      constexpr int P = decltype(pos)::value % 4;
      constexpr int kAfter = kGroupW ? (kXS - 2) * XPW + (P != 3 ? 4 * NS : 0)
                                     : (kXS - 2) * XPW + (kWS < 3 ? kWS : 3) * NS;
      static_assert(kAfter <= 63, "vmcnt range");
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kAfter) : "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      load_x(step + kXS - 1, st_next);
      // P = step % 4 (static); the 8-step scale window's half is (step >> 2) & 1
      if (P == 0 && (step & 4) == 0) {   // a new scale window: unpack it, fetch the next
        unpack_s(sraw, scw);
        load_s((step >> 3) + 1, sraw);
        if constexpr (ZP) {
          unpack_z(zraw, zw);
          load_z((step >> 3) + 1, zraw);
        }
      }
      // (SA with a 4-step unroll: K/64 steps, a multiple of the unroll)
      if ((SA && kU == 4) || step < nsteps) {
        // step t of the window uses the bf16 in half (t >= 4) of dword t % 4:
        // one v_perm with a uniform selector moves it into the top half
        const uint32_t hsel = (step & 4) ? 0x03020C0Cu : 0x01000C0Cu;
        DeqScale d[NS];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const float sc = __uint_as_float(__builtin_amdgcn_perm(0u, scw[ns][P], hsel));
          if constexpr (ZP) {
            const uint32_t zd = (step & 4) ? zw[ns][1] : zw[ns][0];
            d[ns] = deq_scale_zp(sc, (float)((zd >> (8 * P)) & 0xFFu));
          } else {
            d[ns] = deq_scale(sc);
          }
        }
        auto word = [&](int ns, int j) __attribute__((always_inline)) {
          return j == 0 ? wreg[ns].x : j == 1 ? wreg[ns].y : j == 2 ? wreg[ns].z : wreg[ns].w;
        };
        if constexpr (kPipe) {
          // Software pipeline: slice j's MFMAs run while the next slice's
          // words are dequantized, one MFMA issued between every four VALU
          // instructions (a 32x32x16 MFMA holds the matrix unit for about
          // eight wave64 VALU issue slots, so four leave room for the other
          // wave on the SIMD).  The activation operands of slice j + 1 are
          // read from LDS during slice j as well (slice 0's at the top of
          // the step).
          auto read_a = [&](int j, u32x4 (&a)[MSE]) __attribute__((always_inline)) {
#pragma unroll
            for (int ms = 0; ms < MSE; ++ms) {
              const int R = ms * 32 + l32;
              a[ms] = *(const u32x4*)(st + R * kStepK + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
            }
          };
          u32x4 bcur[NS], bnext[NS], acur[MSE], anext[MSE];
          read_a(0, acur);
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) bcur[ns] = dequant8<ZP>(word(ns, 0), d[ns]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            if (j < 3) {
              read_a(j + 1, anext);
#pragma unroll
              for (int ns = 0; ns < NS; ++ns) bnext[ns] = dequant8<ZP>(word(ns, j + 1), d[ns]);
            }
#pragma unroll
            for (int ms = 0; ms < MSE; ++ms)
#pragma unroll
              for (int ns = 0; ns < NS; ++ns) acc[ms][ns] = mfma32(acur[ms], bcur[ns], acc[ms][ns]);
            if (j < 3) {
              __builtin_amdgcn_sched_group_barrier(0x100, MSE, 0);   // the next operand reads
              __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
#pragma unroll
              for (int i = 0; i < MSE * NS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) bcur[ns] = bnext[ns];
#pragma unroll
            for (int ms = 0; ms < MSE; ++ms) acur[ms] = anext[ms];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // word j of each code register feeds MFMA slice j
            u32x4 bop[NS];
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
              bop[ns] = dequant8<ZP>(j == 0 ? wreg[ns].x : j == 1 ? wreg[ns].y
                                                       : j == 2 ? wreg[ns].z : wreg[ns].w,
                                     d[ns]);
            u32x4 a[MSE];
#pragma unroll
            for (int ms = 0; ms < MSE; ++ms) {
              const int R = ms * 32 + l32;
              a[ms] = *(const u32x4*)(st + R * kStepK + 8 * ((4 * h + j) ^ ((R >> 1) & 7)));
            }
#pragma unroll
            for (int ms = 0; ms < MSE; ++ms)
#pragma unroll
              for (int ns = 0; ns < NS; ++ns) acc[ms][ns] = mfma32(a[ms], bop[ns], acc[ms][ns]);
          }
        }
      }
      if constexpr (kGroupW) {
        if constexpr (P == 3) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            load_w(step + 5 + i, wset[(decltype(pos)::value + 5 + i) % kWS]);
        }
      } else {
        load_w(step + kWS, wreg);
      }
    };

    if constexpr (kGroupW) {
      // the order of the steady state: codes of steps 0..3, then the
      // activations of steps 0..2, then codes of steps 4..7 (as issued at
      // the end of a step 4u + 3)
#pragma unroll
      for (int i = 0; i < 4; ++i) load_w(i, wset[i]);
      load_s(0, sraw);
      if constexpr (ZP) load_z(0, zraw);
      load_x(0, xs0);
      load_x(1, xs1);
      load_x(2, xs2);
#pragma unroll
      for (int i = 4; i < 8; ++i) load_w(i, wset[i]);
    } else {
      load_x(0, xs0);
      load_w(0, wset[0]);
      load_s(0, sraw);
      if constexpr (ZP) load_z(0, zraw);
      load_x(1, xs1);
      load_w(1, wset[1]);
      load_x(2, xs2);
#pragma unroll
      for (int i = 2; i < kWS; ++i) load_w(i, wset[i]);
    }
    // The steps and the epilogue, for MSE valid 32-row tiles
    // (accumulators of tiles that hold no valid row are never allocated).
    auto run_tile = [&](auto mse) __attribute__((always_inline)) {
      constexpr int MSE = decltype(mse)::value;
      f32x16 acc[MSE][NS];
#pragma unroll
      for (int ms = 0; ms < MSE; ++ms)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[ms][ns][v] = 0.0f;
      for (int step = 0; step < nstepsp; step += kU) {
        step_body(mse, std::integral_constant<int, 0>{}, step + 0, xs0, xs3, wset[0 % kWS], acc);
        step_body(mse, std::integral_constant<int, 1>{}, step + 1, xs1, xs0, wset[1 % kWS], acc);
        step_body(mse, std::integral_constant<int, 2>{}, step + 2, xs2, xs1, wset[2 % kWS], acc);
        step_body(mse, std::integral_constant<int, 3>{}, step + 3, xs3, xs2, wset[3 % kWS], acc);
        if constexpr (kU == 8) {
          step_body(mse, std::integral_constant<int, 4>{}, step + 4, xs0, xs3, wset[4 % kWS], acc);
          step_body(mse, std::integral_constant<int, 5>{}, step + 5, xs1, xs0, wset[5 % kWS], acc);
          step_body(mse, std::integral_constant<int, 6>{}, step + 6, xs2, xs1, wset[6 % kWS], acc);
          step_body(mse, std::integral_constant<int, 7>{}, step + 7, xs3, xs2, wset[7 % kWS], acc);
        }
      }
      // drain the loads of the padding steps before LDS is reused
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

      // ---- epilogue: lane holds D[8*(v/4) + 4*h + v%4][l32] of each tile
      if constexpr (SWI) {
        // the up waves park bf16(up) in the activation stages; the gate
        // waves combine it with their own bf16(gate).  Up wave u's element
        // (tile ms, row rl, column cw): for BM = 128 rows 0..63 in stage 0,
        // 64..127 in stage 1, 128 columns each; for BM = 32 stage u holds
        // that wave's 32 x 64 block.
        const int I = N >> 1;
        auto park = [&](int ms, int rl, int u, int cw) __attribute__((always_inline)) {
          if constexpr (BM == 32)
            return (u ? xs1 : xs0) + rl * WN + cw;
          else
            return (ms < 2 ? xs0 : xs1) + ((ms & 1) * 32 + rl) * (2 * WN) + u * WN + cw;
        };
        static_assert(BM == 32 || BM == 128, "parking layout");
        __syncthreads();   // every wave is done reading the activation stages
        if (wave >= 2) {
#pragma unroll
          for (int ms = 0; ms < MSE; ++ms) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rl = 8 * (v >> 2) + 4 * h + (v & 3);
#pragma unroll
              for (int ns = 0; ns < NS; ++ns)
                *park(ms, rl, wave & 1, ns * 32 + l32) = to_bf16(acc[ms][ns][v]);
            }
          }
        }
        __syncthreads();
        if (wave < 2) {
#pragma unroll
          for (int ms = 0; ms < MSE; ++ms) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rl = 8 * (v >> 2) + 4 * h + (v & 3);
              const int yr = orow[ms * 32 + rl];
              if (yr < 0) continue;
#pragma unroll
              for (int ns = 0; ns < NS; ++ns) {
                const int c = wave * WN + ns * 32 + l32;
                const int col = tile_n * (2 * WN) + c;
                if (col < I) {
                  const float g = bf16f(to_bf16(acc[ms][ns][v]));
                  const float u = bf16f(*park(ms, rl, wave, ns * 32 + l32));
                  Y[(int64_t)yr * I + col] = to_bf16(silu_mul(g, u));
                }
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int ms = 0; ms < MSE; ++ms) {
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
                if constexpr (CMB)
                  __hip_atomic_store(&Y[(int64_t)yr * N + n], to_bf16(y), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
                else
                  Y[(int64_t)yr * N + n] = to_bf16(y);
              }
            }
          }
        }
        if constexpr (CMB) {
          __shared__ int last_tok[BM];
          __shared__ int n_last;
          constexpr int kCols = NW * WN;                  // weight rows (output columns) of the tile
          const int ntn = (N + kCols - 1) / kCols;
          // every wave's coherent stores are done before any count goes out
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (tid == 0) n_last = 0;
          __syncthreads();
          if (tid < BM) {
            const int f = orow[tid];
            if (f >= 0) {
              const int t = f / topk;
              int need = 0;
              for (int j = 0; j < topk; ++j) {
                const int e = topk_ids[(int64_t)t * topk + j];
                need += (e >= 0 && e < E) ? 1 : 0;
              }
              int32_t* c = cnt + (int64_t)t * ntn + tile_n;
              const int prev = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
              if (prev == need - 1) {
                __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last_tok[atomicAdd(&n_last, 1)] = t;
              }
            }
          }
          __syncthreads();
          const int nl = n_last;
          if (nl > 0) {
            const int col0 = tile_n * kCols;
            constexpr int kMaxK = 16;
            if ((N & 3) == 0 && (((uintptr_t)Out | (uintptr_t)Y) & 7) == 0) {
              // four columns per item, items of all tokens spread over the
              // workgroup, a pair's 8 bytes in one coherent load, every load
              // of an item issued before its sums
              constexpr int kG = kCols / 4;
              const int items = nl * kG;
              for (int it = tid; it < items; it += NT) {
                const int i = it / kG;
                const int n = col0 + 4 * (it - i * kG);
                const int t = last_tok[i];
                if (n < N) {
                  uint64_t hv[kMaxK];
                  float wv[kMaxK];
                  uint32_t vm = 0;   // bit j: pair j routed to an expert
#pragma unroll
                  for (int j = 0; j < kMaxK; ++j) {
                    hv[j] = 0;
                    wv[j] = 0.0f;
                    if (j < topk) {
                      const int64_t f = (int64_t)t * topk + j;
                      const int e = topk_ids[f];
                      if (e >= 0 && e < E) {
                        vm |= 1u << j;
                        wv[j] = cw[f];
                        hv[j] = __hip_atomic_load((const uint64_t*)&Y[f * N + n], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                      }
                    }
                  }
                  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
                  for (int j = 0; j < kMaxK; ++j) {
                    if ((vm >> j) & 1u) {
                      const uint32_t lo = (uint32_t)hv[j], hi = (uint32_t)(hv[j] >> 32);
                      a0 = __builtin_fmaf(wv[j], bf16_lo(lo), a0);
                      a1 = __builtin_fmaf(wv[j], bf16_hi(lo), a1);
                      a2 = __builtin_fmaf(wv[j], bf16_lo(hi), a2);
                      a3 = __builtin_fmaf(wv[j], bf16_hi(hi), a3);
                    }
                  }
                  *(uint64_t*)&Out[(int64_t)t * N + n] =
                      (uint64_t)pk_bf16(a0, a1) | ((uint64_t)pk_bf16(a2, a3) << 32);
                }
              }
            } else {
              for (int i = 0; i < nl; ++i) {
                const int t = last_tok[i];
                for (int cc = tid; cc < kCols; cc += NT) {
                  const int n = col0 + cc;
                  if (n < N) {
                    float s = 0.0f;
                    for (int j = 0; j < topk; ++j) {
                      const int64_t f = (int64_t)t * topk + j;
                      const int e = topk_ids[f];
                      if (e >= 0 && e < E) {
                        const uint16_t h = __hip_atomic_load(&Y[f * N + n], __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                        s = __builtin_fmaf(cw[f], bf16f(h), s);
                      }
                    }
                    Out[(int64_t)t * N + n] = to_bf16(s);
                  }
                }
              }
            }
          }
        }
      }
    };
    if constexpr (MOE) {
      // MFMA row tiles that hold valid rows (a run of one expert is often
      // a single 32-row tile; a run of 85 rows padded to 128 needs three)
      static_assert(MS == 1 || MS == 4, "one instantiation per row-tile count");
      if constexpr (MS == 1) {
        run_tile(std::integral_constant<int, 1>{});
      } else {
        if (ms_valid == 1)
          run_tile(std::integral_constant<int, 1>{});
        else if (ms_valid == 2)
          run_tile(std::integral_constant<int, 2>{});
        else if (ms_valid == 3)
          run_tile(std::integral_constant<int, 3>{});
        else
          run_tile(std::integral_constant<int, 4>{});
      }
    } else {
      run_tile(std::integral_constant<int, MS>{});
    }
  }
}

namespace {
constexpr int kWN = 64;
constexpr int kNW = 4;
constexpr int kBMDense = 128;   // dense prefill tile rows (two workgroups per CU)
constexpr int kBMMoe = 128;     // expert blocks of 64 rows and more
constexpr int kBMMoeSmall = 32; // expert blocks of 32 rows or fewer (few rows per expert)
constexpr int kWNMoeSmall = 32;  // weight rows per wave of the 32-row tile (64 measured the same)

// Tile rows of the grouped product.  With at most 32 rows per expert on
// average (and blocks of at most 32 rows) the product streams weights and
// the 32-row tile keeps more of them in flight; with more rows per expert a
// 32-row tile would split an expert into several runs that each re-read its
// weights, so the 128-row tile runs.
int64_t moe_tile_rows(int64_t T, int32_t k, int32_t E, int32_t B) {
  const int64_t mean_rows = (T * k + E - 1) / E;
  return (B <= kBMMoeSmall && mean_rows <= kBMMoeSmall) ? kBMMoeSmall : kBMMoe;
}
}  // namespace

namespace {
template <bool ZP, bool TL>
hipError_t launch_dense_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  const int64_t tiles = ((N + kNW * kWN - 1) / (kNW * kWN)) * ((M + kBMDense - 1) / kBMDense);
  const dim3 grid((unsigned)(((tiles + 7) / 8) * 8));   // whole rounds over the 8 XCDs
  if (K % 256 == 0)
    hipLaunchKernelGGL((k_gemm<kBMDense, kWN, kNW, false, true, false, ZP, TL>), grid,
                       dim3(kNW * 64), 0, st, X, (const uint32_t*)Wq, S, Z, Y, (int)M, (int)N,
                       (int)K, nullptr, nullptr, nullptr, nullptr, 0, 1, 1, 0, nullptr, nullptr,
                       nullptr, nullptr, 0);
  else
    hipLaunchKernelGGL((k_gemm<kBMDense, kWN, kNW, false, false, false, ZP, TL>), grid,
                       dim3(kNW * 64), 0, st, X, (const uint32_t*)Wq, S, Z, Y, (int)M, (int)N,
                       (int)K, nullptr, nullptr, nullptr, nullptr, 0, 1, 1, 0, nullptr, nullptr,
                       nullptr, nullptr, 0);
  return hipGetLastError();
}
}  // namespace

// Z == nullptr: symmetric codes; tiled: codes in the kernel-order layout
hipError_t launch_gemm_any(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                           bool tiled, hipStream_t st) {
  if (Z != nullptr)
    return tiled ? launch_dense_t<true, true>(X, Wq, S, Z, Y, M, N, K, st)
                 : launch_dense_t<true, false>(X, Wq, S, Z, Y, M, N, K, st);
  return tiled ? launch_dense_t<false, true>(X, Wq, S, nullptr, Y, M, N, K, st)
               : launch_dense_t<false, false>(X, Wq, S, nullptr, Y, M, N, K, st);
}

hipError_t launch_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  return launch_gemm_any(X, Wq, S, nullptr, Y, M, N, K, false, st);
}

hipError_t launch_gemm_zp(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  return launch_gemm_any(X, Wq, S, Z, Y, M, N, K, false, st);
}

// Slots (at most BM rows each: an alignment block, or one BM-row part of a
// larger block), padded to whole rounds of one run's worth over the 8 XCDs.
int64_t moe_gemm_slots(int64_t T, int32_t k, int32_t E, int32_t B) {
  const int64_t bm = moe_tile_rows(T, k, E, B);
  const int64_t cap = ((T * k + (int64_t)E * (B - 1) + B - 1) / B) * B;
  const int64_t bpw = bm >= B ? bm / B : 1;
  const int64_t ppb = B > bm ? (B + bm - 1) / bm : 1;   // slots per block
  const int64_t slots = (cap / B) * ppb;
  // 32-row tile: slots index runs; else groups of bpw slots per XCD
  const int64_t round = bm == kBMMoeSmall ? 8 : 8 * bpw;
  return (slots + round - 1) / round * round;
}

// Workgroups of one grouped launch: N-tiles x slots (a 1-D grid).
int64_t moe_gemm_workgroups(int64_t T, int32_t k, int32_t E, int64_t N, int32_t B, bool swiglu) {
  const int64_t wn = moe_tile_rows(T, k, E, B) == kBMMoeSmall ? kWNMoeSmall : kWN;
  const int64_t ntn = swiglu ? (N / 2 + 2 * wn - 1) / (2 * wn) : (N + kNW * wn - 1) / (kNW * wn);
  return ntn * moe_gemm_slots(T, k, E, B);
}

namespace {
// the fused combine's operands (all null / 0 without it)
struct CmbArgs {
  uint16_t* out = nullptr;
  int32_t* cnt = nullptr;
  const int32_t* topk_ids = nullptr;
  const float* w = nullptr;
};

template <int BM, int WN, bool SWI, bool ZP, bool TL, bool CMB = false>
hipError_t launch_grouped_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, const int32_t* sorted_ids, const int32_t* expert_ids,
                          const int32_t* ntpp, const float* topk_w, uint16_t* Y, int64_t T,
                          int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                          int32_t x_row_div, hipStream_t st, const CmbArgs& c = CmbArgs()) {
  // a fused SwiGLU workgroup covers 2 WN gate rows and the matching up rows
  const int64_t ntn = SWI ? (N / 2 + 2 * WN - 1) / (2 * WN) : (N + kNW * WN - 1) / (kNW * WN);
  const dim3 grid((unsigned)(ntn * moe_gemm_slots(T, k, E, B)));
  const int n_pairs = (int)(T * k);
  if (K % 256 == 0)
    hipLaunchKernelGGL((k_gemm<BM, WN, kNW, true, true, SWI, ZP, TL, CMB>), grid, dim3(kNW * 64), 0, st, X,
                       (const uint32_t*)Wq, S, Z, Y, 0, (int)N, (int)K, sorted_ids,
                       expert_ids, ntpp, topk_w, n_pairs, (int)B, (int)x_row_div, (int)E, c.out, c.cnt,
                       c.topk_ids, c.w, (int)k);
  else
    hipLaunchKernelGGL((k_gemm<BM, WN, kNW, true, false, SWI, ZP, TL, CMB>), grid, dim3(kNW * 64), 0, st, X,
                       (const uint32_t*)Wq, S, Z, Y, 0, (int)N, (int)K, sorted_ids,
                       expert_ids, ntpp, topk_w, n_pairs, (int)B, (int)x_row_div, (int)E, c.out, c.cnt,
                       c.topk_ids, c.w, (int)k);
  return hipGetLastError();
}

template <bool SWI, bool ZP, bool TL>
hipError_t launch_grouped_z(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                            const uint8_t* Z, const int32_t* sorted_ids,
                            const int32_t* expert_ids, const int32_t* ntpp, const float* topk_w,
                            uint16_t* Y, int64_t T, int32_t k, int32_t E, int64_t N, int64_t K,
                            int32_t B, int32_t x_row_div, hipStream_t st) {
  if (moe_tile_rows(T, k, E, B) == kBMMoeSmall)
    return launch_grouped_t<kBMMoeSmall, kWNMoeSmall, SWI, ZP, TL>(
        X, Wq, S, Z, sorted_ids, expert_ids, ntpp, topk_w, Y, T, k, E, N, K, B, x_row_div, st);
  return launch_grouped_t<kBMMoe, kWN, SWI, ZP, TL>(X, Wq, S, Z, sorted_ids, expert_ids, ntpp,
                                                    topk_w, Y, T, k, E, N, K, B, x_row_div, st);
}

// Z == nullptr: symmetric codes; else zero-point codes with Z [E, N, K/32].
// tiled: every expert's codes in the kernel-order layout.
template <bool SWI>
hipError_t launch_grouped(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, const int32_t* sorted_ids, const int32_t* expert_ids,
                          const int32_t* ntpp, const float* topk_w, uint16_t* Y, int64_t T,
                          int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                          int32_t x_row_div, bool tiled, hipStream_t st) {
  if (Z != nullptr)
    return tiled ? launch_grouped_z<SWI, true, true>(X, Wq, S, Z, sorted_ids, expert_ids, ntpp,
                                                     topk_w, Y, T, k, E, N, K, B, x_row_div, st)
                 : launch_grouped_z<SWI, true, false>(X, Wq, S, Z, sorted_ids, expert_ids, ntpp,
                                                      topk_w, Y, T, k, E, N, K, B, x_row_div, st);
  return tiled ? launch_grouped_z<SWI, false, true>(X, Wq, S, nullptr, sorted_ids, expert_ids,
                                                    ntpp, topk_w, Y, T, k, E, N, K, B, x_row_div,
                                                    st)
               : launch_grouped_z<SWI, false, false>(X, Wq, S, nullptr, sorted_ids, expert_ids,
                                                     ntpp, topk_w, Y, T, k, E, N, K, B, x_row_div,
                                                     st);
}
}  // namespace

hipError_t launch_moe_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* ntpp, const float* topk_w, uint16_t* Y, int64_t T,
                           int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                           int32_t x_row_div, bool tiled, hipStream_t st) {
  return launch_grouped<false>(X, Wq, S, Z, sorted_ids, expert_ids, ntpp, topk_w, Y, T, k, E, N,
                               K, B, x_row_div, tiled, st);
}

// The grouped down product with the top-k combine fused (symmetric codes;
// tiled: codes and scales in kernel order).  H2 receives the unweighted
// bf16 rows, Out the combined tokens, cnt the arrival counters (zero before,
// zero after).
hipError_t launch_moe_gemm_combine(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                                   const int32_t* sorted_ids, const int32_t* expert_ids,
                                   const int32_t* ntpp, const int32_t* topk_ids,
                                   const float* topk_w, uint16_t* H2, uint16_t* Out, int32_t* cnt,
                                   int64_t T, int32_t k, int32_t E, int64_t N, int64_t K,
                                   int32_t B, bool tiled, hipStream_t st) {
  CmbArgs c;
  c.out = Out;
  c.cnt = cnt;
  c.topk_ids = topk_ids;
  c.w = topk_w;
  if (moe_tile_rows(T, k, E, B) == kBMMoeSmall)
    return tiled ? launch_grouped_t<kBMMoeSmall, kWNMoeSmall, false, false, true, true>(
                       A, Wq, S, nullptr, sorted_ids, expert_ids, ntpp, nullptr, H2, T, k, E, N, K,
                       B, 1, st, c)
                 : launch_grouped_t<kBMMoeSmall, kWNMoeSmall, false, false, false, true>(
                       A, Wq, S, nullptr, sorted_ids, expert_ids, ntpp, nullptr, H2, T, k, E, N, K,
                       B, 1, st, c);
  return tiled ? launch_grouped_t<kBMMoe, kWN, false, false, true, true>(
                     A, Wq, S, nullptr, sorted_ids, expert_ids, ntpp, nullptr, H2, T, k, E, N, K, B,
                     1, st, c)
               : launch_grouped_t<kBMMoe, kWN, false, false, false, true>(
                     A, Wq, S, nullptr, sorted_ids, expert_ids, ntpp, nullptr, H2, T, k, E, N, K, B,
                     1, st, c);
}

// The arrival counters of w4a16_moe_gemm_combine_noalloc: a fixed device
// array per GPU, held until the process ends, zero when the library loads
// and left zero by every call.  On the host `scratch` names a stand-in, not
// a device address: each device's copy is looked up once, with that device
// current, and only the looked-up address is passed to a kernel.
static __device__ __align__(256) int32_t scratch[kCombineScratchWords];

hipError_t combine_scratch(int32_t** words) {
  static std::mutex mu;
  static int32_t* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = (int32_t*)p;
  }
  *words = ptrs[dev];
  return hipSuccess;
}

// Arrival counters of the fused combine: one per token and weight-row tile.
int64_t moe_combine_counters(int64_t T, int32_t k, int32_t E, int64_t N, int32_t B) {
  const int64_t cols = moe_tile_rows(T, k, E, B) == kBMMoeSmall ? kNW * kWNMoeSmall : kNW * kWN;
  return T * ((N + cols - 1) / cols);
}

hipError_t launch_moe_gemm_swiglu(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                                  const uint8_t* Z, const int32_t* sorted_ids,
                                  const int32_t* expert_ids, const int32_t* ntpp, uint16_t* A,
                                  int64_t T, int32_t k, int32_t E, int64_t I, int64_t K, int32_t B,
                                  int32_t x_row_div, bool tiled, hipStream_t st) {
  return launch_grouped<true>(X, Wq, S, Z, sorted_ids, expert_ids, ntpp, nullptr, A, T, k, E,
                              2 * I, K, B, x_row_div, tiled, st);
}

}  // namespace w4
