// W4A16 product for small M (decode): Y[M, N] = X[M, K] * dequant(W)^T.
//
// Method: "INT4 QAT end-to-end for RL" §4 (INT4 weights are dequantized in
// registers and multiplied against BF16 activations on BF16 matrix units);
// "Quantization basics: from FP32 to INT4" §2.1 (w = q * s, z = 0) and the
// tutorial's opening remark that decode reads every weight once per token,
// so this path is bound by HBM bandwidth.
//
// Arithmetic.  Within one 32-element group every weight shares the scale
// s, so   sum_k x_k q_k s = s * sum_k x_k q_k :  the MFMA contracts the
// integer codes of exactly one group and the fp32 partial is scaled once
// (4 FMAs per lane per 16 x 32 weights instead of one per weight).  A code
// becomes a bf16 MFMA operand with one AND-OR: the bit pattern 0x4300 | n
// is the bf16 number 128 + n, and n = q + 8 after flipping each nibble's
// top bit (XOR 0x8 per nibble turns two's complement into offset binary).
// The MFMA therefore sums x * (136 + q); its C operand starts at
// -136 * sum_k x_k (itself one MFMA of X against the constant -136), so the
// result is sum_k x_k q_k up to fp32 rounding.  Exact integer inputs stay
// exact.  The scaled product is q * s exactly, not bf16(q * s): within the
// fp32-accumulation tolerance of the definition.
//
// Mapping (MI355X).  One workgroup of 16 waves per CU; wave w owns a
// 256-element K slice (two 128-element "chunks") and keeps its slice of X
// in registers for the whole kernel (loaded once, reused for every weight
// row).  The workgroup walks TPW tiles of 16 weight rows.  For one chunk,
// lane (n = l % 16, kq = l / 16) loads 16 bytes = group 4c + kq of row n
// (a 16-row tile is 16 contiguous 64-byte runs) with a raw buffer load:
// rows or groups past the end read as zero in hardware, so no load sits
// behind a branch and all of them are in flight together.  A 4 x 4
// transpose across the four 16-lane rows (v_permlane32_swap +
// v_permlane16_swap) then gives lane (n, kq) word kq of all four groups,
// which is exactly its B operand slot for a one-group MFMA
// (v_mfma_f32_16x16x32_bf16: A = X rows, B = weight rows).  Per-wave
// partials meet in LDS (fixed wave order, deterministic) once per tile;
// each output is owned by one thread across tiles and K passes.
#include "common.h"

namespace w4 {

namespace {

constexpr int kWaves = 16;
constexpr int kCPW = 2;                 // 128-element chunks per wave per pass
constexpr int kPassK = kWaves * kCPW * 128;
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past any buffer: reads 0
constexpr uint32_t kNeg136 = 0xC308C308u;   // bf16 pair (-136, -136)
constexpr int kNonTemporal = 2;             // buffer-load cache policy: streaming

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 8 bf16 from 16 bytes of X in the slot order the weight operand uses:
// (x0, x4), (x1, x5), (x2, x6), (x3, x7).
__device__ __forceinline__ u32x4 x_slots(u32x4 d) {
  u32x4 o;
  o.x = (d.x & 0xFFFFu) | (d.z << 16);
  o.y = (d.x >> 16) | (d.z & 0xFFFF0000u);
  o.z = (d.y & 0xFFFFu) | (d.w << 16);
  o.w = (d.y >> 16) | (d.w & 0xFFFF0000u);
  return o;
}

// One packed word (8 codes, nibble t = element t) -> bf16 operand holding
// 136 + q in slot order (t0, t4), (t1, t5), (t2, t6), (t3, t7).  Each pair
// is one v_bitop3: where the mask 0x000F000F is set the result is the
// nibble XOR 8 (two's complement -> offset binary), elsewhere the bits of
// 0x43004300 (bf16 128 with a zero mantissa); truth table 0x6A =
// "mask ? x ^ c : c" with c = 0x43084308.
__device__ __forceinline__ uint32_t code_pair(uint32_t x) {
  return __builtin_amdgcn_bitop3_b32(x, 0x000F000Fu, 0x43084308u, 0x6A);
}
__device__ __forceinline__ u32x4 code_slots(uint32_t w) {
  return u32x4{code_pair(w), code_pair(w >> 4), code_pair(w >> 8), code_pair(w >> 12)};
}

// 4 x 4 transpose across the four 16-lane rows: on entry lane row r holds
// words 0..3 of group r; on exit it holds word r of groups 0..3.
__device__ __forceinline__ u32x4 transpose_rows(u32x4 v) {
  auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return u32x4{c[0], c[1], d[0], d[1]};
}

// Copies of v with all four 16-lane rows replaced by row 0, 1, 2, 3.
__device__ __forceinline__ void broadcast_rows(uint32_t v, uint32_t out[4]) {
  auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);      // [r0 r1 r0 r1], [r2 r3 r2 r3]
  auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
  auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

}  // namespace

// MT: 16-row activation tiles (M <= 16 * MT).  SALIGNED: K / 32 is a
// multiple of 8 (a wave's eight scales of one row are one 16-byte load).  PF: weight
// tiles in flight per wave (a ring of registers; bounded by the register
// budget of 16 resident waves per CU).  The workgroup covers T tiles of 16
// weight rows (T <= max_tpw(MT)), about one workgroup per CU.
constexpr int max_tpw(int MT) { return MT == 1 ? 4 : 3; }   // LDS budget

template <int MT, bool SALIGNED, int T, int PF>
__global__ __launch_bounds__(kWaves * 64) void k_decode(const uint16_t* __restrict__ X,
                                                         const uint32_t* __restrict__ Wq,
                                                         const uint16_t* __restrict__ S,
                                                         uint16_t* __restrict__ Y, int M,
                                                         int N, int K) {
  static_assert(PF >= 1 && PF <= 3 && PF <= T && T <= max_tpw(MT), "tile ring");
  constexpr int MR = MT * 16;
  constexpr int PSTR = MR + 4;                     // LDS row stride (floats)
  // CFOLD: the -136 * sum(x) term is precomputed per group and enters as
  // the MFMA C operand; otherwise a second MFMA against -136 adds it
  // (fewer registers, more matrix-core cycles: used for 32 rows).
  constexpr bool CFOLD = false;
  constexpr int NC = CFOLD ? kCPW : 1;
  constexpr int TMAX = T;
  // per-wave partial sums of every tile: each wave runs through its tiles
  // on its own (no barrier between tiles) and the sum over waves happens
  // once per K pass
  __shared__ __attribute__((aligned(16))) float part[TMAX][kWaves][16][PSTR];
  __shared__ float ybuf[TMAX][MR * 16];            // partials across K passes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int kq = lane >> 4;
  const int G = K >> 5;
  const int C = (G + 3) >> 2;
  const uint32_t rowb = (uint32_t)K >> 1;          // packed bytes per weight row
  const int n0 = blockIdx.x * (T * 16);
  const int rows = min(T * 16, N - n0);
  const int ntiles = (rows + 15) >> 4;

  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wr = rsrc(Wq + (size_t)n0 * (K >> 3), (uint32_t)rows * rowb);
  const __amdgpu_buffer_rsrc_t sr = rsrc(S + (size_t)n0 * G, (uint32_t)rows * (uint32_t)G * 2u);

  const int npass = (K + kPassK - 1) / kPassK;

  for (int pass = 0; pass < npass; ++pass) {
    // ---- activation slice of this wave: operands and the offset term
    u32x4 xop[kCPW][4][MT];
    f32x4 cst[NC][4][MT];
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc) {
      const int c = pass * (kWaves * kCPW) + wave * kCPW + cc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = 4 * c + j;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + n16;
          const uint32_t off = (g < G && m < M)
                                   ? ((uint32_t)m * (uint32_t)K + 32u * g + 8u * kq) * 2u
                                   : kOOB;
          xop[cc][j][mt] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
      }
    }
    const u32x4 neg136 = u32x4{kNeg136, kNeg136, kNeg136, kNeg136};

    // ---- scales: one load per wave and pass.  Lane row r (lanes 16r ..
    // 16r + 15) fetches the wave's eight group scales of row n16 of tile r
    // (16 bytes); every tile's row is then broadcast to all four lane rows.
    // Rows past the end read as zero; a group block past K is clamped into
    // the row (its codes and activations are zero, so the scale is unused).
    const int g0 = pass * (kWaves * kCPW * 4) + wave * (kCPW * 4);
    u32x4 sraw;                                        // this lane row's 8 scales
    {
      const uint32_t srow = (uint32_t)(kq * 16 + n16);
      u32x4 raw;
      if constexpr (SALIGNED) {
        const uint32_t gb = (uint32_t)min(g0, G - 8);
        raw = __builtin_amdgcn_raw_buffer_load_b128(sr, (srow * (uint32_t)G + gb) * 2u, 0, 0);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gj = g0 + j;
          const uint32_t soff = (gj < G) ? (srow * (uint32_t)G + gj) * 2u : kOOB;
          h[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
        }
        raw = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16)};
      }
      sraw = raw;
    }

    // ---- weight ring.  Rows of a tile past the end lie beyond the
    // buffer's size and read as zero, so loads are never conditional (a
    // condition that is the same for the whole wave would be compiled into
    // a branch around the load, and a wait inside it); the only guards are
    // per-lane selects.  Codes are read once: non-temporal loads.
    u32x4 wv[PF][kCPW];
    auto load_tile = [&](int slot, int t) {
      const uint32_t nl = (uint32_t)(t * 16 + n16);          // row within the workgroup
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) {
        const int c = pass * (kWaves * kCPW) + wave * kCPW + cc;
        const int g = 4 * c + kq;
        const uint32_t woff = (g < G) ? nl * rowb + 16u * (uint32_t)g : kOOB;
        wv[slot][cc] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, 0, kNonTemporal);
      }
    };

    // one tile: one-group MFMAs, scale, cross-wave sum, result
    auto compute_tile = [&](int slot, int t) {
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // tile t's scales, broadcast from lane row t (kept per tile: registers)
      uint32_t sct[4];
      {
        const uint32_t rw[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t b[4];
          broadcast_rows(rw[d], b);
          sct[d] = b[t];
        }
      }
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) {
        const u32x4 u = transpose_rows(wv[slot][cc]);
        const uint32_t words[4] = {u.x, u.y, u.z, u.w};
        const uint32_t s01 = sct[2 * cc], s23 = sct[2 * cc + 1];
        const float sc[4] = {bf16_lo(s01), bf16_hi(s01), bf16_lo(s23), bf16_hi(s23)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 b = code_slots(words[j]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            f32x4 d;
            if constexpr (CFOLD) {
              d = mfma16(xop[cc][j][mt], b, cst[cc][j][mt]);
            } else {
              d = mfma16(xop[cc][j][mt], b, f32x4{0.f, 0.f, 0.f, 0.f});
              d = mfma16(xop[cc][j][mt], neg136, d);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][r] = __builtin_fmaf(d[r], sc[j], acc[mt][r]);
          }
        }
      }
      // lane holds D[m = mt*16 + 4 kq + r][n = n16]
      float* pp = &part[t][wave][n16][0];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) *(f32x4*)(pp + mt * 16 + 4 * kq) = acc[mt];
    };

    // called once the weight prologue is in flight: wait for X, put it in
    // slot order (and precompute the offset term when folded)
    auto convert_x = [&]() {
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            xop[cc][j][mt] = x_slots(xop[cc][j][mt]);
            if constexpr (CFOLD)
              cst[cc][j][mt] = mfma16(xop[cc][j][mt], neg136, f32x4{0.f, 0.f, 0.f, 0.f});
          }
    };

    // tiles are unrolled at compile time (TMAX <= 4); a tile past the end
    // costs its (out-of-range, traffic-free) loads and skips its compute
#pragma unroll
    for (int t = 0; t < PF - 1; ++t) load_tile(t, t);
    if constexpr (PF == 1) load_tile(0, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads above ahead of the X wait
    convert_x();
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if constexpr (PF > 1) {
        if (t + PF - 1 < TMAX) load_tile((t + PF - 1) % PF, t + PF - 1);
      }
      if (t < ntiles) compute_tile(t % PF, t);
      if constexpr (PF == 1) {
        if (t + 1 < TMAX) load_tile(0, t + 1);
      }
    }

    // ---- sum over waves in wave order (deterministic); one thread per output
    __syncthreads();
    for (int o = tid; o < ntiles * MR * 16; o += kWaves * 64) {
      const int t = o / (MR * 16);
      const int m = (o >> 4) % MR;
      const int n = o & 15;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += part[t][w][n][m];
      const int row = t * 16 + n;
      if (npass > 1) {
        sum += (pass == 0) ? 0.0f : ybuf[t][m * 16 + n];
        ybuf[t][m * 16 + n] = sum;
      }
      if (pass == npass - 1 && m < M && row < rows) Y[(size_t)m * N + n0 + row] = to_bf16(sum);
    }
    if (npass > 1) __syncthreads();   // part is rewritten by the next pass
  }
}


// M <= 16, group-outer.  All T tiles' codes of the wave's two chunks are in
// registers at once, so for each group the offset term (X against -136) is
// one MFMA whose result is the C operand of the T tile MFMAs: one MFMA per
// group and tile.  RM: rows of each lane's D fragment that are accumulated
// (for M = 1 only row 0 of lane row 0 exists; the other rows are skipped).
template <bool SALIGNED, int T, int RM>
__global__ __launch_bounds__(kWaves * 64) void k_decode1(const uint16_t* __restrict__ X,
                                                          const uint32_t* __restrict__ Wq,
                                                          const uint16_t* __restrict__ S,
                                                          uint16_t* __restrict__ Y, int M, int N,
                                                          int K) {
  static_assert(T >= 1 && T <= 4 && (RM == 1 || RM == 4), "decode shape");
  constexpr int PSTR = 20;                         // LDS row stride (floats)
  constexpr int WSTR = 16 * PSTR + 4;              // per-wave block: padded off the bank period
  __shared__ __attribute__((aligned(16))) float part[T][kWaves][WSTR];
  __shared__ float ybuf[T][256];                   // partials across K passes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int kq = lane >> 4;
  const int G = K >> 5;
  const uint32_t rowb = (uint32_t)K >> 1;          // packed bytes per weight row
  const int n0 = blockIdx.x * (T * 16);
  const int rows = min(T * 16, N - n0);
  const int ntiles = (rows + 15) >> 4;

  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wr = rsrc(Wq + (size_t)n0 * (K >> 3), (uint32_t)rows * rowb);
  const __amdgpu_buffer_rsrc_t sr = rsrc(S + (size_t)n0 * G, (uint32_t)rows * (uint32_t)G * 2u);
  const int npass = (K + kPassK - 1) / kPassK;
  const u32x4 neg136 = u32x4{kNeg136, kNeg136, kNeg136, kNeg136};

  for (int pass = 0; pass < npass; ++pass) {
    const int c0 = pass * (kWaves * kCPW) + wave * kCPW;   // first chunk of this wave
    // ---- activations (issued first: the first wait is for them alone)
    u32x4 xop[kCPW][4];
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = 4 * (c0 + cc) + j;
        const uint32_t off = (g < G && n16 < M)
                                 ? ((uint32_t)n16 * (uint32_t)K + 32u * g + 8u * kq) * 2u
                                 : kOOB;
        xop[cc][j] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
      }
    // ---- scales: lane row r fetches the wave's 8 group scales of row n16
    // of tile r (rows past the end read zero; a group block past K is
    // clamped into the row, where codes and activations are zero)
    const int g0 = 4 * c0;
    u32x4 sraw;
    {
      const uint32_t srow = (uint32_t)(kq * 16 + n16);
      if constexpr (SALIGNED) {
        const uint32_t gb = (uint32_t)min(g0, G - 8);
        sraw = __builtin_amdgcn_raw_buffer_load_b128(sr, (srow * (uint32_t)G + gb) * 2u, 0, 0);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gj = g0 + j;
          const uint32_t soff = (gj < G) ? (srow * (uint32_t)G + gj) * 2u : kOOB;
          h[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
        }
        sraw = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                     h[6] | (h[7] << 16)};
      }
    }
    // ---- codes of every tile (rows past the end read zero); a row's two
    // chunks are adjacent requests (one 128-byte line)
    u32x4 wv[T][kCPW];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint32_t nl = (uint32_t)(t * 16 + n16);
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) {
        const int g = 4 * (c0 + cc) + kq;
        const uint32_t woff = (g < G) ? nl * rowb + 16u * (uint32_t)g : kOOB;
        wv[t][cc] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the first wait

#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j) xop[cc][j] = x_slots(xop[cc][j]);
    uint32_t sct[T][4];                  // [tile][dword]: 8 bf16 scales
    {
      const uint32_t rw[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t b[4];
        broadcast_rows(rw[d], b);
#pragma unroll
        for (int t = 0; t < T; ++t) sct[t][d] = b[t];
      }
    }

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc) {
      u32x4 u[T];
#pragma unroll
      for (int t = 0; t < T; ++t) u[t] = transpose_rows(wv[t][cc]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 cst = mfma16(xop[cc][j], neg136, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t word = j == 0 ? u[t].x : j == 1 ? u[t].y : j == 2 ? u[t].z : u[t].w;
          const f32x4 d = mfma16(xop[cc][j], code_slots(word), cst);
          const uint32_t sp = sct[t][2 * cc + (j >> 1)];
          const float sc = (j & 1) ? bf16_hi(sp) : bf16_lo(sp);
#pragma unroll
          for (int r = 0; r < RM; ++r) acc[t][r] = __builtin_fmaf(d[r], sc, acc[t][r]);
        }
      }
    }
    // lane holds D[m = 4 kq + r][n = n16] of every tile
#pragma unroll
    for (int t = 0; t < T; ++t) *(f32x4*)&part[t][wave][n16 * PSTR + 4 * kq] = acc[t];

    // ---- sum over waves in a fixed order (deterministic): one thread per
    // output, rows m < M only
    __syncthreads();
    const int mrows = min(M, 16);
    const int nout = ntiles * mrows * 16;
    for (int o = tid; o < nout; o += kWaves * 64) {
      const int t = o / (mrows * 16);
      const int m = (o >> 4) % mrows;
      const int n = o & 15;
      const int e = n * PSTR + m;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += part[t][w][e];
      const int row = t * 16 + n;
      if (npass > 1) {
        sum += (pass == 0) ? 0.0f : ybuf[t][m * 16 + n];
        ybuf[t][m * 16 + n] = sum;
      }
      if (pass == npass - 1 && row < rows) Y[(size_t)m * N + n0 + row] = to_bf16(sum);
    }
    if (npass > 1) __syncthreads();   // part is rewritten by the next pass
  }
}

namespace {

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

template <int MT, bool SA, int T>
hipError_t run_decode_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                        int64_t M, int64_t N, int64_t K, hipStream_t st) {
  constexpr int PFMAX = MT == 1 ? (SA ? 3 : 2) : 1;
  constexpr int PF = T < PFMAX ? T : PFMAX;
  const int64_t blocks = (N + T * 16 - 1) / (T * 16);
  hipLaunchKernelGGL((k_decode<MT, SA, T, PF>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, st,
                     X, (const uint32_t*)Wq, S, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <bool SA, int T, int RM>
hipError_t run_decode1_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                         int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t blocks = (N + T * 16 - 1) / (T * 16);
  hipLaunchKernelGGL((k_decode1<SA, T, RM>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, st, X,
                     (const uint32_t*)Wq, S, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <bool SA, int RM>
hipError_t run_decode1(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = cu_count();
  const int64_t tpw = (tiles + cus - 1) / cus;
  if (tpw <= 1) return run_decode1_t<SA, 1, RM>(X, Wq, S, Y, M, N, K, st);
  if (tpw == 2) return run_decode1_t<SA, 2, RM>(X, Wq, S, Y, M, N, K, st);
  if (tpw == 3) return run_decode1_t<SA, 3, RM>(X, Wq, S, Y, M, N, K, st);
  return run_decode1_t<SA, 4, RM>(X, Wq, S, Y, M, N, K, st);
}

template <int MT, bool SA>
hipError_t run_decode(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                      int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = cu_count();
  const int64_t tpw = (tiles + cus - 1) / cus;
  if (tpw <= 1) return run_decode_t<MT, SA, 1>(X, Wq, S, Y, M, N, K, st);
  if (tpw == 2) return run_decode_t<MT, SA, 2>(X, Wq, S, Y, M, N, K, st);
  if (tpw == 3 || MT == 2) return run_decode_t<MT, SA, 3>(X, Wq, S, Y, M, N, K, st);
  return run_decode_t<MT, SA, max_tpw(MT)>(X, Wq, S, Y, M, N, K, st);
}

}  // namespace

hipError_t launch_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const bool sa = ((K >> 5) & 7) == 0;
  if (M == 1)
    return sa ? run_decode1<true, 1>(X, Wq, S, Y, M, N, K, st)
              : run_decode1<false, 1>(X, Wq, S, Y, M, N, K, st);
  if (M <= 16)
    return sa ? run_decode1<true, 4>(X, Wq, S, Y, M, N, K, st)
              : run_decode1<false, 4>(X, Wq, S, Y, M, N, K, st);
  return sa ? run_decode<2, true>(X, Wq, S, Y, M, N, K, st)
            : run_decode<2, false>(X, Wq, S, Y, M, N, K, st);
}

}  // namespace w4
