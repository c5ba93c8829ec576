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
// exact.  The scaled product is q * s exactly, not bf16(q * s).  Per
// product the two differ by at most 2^-9 |q s|, so over K terms the output
// moves by ~2^-9/sqrt(3) * 0.6 * sqrt(K) |x| |w| (about 1e-3 of the
// output's spread), while the tolerance of the definition has a fixed
// absolute part.  Above K = 16384 (EXACT) each code is therefore
// dequantized to w' = bf16(q s) with the 17-op fma_mix step of the tiled
// product and the MFMA accumulates across groups: the definition's
// weights, at about 2x the VALU per weight.
//
// Mapping (MI355X).  One workgroup of 16 waves per CU; wave w owns a
// 256-element K slice (two 128-element "chunks") and keeps its slice of X
// in registers (loaded once, reused for every weight row).  The workgroup
// covers T tiles of 16 weight rows and each wave holds the codes of all T
// tiles of its slice at once.  For one chunk, lane (n = l % 16, kq = l / 16)
// loads 16 bytes = group 4c + kq of row n (a 16-row tile is 16 contiguous
// 64-byte runs) with a raw buffer load: rows or groups past the end read
// as zero in hardware, so no load sits behind a branch and all of them are
// in flight together.  A 4 x 4 transpose across the four 16-lane rows
// (v_permlane32_swap + v_permlane16_swap) then gives lane (n, kq) word kq
// of all four groups, which is exactly its B operand slot for a one-group
// MFMA (v_mfma_f32_16x16x32_bf16: A = X rows, B = weight rows).  Groups
// are the outer loop, so the offset term (X against -136) is one MFMA per
// group shared by the T tile MFMAs.  Per-wave partials meet in LDS (fixed
// wave order, deterministic) once per K pass; each output is owned by one
// thread.
//
// Zero-point weights (ZP; "Quantization basics: from FP32 to INT4" §2.1 and
// §2.3, w' = (q - z) s with unsigned q): the code operand is 128 + q (no
// flip), and the C operand of tile t's MFMA is X against the constant
// column -(128 + z) of each weight row (bf16 0xC300 | z, exact), one MFMA
// per tile and group, so the MFMA returns sum_k x_k (q_k - z) and the scale
// step is unchanged.
#include "common.h"

namespace w4 {

namespace {

constexpr int kWaves = 16;
constexpr int kCPW = 2;                 // 128-element chunks per wave per pass
constexpr int kPassK = kWaves * kCPW * 128;
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past any buffer: reads 0
constexpr uint32_t kNeg136 = 0xC308C308u;   // bf16 pair (-136, -136)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 8 bf16 from 16 bytes of X in the slot order the weight operand uses:
// (x0, x4), (x1, x5), (x2, x6), (x3, x7).
// One v_perm_b32 per dword: bytes 0-3 select from the second operand,
// 4-7 from the first.
__device__ __forceinline__ u32x4 x_slots(u32x4 d) {
  u32x4 o;
  o.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
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
// unsigned codes: 128 + q, no flip (one v_and_or_b32)
__device__ __forceinline__ uint32_t code_pair_u(uint32_t x) {
  return (x & 0x000F000Fu) | 0x43004300u;
}
template <bool ZP>
__device__ __forceinline__ u32x4 code_slots(uint32_t w) {
  if constexpr (ZP)
    return u32x4{code_pair_u(w), code_pair_u(w >> 4), code_pair_u(w >> 8), code_pair_u(w >> 12)};
  else
    return u32x4{code_pair(w), code_pair(w >> 4), code_pair(w >> 8), code_pair(w >> 12)};
}

// bf16 pair (-(128 + z), -(128 + z)) from byte J of a word of zero points
template <int J>
__device__ __forceinline__ uint32_t zp_offset_pair(uint32_t zw) {
  constexpr uint32_t sel = 0x0C000C00u | ((uint32_t)J << 16) | (uint32_t)J;   // 0x0C: zero byte
  return __builtin_amdgcn_perm(0u, zw, sel) | 0xC300C300u;
}

// This lane row's 8 zero points of weight row srow, groups g0 .. g0 + 7
// (two dwords); the SALIGNED block is clamped into the row like the scales.
template <bool SALIGNED>
__device__ __forceinline__ u32x2 load_zp8(__amdgpu_buffer_rsrc_t zr, uint32_t srow, int g0, int G) {
  if constexpr (SALIGNED) {
    const uint32_t gb = (uint32_t)min(g0, G - 8);
    return __builtin_amdgcn_raw_buffer_load_b64(zr, srow * (uint32_t)G + gb, 0, 0);
  } else {
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int gj = g0 + j;
      const uint32_t zoff = (gj < G) ? srow * (uint32_t)G + (uint32_t)gj : kOOB;
      b[j] = __builtin_amdgcn_raw_buffer_load_b8(zr, zoff, 0, 0);
    }
    return u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                 b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
  }
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

// 16 bytes per lane from a buffer straight into LDS (buffer_load ... lds):
// lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           off, 0, 0, 0);
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

// M <= 16.  SALIGNED: K / 32 is a multiple of 8 (a wave's eight scales of
// one row are one 16-byte load).  T: tiles of 16 weight rows per workgroup.
// RM: rows of each lane's D fragment that are accumulated (for M = 1 only
// row 0 of lane row 0 exists; the other rows are skipped).
template <bool SALIGNED, int T, int RM, bool ZP, bool EXACT>
__global__ __launch_bounds__(kWaves * 64) void k_decode16(const uint16_t* __restrict__ X,
                                                          const uint32_t* __restrict__ Wq,
                                                          const uint16_t* __restrict__ S,
                                                          const uint8_t* __restrict__ Z,
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
  const __amdgpu_buffer_rsrc_t zr =
      rsrc(ZP ? Z + (size_t)n0 * G : nullptr, ZP ? (uint32_t)rows * (uint32_t)G : 0u);
  const int npass = (K + kPassK - 1) / kPassK;
  const u32x4 neg136 = u32x4{kNeg136, kNeg136, kNeg136, kNeg136};

  for (int pass = 0; pass < npass; ++pass) {
    const int c0 = pass * (kWaves * kCPW) + wave * kCPW;   // first chunk of this wave
    // ---- codes of every tile first, so the HBM stream starts at once (rows
    // past the end read zero); a row's two chunks are adjacent requests (one
    // 128-byte line)
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
    // ---- activations (L2 hits after the first CU's request)
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
    u32x2 zraw = u32x2{0u, 0u};
    if constexpr (ZP) zraw = load_zp8<SALIGNED>(zr, (uint32_t)(kq * 16 + n16), g0, G);
    __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the first wait

#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if constexpr (!EXACT) xop[cc][j] = x_slots(xop[cc][j]);
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
      uint32_t zc[T];                    // ZP: tile t's zero points of this chunk's groups
      if constexpr (ZP) {
        uint32_t b[4];
        broadcast_rows(cc == 0 ? zraw.x : zraw.y, b);
#pragma unroll
        for (int t = 0; t < T; ++t) zc[t] = b[t];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (EXACT) {
          // w' = bf16(q s) (or bf16((q - z) s)) per weight, the MFMA
          // accumulating across groups
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint32_t word = j == 0 ? u[t].x : j == 1 ? u[t].y : j == 2 ? u[t].z : u[t].w;
            const uint32_t sp = sct[t][2 * cc + (j >> 1)];
            const float sc = (j & 1) ? bf16_hi(sp) : bf16_lo(sp);
            DeqScale dq;
            if constexpr (ZP)
              dq = deq_scale_zp(sc, (float)((zc[t] >> (8 * j)) & 0xFFu));
            else
              dq = deq_scale(sc);
            acc[t] = mfma16(xop[cc][j], dequant8<ZP>(word, dq), acc[t]);
          }
          continue;
        }
        const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 cst = zero4;
        if constexpr (!ZP) cst = mfma16(xop[cc][j], neg136, zero4);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t word = j == 0 ? u[t].x : j == 1 ? u[t].y : j == 2 ? u[t].z : u[t].w;
          f32x4 ct = cst;
          if constexpr (ZP) {
            const uint32_t zz = j == 0   ? zp_offset_pair<0>(zc[t])
                                : j == 1 ? zp_offset_pair<1>(zc[t])
                                : j == 2 ? zp_offset_pair<2>(zc[t])
                                         : zp_offset_pair<3>(zc[t]);
            ct = mfma16(xop[cc][j], u32x4{zz, zz, zz, zz}, zero4);
          }
          const f32x4 d = mfma16(xop[cc][j], code_slots<ZP>(word), ct);
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

// 16 < M <= 32, group-outer over two 16-row activation halves.  Half 0's
// X sits in registers as for M <= 16; half 1's X goes straight into this
// wave's LDS region (direct-to-LDS loads issued with the others) and is read
// per group where it is used.  Each converted code word feeds the MFMAs of
// both halves.  The region then takes the wave's partial sums.
template <bool SALIGNED, int T, bool ZP, bool EXACT>
__global__ __launch_bounds__(kWaves * 64) void k_decode32(const uint16_t* __restrict__ X,
                                                          const uint32_t* __restrict__ Wq,
                                                          const uint16_t* __restrict__ S,
                                                          const uint8_t* __restrict__ Z,
                                                          uint16_t* __restrict__ Y, int M, int N,
                                                          int K) {
  static_assert(T >= 1 && T <= 3, "decode shape");
  constexpr int PSTR = 36;                         // LDS row stride (floats): 32 rows + pad
  constexpr int WSTR = 16 * PSTR + 4;              // per-tile block: padded off the bank period
  constexpr int XREG = kCPW * 4 * 256;             // floats: 8 x 1 KB of half-1 activations
  constexpr int REGION = T * WSTR > XREG ? T * WSTR : XREG;
  __shared__ __attribute__((aligned(16))) float lds[kWaves][REGION];
  __shared__ float ybuf[T][32 * 16];               // partials across K passes

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
  const __amdgpu_buffer_rsrc_t zr =
      rsrc(ZP ? Z + (size_t)n0 * G : nullptr, ZP ? (uint32_t)rows * (uint32_t)G : 0u);
  const int npass = (K + kPassK - 1) / kPassK;
  const u32x4 neg136 = u32x4{kNeg136, kNeg136, kNeg136, kNeg136};

  for (int pass = 0; pass < npass; ++pass) {
    const int c0 = pass * (kWaves * kCPW) + wave * kCPW;   // first chunk of this wave
    // byte offset of lane (n16, kq)'s 16 activation bytes of group 4 c + j
    // in half hh (rows past M and groups past K read zero)
    auto x_off = [&](int hh, int cc, int j) {
      const int g = 4 * (c0 + cc) + j;
      const int row = 16 * hh + n16;
      return (g < G && row < M) ? ((uint32_t)row * (uint32_t)K + 32u * g + 8u * kq) * 2u : kOOB;
    };
    // ---- half 0's activations (issued first: the first wait is for them alone)
    u32x4 xop[kCPW][4];
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xop[cc][j] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off(0, cc, j), 0, 0);
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
        uint32_t hw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gj = g0 + j;
          const uint32_t soff = (gj < G) ? (srow * (uint32_t)G + gj) * 2u : kOOB;
          hw[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
        }
        sraw = u32x4{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16),
                     hw[6] | (hw[7] << 16)};
      }
    }
    u32x2 zraw = u32x2{0u, 0u};
    if constexpr (ZP) zraw = load_zp8<SALIGNED>(zr, (uint32_t)(kq * 16 + n16), g0, G);
    // ---- codes of every tile (rows past the end read zero)
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
    // ---- half 1's activations into this wave's LDS region: load 4 cc + j
    // of lane l lands at byte 1024 (4 cc + j) + 16 l
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16_to_lds(xr, &lds[wave][(4 * cc + j) * 256], x_off(1, cc, j));
    __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the first wait

#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if constexpr (!EXACT) xop[cc][j] = x_slots(xop[cc][j]);
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

    f32x4 acc0[T], acc1[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc) {
      u32x4 u[T];
#pragma unroll
      for (int t = 0; t < T; ++t) u[t] = transpose_rows(wv[t][cc]);
      uint32_t zc[T];                    // ZP: tile t's zero points of this chunk's groups
      if constexpr (ZP) {
        uint32_t b[4];
        broadcast_rows(cc == 0 ? zraw.x : zraw.y, b);
#pragma unroll
        for (int t = 0; t < T; ++t) zc[t] = b[t];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 x1 = *(const u32x4*)&lds[wave][(4 * cc + j) * 256 + 4 * lane];
        if constexpr (EXACT) {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint32_t word = j == 0 ? u[t].x : j == 1 ? u[t].y : j == 2 ? u[t].z : u[t].w;
            const uint32_t sp = sct[t][2 * cc + (j >> 1)];
            const float sc = (j & 1) ? bf16_hi(sp) : bf16_lo(sp);
            DeqScale dq;
            if constexpr (ZP)
              dq = deq_scale_zp(sc, (float)((zc[t] >> (8 * j)) & 0xFFu));
            else
              dq = deq_scale(sc);
            const u32x4 w = dequant8<ZP>(word, dq);
            acc0[t] = mfma16(xop[cc][j], w, acc0[t]);
            acc1[t] = mfma16(x1, w, acc1[t]);
          }
          continue;
        }
        x1 = x_slots(x1);
        const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 cst0 = zero4, cst1 = zero4;
        if constexpr (!ZP) {
          cst0 = mfma16(xop[cc][j], neg136, zero4);
          cst1 = mfma16(x1, neg136, zero4);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t word = j == 0 ? u[t].x : j == 1 ? u[t].y : j == 2 ? u[t].z : u[t].w;
          const u32x4 cs = code_slots<ZP>(word);
          f32x4 ct0 = cst0, ct1 = cst1;
          if constexpr (ZP) {
            const uint32_t zz = j == 0   ? zp_offset_pair<0>(zc[t])
                                : j == 1 ? zp_offset_pair<1>(zc[t])
                                : j == 2 ? zp_offset_pair<2>(zc[t])
                                         : zp_offset_pair<3>(zc[t]);
            const u32x4 zop = u32x4{zz, zz, zz, zz};
            ct0 = mfma16(xop[cc][j], zop, zero4);
            ct1 = mfma16(x1, zop, zero4);
          }
          const f32x4 d0 = mfma16(xop[cc][j], cs, ct0);
          const f32x4 d1 = mfma16(x1, cs, ct1);
          const uint32_t sp = sct[t][2 * cc + (j >> 1)];
          const float sc = (j & 1) ? bf16_hi(sp) : bf16_lo(sp);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc0[t][r] = __builtin_fmaf(d0[r], sc, acc0[t][r]);
            acc1[t][r] = __builtin_fmaf(d1[r], sc, acc1[t][r]);
          }
        }
      }
    }
    // lane holds D[m = 16 hh + 4 kq + r][n = n16]; the region's activations
    // have all been read by this wave (LDS accesses in program order)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      *(f32x4*)&lds[wave][t * WSTR + n16 * PSTR + 4 * kq] = acc0[t];
      *(f32x4*)&lds[wave][t * WSTR + n16 * PSTR + 16 + 4 * kq] = acc1[t];
    }

    // ---- sum over waves in a fixed order (deterministic): one thread per
    // output, rows m < M only
    __syncthreads();
    const int mrows = min(M, 32);
    const int nout = ntiles * mrows * 16;
    for (int o = tid; o < nout; o += kWaves * 64) {
      const int t = o / (mrows * 16);
      const int m = (o >> 4) % mrows;
      const int n = o & 15;
      const int e = t * WSTR + n * PSTR + m;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += lds[w][e];
      const int row = t * 16 + n;
      if (npass > 1) {
        sum += (pass == 0) ? 0.0f : ybuf[t][m * 16 + n];
        ybuf[t][m * 16 + n] = sum;
      }
      if (pass == npass - 1 && row < rows) Y[(size_t)m * N + n0 + row] = to_bf16(sum);
    }
    __syncthreads();   // the regions are rewritten by the next pass (and the DMA)
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

template <bool SA, int T, int RM, bool ZP, bool EX>
hipError_t run_decode16_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  const int64_t blocks = (N + T * 16 - 1) / (T * 16);
  hipLaunchKernelGGL((k_decode16<SA, T, RM, ZP, EX>), dim3((unsigned)blocks), dim3(kWaves * 64), 0,
                     st, X, (const uint32_t*)Wq, S, Z, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <bool SA, int RM, bool ZP, bool EX>
hipError_t run_decode16(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                        uint16_t* Y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = cu_count();
  const int64_t tpw = (tiles + cus - 1) / cus;
  if (tpw <= 1) return run_decode16_t<SA, 1, RM, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  if (tpw == 2) return run_decode16_t<SA, 2, RM, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  if (tpw == 3) return run_decode16_t<SA, 3, RM, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  return run_decode16_t<SA, 4, RM, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
}

template <bool SA, int T, bool ZP, bool EX>
hipError_t run_decode32_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  const int64_t blocks = (N + T * 16 - 1) / (T * 16);
  hipLaunchKernelGGL((k_decode32<SA, T, ZP, EX>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, st,
                     X, (const uint32_t*)Wq, S, Z, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <bool SA, bool ZP, bool EX>
hipError_t run_decode32(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                        uint16_t* Y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = cu_count();
  const int64_t tpw = (tiles + cus - 1) / cus;
  if (tpw <= 1) return run_decode32_t<SA, 1, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  if (tpw == 2) return run_decode32_t<SA, 2, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  return run_decode32_t<SA, 3, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
}

template <bool ZP, bool EX>
hipError_t launch_decode_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                           hipStream_t st) {
  const bool sa = ((K >> 5) & 7) == 0;
  if (M == 1)
    return sa ? run_decode16<true, 1, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st)
              : run_decode16<false, 1, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  if (M <= 16)
    return sa ? run_decode16<true, 4, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st)
              : run_decode16<false, 4, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
  return sa ? run_decode32<true, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st)
            : run_decode32<false, ZP, EX>(X, Wq, S, Z, Y, M, N, K, st);
}

// Above this K the decode kernels dequantize each code to bf16(q s) (the
// definition's weights) instead of scaling exact integer-code sums.
constexpr int64_t kExactK = 16384;

template <bool ZP>
hipError_t launch_decode(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                         const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                         hipStream_t st) {
  if (K > kExactK) return launch_decode_t<ZP, true>(X, Wq, S, Z, Y, M, N, K, st);
  return launch_decode_t<ZP, false>(X, Wq, S, Z, Y, M, N, K, st);
}

}  // namespace

hipError_t launch_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  return launch_decode<false>(X, Wq, S, nullptr, Y, M, N, K, st);
}

hipError_t launch_gemv_zp(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  return launch_decode<true>(X, Wq, S, Z, Y, M, N, K, st);
}

}  // namespace w4
