// W4A16 product for small M (decode): Y[M, N] = X[M, K] * dequant(W)^T.
//
// Method: "INT4 QAT end-to-end for RL" §4 (INT4 weights are dequantized in
// registers to BF16 and multiplied against BF16 activations on BF16 matrix
// units); "Quantization basics: from FP32 to INT4" §2.1 (w = q * s, z = 0)
// and the tutorial's opening remark that decode reads every weight once per
// token, so this path is bound by HBM bandwidth.
//
// Arithmetic.  Every code becomes the definition's weight w' = bf16(q s)
// (or bf16((q - z) s) for zero-point codes) with the 17-op fma_mix step of
// dequant8, and the MFMA accumulates x * w' in fp32 across all groups.  No
// step rounds anything the definition does not: the MFMA's products of two
// bf16 are exact, only the order of the fp32 additions is the kernel's.
//
// Mapping (MI355X).  One workgroup of 16 waves per CU; wave w owns a
// 256-element K slice (two 128-element "chunks" of four groups) and keeps
// its slice of X in registers (loaded once, reused for every weight row).
// The workgroup covers T tiles of 16 weight rows.  For one chunk c, lane
// (n = l % 16, kq = l / 16) loads the 16 bytes of group 4 c + kq of row n
// (a 16-row tile is 16 contiguous 64-byte runs) with a raw buffer load;
// rows or groups past the end read as zero in hardware, so no load sits
// behind a branch.  Word j of those 16 bytes is the lane's B operand of
// MFMA j (v_mfma_f32_16x16x32_bf16: A = X rows, B = weight rows), whose 32
// k values are elements 8 j .. 8 j + 7 of the four groups of the chunk, so
// a lane dequantizes all four words of one group with one scale.  Lane
// (m, kq)'s A operand of MFMA j is elements 8 j .. 8 j + 7 of group
// 4 c + kq of row m: for M <= 8 each lane loads those 16 bytes itself; for
// more rows the activations come in whole lines through LDS (below) or, with
// four tiles, as contiguous 64-byte runs per row (lane (m, kq): elements
// 8 kq .. 8 kq + 7 of group 4 c + j, one load per j) followed by a 4 x 4
// transpose of 16-byte pieces across the four 16-lane rows
// (v_permlane32_swap + v_permlane16_swap), done once per wave.  A wave's
// eight scales of a row are one 16-byte load: lane row r fetches tile r's,
// permlane swaps broadcast them, and each lane picks its group's.
//   Each wave issues all of its loads at once (scales and activations first,
// then the codes tile by tile) and processes tile t as soon as its codes
// are in, while the later tiles' are still on the way.  Per-wave partials
// meet in LDS (fixed wave order, deterministic) once per K pass; each
// output is owned by one thread.
//
// Kernel-order codes (TL, written by w4_repack): the 16 bytes of group g of
// row n sit in the 1 KB block (n / 32, g / 2) at unit 32 (g % 2) + n % 32,
// so one load instruction reads four 256-byte runs instead of 16 rows'
// 64-byte pieces.  Its scales and zero points then come in kernel order
// too (w4_repack_groups): a tile's 8 values of a wave's slice are one
// 256-byte piece (128 for zero points); the arithmetic is unchanged.
//
// Zero-point weights (ZP; "Quantization basics: from FP32 to INT4" §2.1 and
// §2.3, w' = bf16((q - z) s) with unsigned q): the same step with the
// unsigned form of dequant8; a lane row loads its row's eight zero points
// beside the scales and they are broadcast like the scales.
#include "common.h"

namespace w4 {

namespace {

constexpr int kWaves = 16;
constexpr int kCPW = 2;                 // 128-element chunks per wave per pass
constexpr int kPassK = kWaves * kCPW * 128;
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past any buffer: reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 4 x 4 transpose across the four 16-lane rows: on entry lane row r holds
// dwords 0..3 of item r; on exit it holds dword r of items 0..3.
__device__ __forceinline__ u32x4 transpose_rows(u32x4 v) {
  auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return u32x4{c[0], c[1], d[0], d[1]};
}

// On entry lane (m, kq) holds in x[j] elements 8 kq .. 8 kq + 7 of group
// 4 c + j of its row; on exit x[j] holds elements 8 j .. 8 j + 7 of group
// 4 c + kq (the same transpose for each of the four dwords of a piece).
__device__ __forceinline__ void transpose_pieces(u32x4 (&x)[4]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x4 v = transpose_rows(u32x4{x[0][d], x[1][d], x[2][d], x[3][d]});
    x[0][d] = v.x;
    x[1][d] = v.y;
    x[2][d] = v.z;
    x[3][d] = v.w;
  }
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load ... lds):
// lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           off, 0, 0, 0);
}

// 16 rows x 256 activations (rows row0 .. row0 + 15 of X, the wave's K
// slice from chunk c0) into an LDS region of 16 rows x 512 bytes, whole
// 128-byte lines: load i brings rows 2 i, 2 i + 1; lane l's 16 bytes land in
// slot l % 32 of row r = 2 i + l / 32 and hold the slice's piece
// (l % 32) ^ r, so that 16 lanes reading one piece of 16 rows hit 16
// different slots (no bank conflicts).  Rows past M lie past X's buffer and
// groups past K are sent past it: both read zero.
template <bool FULL>
__device__ __forceinline__ void load_x_lines(__amdgpu_buffer_rsrc_t xr, float* region, int row0,
                                             int c0, int lane, int K, int G) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 2 * i + (lane >> 5);
    const int gp = (lane & 31) ^ r;
    const int g = 4 * c0 + (gp >> 2);
    const uint32_t off =
        (FULL || g < G)
            ? ((uint32_t)(row0 + r) * (uint32_t)K + 128u * (uint32_t)c0 + 8u * (uint32_t)gp) * 2u
            : kOOB;
    dma16_to_lds(xr, region + 256 * i, off);
  }
}

// float index of piece 16 cc + 4 kq + j of row r (< 16) in a region written
// by load_x_lines: the XOR with r leaves bit 4 alone, so chunk cc is a
// constant offset from the index of chunk 0
__device__ __forceinline__ int x_slot(int r, int kq, int j, int cc) {
  return 128 * r + 4 * ((4 * kq + j) ^ r) + 64 * cc;
}

// Code buffer of a workgroup's rows [n0, n0 + rows) and the byte offset of
// the 16 bytes of group g of its row nl (kOOB past K).  Canonical: rows of
// K / 2 bytes from row n0.  Kernel order: the 1 KB blocks of the 32-row
// blocks that hold those rows, ceil(K / 64) blocks per 32 rows.
template <bool TL>
struct CodeRows {
  __amdgpu_buffer_rsrc_t r;
  uint32_t rowb, nsteps, first;
  __device__ CodeRows(const uint32_t* Wq, int n0, int rows, int K) {
    rowb = (uint32_t)K >> 1;
    nsteps = (uint32_t)(K + 63) >> 6;
    if constexpr (TL) {
      first = (uint32_t)n0 & 31u;              // row n0's place in its 32-row block
      const uint32_t b0 = (uint32_t)n0 >> 5, b1 = ((uint32_t)(n0 + rows) + 31u) >> 5;
      r = rsrc(Wq + (size_t)b0 * nsteps * 256u, (b1 - b0) * nsteps * 1024u);
    } else {
      first = 0;
      r = rsrc(Wq + (size_t)n0 * (K >> 3), (uint32_t)rows * rowb);
    }
  }
  // FULL: every group index the caller passes is below G
  template <bool FULL>
  __device__ __forceinline__ uint32_t off(uint32_t nl, int g, int G) const {
    if (!FULL && g >= G) return kOOB;
    if constexpr (TL) {
      const uint32_t n = first + nl;
      return (((n >> 5) * nsteps + ((uint32_t)g >> 1)) * 64u + ((uint32_t)g & 1u) * 32u +
              (n & 31u)) * 16u;
    } else {
      return nl * rowb + 16u * (uint32_t)g;
    }
  }
};

__device__ __forceinline__ uint32_t word_of(u32x4 v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// This lane row's 8 scales of weight row srow, groups g0 .. g0 + 7 (four
// dwords, bf16 pairs); SALIGNED (K / 32 a multiple of 8): one 16-byte load,
// a block past K clamped into the row (where codes and activations read
// zero); otherwise eight 2-byte loads, groups past K reading zero.
template <bool SALIGNED>
__device__ __forceinline__ u32x4 load_scale8(__amdgpu_buffer_rsrc_t sr, uint32_t srow, int g0,
                                             int G) {
  if constexpr (SALIGNED) {
    const uint32_t gb = (uint32_t)min(g0, G - 8);
    return __builtin_amdgcn_raw_buffer_load_b128(sr, (srow * (uint32_t)G + gb) * 2u, 0, 0);
  } else {
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int gj = g0 + j;
      const uint32_t soff = (gj < G) ? (srow * (uint32_t)G + gj) * 2u : kOOB;
      h[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
    }
    return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                 h[6] | (h[7] << 16)};
  }
}

// The same for the row's 8 zero points (two dwords).
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

// Per-group values (scales, zero points) of a workgroup's rows [n0, n0 +
// rows), n0 a multiple of 16: the first element and the element count.
// Canonical: rows of G values.  Kernel order (w4_repack_groups): the
// ceil(G / 8) blocks of 128 values of each of the workgroup's 16-row
// blocks; value 8 i + j of block (r, c) is row 16 r + i, group 8 c + j.
template <bool TL>
__device__ __forceinline__ void group_span(int n0, int rows, int G, size_t& first,
                                           uint32_t& count) {
  if constexpr (TL) {
    const uint32_t gblk = (uint32_t)(G + 7) >> 3;
    first = (size_t)(n0 >> 4) * gblk * 128u;
    count = (((uint32_t)rows + 15u) >> 4) * gblk * 128u;
  } else {
    first = (size_t)n0 * G;
    count = (uint32_t)rows * (uint32_t)G;
  }
}

// Copies of v with all four 16-lane rows replaced by row 0, 1, 2, 3.
__device__ __forceinline__ void broadcast_rows(uint32_t v, uint32_t out[4]) {
  auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // [r0 r1 r0 r1], [r2 r3 r2 r3]
  auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
  auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// The wave's scales (and zero points) of one pass.  Lane row r loads the 8
// groups of the wave's slice of row n16 of tile r (one 16-byte load; 8
// bytes of zero points) and permlane swaps broadcast them, so every lane
// holds its row's 8 scales of every tile; lane (n16, kq) then takes group
// 4 cc + kq of chunk cc (a dword select and a byte permute).
template <int KM, int T, bool ZP, bool TL>
struct PassScales {
  static constexpr bool SALIGNED = KM >= 1, FULL = KM == 2;
  uint32_t sct[T][4];      // [tile][dword]: 8 bf16 scales
  uint32_t zc[kCPW][T];    // [chunk][tile]: the 4 zero points of the chunk's groups
  u32x4 sraw;
  u32x2 zraw;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t sr, __amdgpu_buffer_rsrc_t zr,
                                       int n16, int kq, int g0, int G) {
    zraw = u32x2{0u, 0u};
    if constexpr (TL) {
      // one piece of block (tile kq, g0 / 8); g0 is a multiple of 8 and the
      // blocks are zero-padded, so no clamp (tiles past the rows read zero)
      const uint32_t e =
          ((uint32_t)kq * ((uint32_t)(G + 7) >> 3) + ((uint32_t)g0 >> 3)) * 128u + 8u * n16;
      const bool in = FULL || g0 < G;
      sraw = __builtin_amdgcn_raw_buffer_load_b128(sr, in ? e * 2u : kOOB, 0, 0);
      if constexpr (ZP) zraw = __builtin_amdgcn_raw_buffer_load_b64(zr, in ? e : kOOB, 0, 0);
    } else {
      sraw = load_scale8<SALIGNED>(sr, (uint32_t)(kq * 16 + n16), g0, G);
      if constexpr (ZP) zraw = load_zp8<SALIGNED>(zr, (uint32_t)(kq * 16 + n16), g0, G);
    }
  }
  __device__ __forceinline__ void spread() {
    const uint32_t rw[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t b[4];
      broadcast_rows(rw[d], b);
#pragma unroll
      for (int t = 0; t < T; ++t) sct[t][d] = b[t];
    }
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc) {
      if constexpr (ZP) {
        uint32_t b[4];
        broadcast_rows(cc == 0 ? zraw.x : zraw.y, b);
#pragma unroll
        for (int t = 0; t < T; ++t) zc[cc][t] = b[t];
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t) zc[cc][t] = 0u;
      }
    }
  }
  // dequant8 constants of group 4 cc + kq of tile t: its bf16 is bytes
  // 2 kq, 2 kq + 1 of dwords 2 cc, 2 cc + 1 taken as one 8-byte value; one
  // byte permute (sel) moves them to the high half over zero bits (an fp32)
  __device__ __forceinline__ DeqScale consts(int t, int cc, uint32_t sel, int kq) const {
    const uint32_t b = __builtin_amdgcn_perm(sct[t][2 * cc + 1], sct[t][2 * cc], sel);
    const float s = __uint_as_float(b);
    if constexpr (ZP)
      return deq_scale_zp(s, (float)((zc[cc][t] >> (8 * kq)) & 0xFFu));
    else
      return deq_scale(s);
  }
};

// The codes of one pass: lane (n16, kq) loads words 0..3 of group
// 4 (c0 + cc) + kq of row t * 16 + n16, tile by tile (rows past the
// workgroup's and groups past K read zero).
template <bool FULL, int T, bool TL>
__device__ __forceinline__ void load_codes(u32x4 (&wv)[T][kCPW], const CodeRows<TL>& wr, int c0,
                                           int n16, int kq, int G) {
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int cc = 0; cc < kCPW; ++cc)
      wv[t][cc] = __builtin_amdgcn_raw_buffer_load_b128(
          wr.r, wr.template off<FULL>((uint32_t)(t * 16 + n16), 4 * (c0 + cc) + kq, G), 0, 0);
}

// The same for tile t alone.
template <bool FULL, int T, bool TL>
__device__ __forceinline__ void load_codes_tile(u32x4 (&wv)[T][kCPW], int t, const CodeRows<TL>& wr,
                                                int c0, int n16, int kq, int G) {
#pragma unroll
  for (int cc = 0; cc < kCPW; ++cc)
    wv[t][cc] = __builtin_amdgcn_raw_buffer_load_b128(
        wr.r, wr.template off<FULL>((uint32_t)(t * 16 + n16), 4 * (c0 + cc) + kq, G), 0, 0);
}

}  // namespace

// M <= 16.  KM: 0 = any K; 1 = K / 32 is a multiple of 8 (a wave's eight
// scales of one row are one 16-byte load); 2 = K is a multiple of the
// 4096-element pass as well (no group index is ever past K, so no offset
// needs a range check).  Activation rows past M need none either: they lie
// past the end of X's buffer and read zero.  T: tiles of 16 weight rows per
// workgroup.  XM, how the activations arrive:
//   kXLines (8 < M <= 16, T <= 3): through the wave's LDS region in whole
//     128-byte lines (two rows per load, half the cache-line requests of the
//     64-byte runs); each lane reads its operands in MFMA order.
//   kXOperand (M <= 8): each lane loads its own operands into registers in
//     MFMA order (16 bytes per MFMA, spread over two lines per row): with at
//     most 8 rows in the buffer the requests stay few, and neither the LDS
//     round trip nor a transpose is needed.
//   kXRuns (8 < M <= 16, T = 4, where the LDS path has no registers left):
//     64-byte runs per row into registers, then the transpose to operand
//     order (one cache line per row and load).
enum XMode { kXRuns = 0, kXLines = 1, kXOperand = 2 };
template <int KM, int T, bool ZP, bool TL, int XM>
__global__ __launch_bounds__(kWaves * 64) void k_decode16(const uint16_t* __restrict__ X,
                                                          const uint32_t* __restrict__ Wq,
                                                          const uint16_t* __restrict__ S,
                                                          const uint8_t* __restrict__ Z,
                                                          uint16_t* __restrict__ Y, int M, int N,
                                                          int K) {
  static_assert(T >= 1 && T <= 4, "decode shape");
  constexpr bool FULL = KM == 2;
  constexpr int PSTR = 20;                         // LDS row stride (floats)
  constexpr int WSTR = 16 * PSTR + 4;              // per-tile block: padded off the bank period
  constexpr int XREG = XM == kXLines ? 2048 : 0;   // floats: the wave's 16 x 256 activations
  constexpr int REGION = T * WSTR > XREG ? T * WSTR : XREG;
  __shared__ __attribute__((aligned(16))) float lds[kWaves][REGION];
  __shared__ float ybuf[T][256];                   // partials across K passes

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;
  const int kq = lane >> 4;
  const int G = K >> 5;
  const int n0 = blockIdx.x * (T * 16);
  const int rows = min(T * 16, N - n0);
  const int ntiles = (rows + 15) >> 4;

  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const CodeRows<TL> wr(Wq, n0, rows, K);
  size_t gfirst;
  uint32_t gcount;
  group_span<TL>(n0, rows, G, gfirst, gcount);
  const __amdgpu_buffer_rsrc_t sr = rsrc(S + gfirst, gcount * 2u);
  const __amdgpu_buffer_rsrc_t zr = rsrc(ZP ? Z + gfirst : nullptr, ZP ? gcount : 0u);
  const int npass = (K + kPassK - 1) / kPassK;
  // byte permute selector: bytes 2 kq + 1, 2 kq of the 8-byte value (low
  // dword = bytes 0..3) to the high half, zero bytes (0x0C) below
  const uint32_t sel = ((2u * kq + 1u) << 24) | ((2u * kq) << 16) | 0x0C0Cu;

  for (int pass = 0; pass < npass; ++pass) {
    const int c0 = pass * (kWaves * kCPW) + wave * kCPW;   // first chunk of this wave
    // ---- scales (and zero points) first
    PassScales<KM, T, ZP, TL> sc;
    sc.load(sr, zr, n16, kq, 4 * c0, G);
    // ---- activations (L2 hits after the first CU's request)
    u32x4 xop[kCPW][4];
    if constexpr (XM == kXLines) {
      // into this wave's LDS region: load i brings rows 2 i, 2 i + 1 of the
      // wave's 16 x 256 slice; lane l's 16 bytes land in slot l % 32 of row
      // 2 i + l / 32 and hold piece (l % 32) ^ row of it
      load_x_lines<FULL>(xr, &lds[wave][0], 0, c0, lane, K, G);
    } else {
      // kXRuns: lane (m, kq) takes elements 8 kq .. 8 kq + 7 of group
      // 4 c + j of row m; kXOperand: elements 8 j .. 8 j + 7 of group
      // 4 c + kq, its operand of MFMA j
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g = 4 * (c0 + cc) + (XM == kXOperand ? kq : j);
          const uint32_t e = XM == kXOperand ? 8u * j : 8u * kq;
          const uint32_t off =
              (FULL || g < G) ? ((uint32_t)n16 * (uint32_t)K + 32u * g + e) * 2u : kOOB;
          xop[cc][j] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // the codes are issued after every activation load
    // ---- codes, tile by tile; a row's two chunks are adjacent requests (one
    // 128-byte line).  Loads return in issue order, so tile t is processed as
    // soon as its codes are in while the later tiles' are still on the way.
    u32x4 wv[T][kCPW];
    load_codes<FULL, T, TL>(wv, wr, c0, n16, kq, G);
    __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the first wait

    if constexpr (XM == kXLines) {
      // the activations have landed once only the codes are in flight; lane
      // (m, kq)'s operand of MFMA j of chunk cc (elements 8 j .. 8 j + 7 of
      // group 4 c + kq of row m) is piece 16 cc + 4 kq + j of row m
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T * kCPW) : "memory");
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xop[cc][j] = *(const u32x4*)&lds[wave][x_slot(n16, kq, j, cc)];
    }
    sc.spread();
    if constexpr (XM == kXRuns) {
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) transpose_pieces(xop[cc]);
    }

#pragma unroll
    for (int t = 0; t < T; ++t) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) {
        const DeqScale dq = sc.consts(t, cc, sel, kq);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = mfma16(xop[cc][j], dequant8<ZP>(word_of(wv[t][cc], j), dq), acc);
      }
      // lane holds D[m = 4 kq + r][n = n16] of tile t; the wave has read all
      // of its activations (LDS accesses in program order)
      *(f32x4*)&lds[wave][t * WSTR + n16 * PSTR + 4 * kq] = acc;
      __builtin_amdgcn_sched_barrier(0);   // tile t's work stays ahead of tile t + 1's wait
    }

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
      for (int w = 0; w < kWaves; ++w) sum += lds[w][t * WSTR + e];
      const int row = t * 16 + n;
      if (npass > 1) {
        sum += (pass == 0) ? 0.0f : ybuf[t][m * 16 + n];
        ybuf[t][m * 16 + n] = sum;
      }
      if (pass == npass - 1 && row < rows) Y[(size_t)m * N + n0 + row] = to_bf16(sum);
    }
    if (npass > 1) __syncthreads();   // the regions are rewritten by the next pass
  }
}

// 16 < M <= 32 over two 16-row activation halves.  K a whole number of
// passes: both halves come through this wave's LDS region in whole lines,
// one after the other (half 0 is read into registers in operand order once
// it has landed, and half 1 takes its place); otherwise half 0 comes into
// registers as 64-byte runs per row and is transposed.  Each lane reads its
// half-1 operand of MFMA j where it landed.  Each dequantized word feeds the
// MFMAs of both halves.  The region then takes the wave's partial sums.
template <int KM, int T, bool ZP, bool TL>
__global__ __launch_bounds__(kWaves * 64) void k_decode32(const uint16_t* __restrict__ X,
                                                          const uint32_t* __restrict__ Wq,
                                                          const uint16_t* __restrict__ S,
                                                          const uint8_t* __restrict__ Z,
                                                          uint16_t* __restrict__ Y, int M, int N,
                                                          int K) {
  static_assert(T >= 1 && T <= 3, "decode shape");
  constexpr bool FULL = KM == 2;
  // tiles whose codes go out before half 1 (two measured slightly faster
  // than one at M = 32)
  constexpr int kEarly = T < 2 ? 1 : 2;
  static_assert(kEarly <= 2, "early code tiles");
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
  const int n0 = blockIdx.x * (T * 16);
  const int rows = min(T * 16, N - n0);
  const int ntiles = (rows + 15) >> 4;

  const __amdgpu_buffer_rsrc_t xr = rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const CodeRows<TL> wr(Wq, n0, rows, K);
  size_t gfirst;
  uint32_t gcount;
  group_span<TL>(n0, rows, G, gfirst, gcount);
  const __amdgpu_buffer_rsrc_t sr = rsrc(S + gfirst, gcount * 2u);
  const __amdgpu_buffer_rsrc_t zr = rsrc(ZP ? Z + gfirst : nullptr, ZP ? gcount : 0u);
  const int npass = (K + kPassK - 1) / kPassK;
  // byte permute selector: bytes 2 kq + 1, 2 kq of the 8-byte value (low
  // dword = bytes 0..3) to the high half, zero bytes (0x0C) below
  const uint32_t sel = ((2u * kq + 1u) << 24) | ((2u * kq) << 16) | 0x0C0Cu;

  for (int pass = 0; pass < npass; ++pass) {
    const int c0 = pass * (kWaves * kCPW) + wave * kCPW;   // first chunk of this wave
    // ---- scales (and zero points) first
    PassScales<KM, T, ZP, TL> sc;
    sc.load(sr, zr, n16, kq, 4 * c0, G);
    u32x4 xop[kCPW][4];
    u32x4 wv[T][kCPW];
    if constexpr (FULL) {
      // ---- both halves' activations go through this wave's LDS region in
      // whole lines, one after the other: half 0, then tile 0's codes; once
      // half 0 has landed it is read into registers in operand order and
      // half 1 takes its place, followed by the other tiles' codes.  Loads
      // return in issue order, so tile t is processed as soon as its codes
      // are in.
      __builtin_amdgcn_sched_barrier(0);   // the waits below count loads in issue order
      load_x_lines<FULL>(xr, &lds[wave][0], 0, c0, lane, K, G);
      __builtin_amdgcn_sched_barrier(0);
      load_codes_tile<FULL, T, TL>(wv, 0, wr, c0, n16, kq, G);
      if constexpr (kEarly > 1) load_codes_tile<FULL, T, TL>(wv, 1, wr, c0, n16, kq, G);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kEarly * kCPW) : "memory");   // half 0 has landed
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xop[cc][j] = *(const u32x4*)&lds[wave][x_slot(n16, kq, j, cc)];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the region is refilled
      __builtin_amdgcn_sched_barrier(0);
      load_x_lines<FULL>(xr, &lds[wave][0], 16, c0, lane, K, G);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = kEarly; t < T; ++t) load_codes_tile<FULL, T, TL>(wv, t, wr, c0, n16, kq, G);
      __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the next wait
      sc.spread();
      // half 1 has landed once only the later tiles' codes are in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((T - kEarly) * kCPW) : "memory");
    } else {
      // ---- K not a whole number of passes (range checks on every load;
      // the staging above would spill): half 0's activations into
      // registers, 64-byte runs per row, transposed to operand order; half
      // 1's into this wave's LDS region in whole lines
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g = 4 * (c0 + cc) + j;
          const uint32_t off =
              (g < G) ? ((uint32_t)n16 * (uint32_t)K + 32u * g + 8u * kq) * 2u : kOOB;
          xop[cc][j] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
      load_x_lines<FULL>(xr, &lds[wave][0], 16, c0, lane, K, G);
      load_codes<FULL, T, TL>(wv, wr, c0, n16, kq, G);
      __builtin_amdgcn_sched_barrier(0);   // keep every load above ahead of the first wait
      sc.spread();
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) transpose_pieces(xop[cc]);
      // half 1 has landed once only the codes are in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(T * kCPW) : "memory");
    }

    f32x4 acc0[T], acc1[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < kCPW; ++cc) {
        const DeqScale dq = sc.consts(t, cc, sel, kq);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // elements 8 j .. 8 j + 7 of group 4 c + kq of half-1 row n16
          const u32x4 x1 = *(const u32x4*)&lds[wave][x_slot(n16, kq, j, cc)];
          const u32x4 w = dequant8<ZP>(word_of(wv[t][cc], j), dq);
          acc0[t] = mfma16(xop[cc][j], w, acc0[t]);
          acc1[t] = mfma16(x1, w, acc1[t]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // tile t's work stays ahead of tile t + 1's wait
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

template <int KM, int T, bool ZP, bool TL, int XM>
hipError_t run_decode16_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  const int64_t blocks = (N + T * 16 - 1) / (T * 16);
  hipLaunchKernelGGL((k_decode16<KM, T, ZP, TL, XM>), dim3((unsigned)blocks), dim3(kWaves * 64), 0,
                     st, X, (const uint32_t*)Wq, S, Z, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <int KM, bool ZP, bool TL>
hipError_t run_decode16(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                        uint16_t* Y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = cu_count();
  const int64_t tpw = (tiles + cus - 1) / cus;
  if (M > 8) {
    // (four tiles leave no registers for the LDS path)
    if (tpw <= 1) return run_decode16_t<KM, 1, ZP, TL, kXLines>(X, Wq, S, Z, Y, M, N, K, st);
    if (tpw == 2) return run_decode16_t<KM, 2, ZP, TL, kXLines>(X, Wq, S, Z, Y, M, N, K, st);
    if (tpw == 3) return run_decode16_t<KM, 3, ZP, TL, kXLines>(X, Wq, S, Z, Y, M, N, K, st);
    return run_decode16_t<KM, 4, ZP, TL, kXRuns>(X, Wq, S, Z, Y, M, N, K, st);
  }
  if (tpw <= 1) return run_decode16_t<KM, 1, ZP, TL, kXOperand>(X, Wq, S, Z, Y, M, N, K, st);
  if (tpw == 2) return run_decode16_t<KM, 2, ZP, TL, kXOperand>(X, Wq, S, Z, Y, M, N, K, st);
  if (tpw == 3) return run_decode16_t<KM, 3, ZP, TL, kXOperand>(X, Wq, S, Z, Y, M, N, K, st);
  return run_decode16_t<KM, 4, ZP, TL, kXOperand>(X, Wq, S, Z, Y, M, N, K, st);
}

template <int KM, int T, bool ZP, bool TL>
hipError_t run_decode32_t(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  const int64_t blocks = (N + T * 16 - 1) / (T * 16);
  hipLaunchKernelGGL((k_decode32<KM, T, ZP, TL>), dim3((unsigned)blocks), dim3(kWaves * 64), 0,
                     st, X, (const uint32_t*)Wq, S, Z, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <int KM, bool ZP, bool TL>
hipError_t run_decode32(const uint16_t* X, const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                        uint16_t* Y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = cu_count();
  const int64_t tpw = (tiles + cus - 1) / cus;
  if (tpw <= 1) return run_decode32_t<KM, 1, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
  if (tpw == 2) return run_decode32_t<KM, 2, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
  return run_decode32_t<KM, 3, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
}

template <bool ZP, bool TL>
hipError_t launch_decode(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                         const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                         hipStream_t st) {
  const int km = K % kPassK == 0 ? 2 : ((K >> 5) & 7) == 0 ? 1 : 0;
  if (M <= 16) {
    if (km == 2) return run_decode16<2, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
    if (km == 1) return run_decode16<1, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
    return run_decode16<0, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
  }
  if (km == 2) return run_decode32<2, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
  if (km == 1) return run_decode32<1, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
  return run_decode32<0, ZP, TL>(X, Wq, S, Z, Y, M, N, K, st);
}

}  // namespace

// Z == nullptr: symmetric codes; tiled: codes in the kernel-order layout
hipError_t launch_gemv_any(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                           const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                           bool tiled, hipStream_t st) {
  if (Z != nullptr)
    return tiled ? launch_decode<true, true>(X, Wq, S, Z, Y, M, N, K, st)
                 : launch_decode<true, false>(X, Wq, S, Z, Y, M, N, K, st);
  return tiled ? launch_decode<false, true>(X, Wq, S, nullptr, Y, M, N, K, st)
               : launch_decode<false, false>(X, Wq, S, nullptr, Y, M, N, K, st);
}

hipError_t launch_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  return launch_gemv_any(X, Wq, S, nullptr, Y, M, N, K, false, st);
}

hipError_t launch_gemv_zp(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                          hipStream_t st) {
  return launch_gemv_any(X, Wq, S, Z, Y, M, N, K, false, st);
}

}  // namespace w4
