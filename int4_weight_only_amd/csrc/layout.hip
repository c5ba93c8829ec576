// Kernel-order code layout: conversion from the canonical packed layout and
// back (the MI355X counterpart of the weight-layout conversion that the
// "INT4 QAT end-to-end for RL" write-up, section 4, applies after loading
// INT4 weights for its inference kernel, and of the restore step that
// undoes it before new weights are loaded).
//
// Canonical: Wq [N, K/8] int32, row-major; the 16 bytes of group g (32
// codes, one scale) of row n start at byte n K/2 + 16 g.
// Kernel order, per matrix: ceil(N/32) x ceil(K/64) blocks of 1 KB, block
// (r, c) at byte 1024 (r ceil(K/64) + c); unit u (16 bytes) of a block
// holds group 2 c + u / 32 of row 32 r + u % 32.  Units naming a row past
// N or a group past K/32 are zero.  E matrices (experts) are stored one
// after the other, each with its own blocks.
//
// One lane per 16-byte unit of the kernel-order buffer: a 64-lane wave
// writes one whole block (1 KB, coalesced) and reads 32 rows x 32 bytes.
//
// Per-group values (bf16 scales, uint8 zero points; canonical [N, K/32]):
// per matrix, ceil(N/16) x ceil(G/8) blocks of 128 elements (G = K/32),
// block (r, c) at element 128 (r ceil(G/8) + c), and element 8 i + j of a
// block is row 16 r + i, group 8 c + j.  Elements naming a row past N or a
// group past G are zero.  The products read a wave's eight values of 16
// consecutive rows as one contiguous piece instead of 16 pieces one row
// apart.  One thread per 8-element row piece of a block (16 or 8 bytes).
#include "common.h"

namespace w4 {

template <bool RESTORE>
__global__ __launch_bounds__(256) void k_relayout(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, int64_t N,
                                                  int64_t G, int64_t nsteps, int64_t units,
                                                  int64_t total) {
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t e = i / units;            // matrix
    const int64_t u = i - e * units;        // unit inside the matrix's kernel-order blocks
    const int64_t blk = u >> 6;
    const int64_t r = blk / nsteps, c = blk - r * nsteps;
    const int64_t n = 32 * r + (u & 31);
    const int64_t g = 2 * c + ((u >> 5) & 1);
    const bool valid = n < N && g < G;
    const int64_t canon = (e * N + n) * G + g;   // 16-byte units of the canonical layout
    if constexpr (RESTORE) {
      if (valid) dst[canon] = src[i];
    } else {
      dst[i] = valid ? src[canon] : zero;
    }
  }
}

int64_t tiled_words(int64_t N, int64_t K) { return ((N + 31) / 32) * ((K + 63) / 64) * 256; }

int64_t tiled_group_elems(int64_t N, int64_t K) {
  return ((N + 15) / 16) * ((K / 32 + 7) / 8) * 128;
}

template <bool RESTORE, typename V>
__global__ __launch_bounds__(256) void k_relayout_groups(const V* __restrict__ src,
                                                         V* __restrict__ dst, int64_t N,
                                                         int64_t G, int64_t gb, int64_t pieces,
                                                         int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t e = i / pieces;           // matrix
    const int64_t p = i - e * pieces;       // row piece inside the matrix's blocks
    const int64_t blk = p >> 4;
    const int64_t r = blk / gb, c = blk - r * gb;
    const int64_t n = 16 * r + (p & 15);
    const V* s = src;
    V* d = dst;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t g = 8 * c + j;
      const bool valid = n < N && g < G;
      const int64_t canon = (e * N + n) * G + g;
      const int64_t tiled = 8 * i + j;
      if constexpr (RESTORE) {
        if (valid) d[canon] = s[tiled];
      } else {
        d[tiled] = valid ? s[canon] : (V)0;
      }
    }
  }
}

// K/32 a multiple of 8 and both buffers aligned to a whole piece: a piece
// (8 values of one row) is contiguous on both sides, one vector load and
// one vector store (P: 16 bytes of bf16 or 8 bytes of uint8)
template <bool RESTORE, typename P, typename I>
__global__ __launch_bounds__(256) void k_relayout_groups_vec(const P* __restrict__ src,
                                                             P* __restrict__ dst, I N, I gb,
                                                             I pieces, I total) {
  // I: 32-bit index arithmetic whenever every index fits (the divisions
  // dominate otherwise)
  for (I i = (I)blockIdx.x * 256 + threadIdx.x; i < total; i += (I)gridDim.x * 256) {
    const I e = i / pieces;
    const I p = i - e * pieces;
    const I blk = p >> 4;
    const I r = blk / gb, c = blk - r * gb;
    const I n = 16 * r + (p & 15);
    const I canon = (e * N + n) * gb + c;   // in pieces: rows of gb pieces
    if constexpr (RESTORE) {
      if (n < N) dst[canon] = src[i];
    } else {
      P v{};
      if (n < N) v = src[canon];
      dst[i] = v;
    }
  }
}

template <typename P, typename I>
void launch_groups_vec(const void* src, void* dst, bool restore, I N, I gb, I pieces, I total,
                       unsigned blocks, hipStream_t st) {
  if (restore)
    hipLaunchKernelGGL((k_relayout_groups_vec<true, P, I>), dim3(blocks), dim3(256), 0, st,
                       (const P*)src, (P*)dst, N, gb, pieces, total);
  else
    hipLaunchKernelGGL((k_relayout_groups_vec<false, P, I>), dim3(blocks), dim3(256), 0, st,
                       (const P*)src, (P*)dst, N, gb, pieces, total);
}

hipError_t launch_relayout_groups(const void* src, void* dst, int elem_bytes, int64_t E,
                                  int64_t N, int64_t K, bool restore, hipStream_t st) {
  const int64_t pieces = tiled_group_elems(N, K) / 8;
  const int64_t total = E * pieces;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const int64_t G = K / 32, gb = (G + 7) / 8;
  const uintptr_t piece_bytes = 8u * (uintptr_t)elem_bytes;
  if (G % 8 == 0 && (uintptr_t)src % piece_bytes == 0 && (uintptr_t)dst % piece_bytes == 0) {
    // the largest index: the tiled piece count (canonical indexes are smaller)
    const bool small = total + (int64_t)blocks * 256 < ((int64_t)1 << 31);
    if (elem_bytes == 2) {
      if (small)
        launch_groups_vec<u32x4, uint32_t>(src, dst, restore, (uint32_t)N, (uint32_t)gb,
                                           (uint32_t)pieces, (uint32_t)total, (unsigned)blocks, st);
      else
        launch_groups_vec<u32x4, int64_t>(src, dst, restore, N, gb, pieces, total,
                                          (unsigned)blocks, st);
    } else {
      if (small)
        launch_groups_vec<u32x2, uint32_t>(src, dst, restore, (uint32_t)N, (uint32_t)gb,
                                           (uint32_t)pieces, (uint32_t)total, (unsigned)blocks, st);
      else
        launch_groups_vec<u32x2, int64_t>(src, dst, restore, N, gb, pieces, total,
                                          (unsigned)blocks, st);
    }
    return hipGetLastError();
  }
  if (elem_bytes == 2) {
    if (restore)
      hipLaunchKernelGGL((k_relayout_groups<true, uint16_t>), dim3((unsigned)blocks), dim3(256),
                         0, st, (const uint16_t*)src, (uint16_t*)dst, N, G, gb, pieces, total);
    else
      hipLaunchKernelGGL((k_relayout_groups<false, uint16_t>), dim3((unsigned)blocks), dim3(256),
                         0, st, (const uint16_t*)src, (uint16_t*)dst, N, G, gb, pieces, total);
  } else {
    if (restore)
      hipLaunchKernelGGL((k_relayout_groups<true, uint8_t>), dim3((unsigned)blocks), dim3(256),
                         0, st, (const uint8_t*)src, (uint8_t*)dst, N, G, gb, pieces, total);
    else
      hipLaunchKernelGGL((k_relayout_groups<false, uint8_t>), dim3((unsigned)blocks), dim3(256),
                         0, st, (const uint8_t*)src, (uint8_t*)dst, N, G, gb, pieces, total);
  }
  return hipGetLastError();
}

hipError_t launch_relayout(const int32_t* src, int32_t* dst, int64_t E, int64_t N, int64_t K,
                           bool restore, hipStream_t st) {
  const int64_t units = tiled_words(N, K) / 4;
  const int64_t total = E * units;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const int64_t G = K / 32, nsteps = (K + 63) / 64;
  if (restore)
    hipLaunchKernelGGL(k_relayout<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const u32x4*)src, (u32x4*)dst, N, G, nsteps, units, total);
  else
    hipLaunchKernelGGL(k_relayout<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const u32x4*)src, (u32x4*)dst, N, G, nsteps, units, total);
  return hipGetLastError();
}

}  // namespace w4
