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
