// MoE support kernels: moe_align_block_size, routing, SwiGLU, top-k combine.
//
// Method: "INT4 QAT end-to-end for RL" §4 and the "Quantization-aware
// training" tag summary [35]: before the fused expert GEMMs, the tokens of
// each expert are merged and aligned to a block size chosen from the token
// count and expert spread; gating is fused into one kernel.  The pages give
// no formulas; the kernels implement these readings:
//  * alignment: experts ascending, each expert's pairs f = t*k + j in
//    ascending f, padded with the sentinel T*k to a multiple of B, one
//    expert id per block, -1 / sentinel past the end;
//  * routing: softmax over the experts, the k largest logits (ties to the
//    lower index), renormalised weights (= softmax over the chosen logits);
//  * activation: silu(gate) * up with gate the first half of each row;
//  * combine: fp32 sum over j = 0..k-1 in order of w[t, j] * h2[t*k + j].
#include "common.h"

namespace w4 {

// ------------------------------------------------------------------ align --
//
// One workgroup of 1024 threads (the alignment touches T*k ids, a few
// thousand to a few tens of thousands, and must be stable and exact).  Wave
// w owns the contiguous pair range [w*P/16, (w+1)*P/16).
//  1. per-wave histograms of experts in LDS (atomics on the wave's own
//     counters, which the wave clears itself: counts do not depend on
//     order);
//  2. exclusive scan of the padded counts -> segment starts; then, per
//     expert, a scan over the waves in wave order turns the wave's count
//     into the position where its first pair of that expert goes;
//  3. every wave walks its range in order, 64 pairs per round: the lanes
//     with the same expert are found with one ballot per bit of the id
//     (ceil(log2 E) of them), giving each lane its rank among equal lanes
//     before it; the
//     round's first lane of each expert then advances the wave's position
//     for that expert.  No barrier between rounds: positions are private to
//     the wave, read and advanced in program order;
//  4. padding slots, the tail and the block -> expert map are written by
//     disjoint threads, so no location is written twice.
constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 1024;

// Inclusive prefix sum over the wave's 64 lanes (DPP row shifts within
// each 16-lane row, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__global__ __launch_bounds__(kAlignThreads) void k_align(const int32_t* __restrict__ ids,
                                                         int P, int E, int B, int cap,
                                                         int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ expert_ids,
                                                         int32_t* __restrict__ ntpp) {
  __shared__ int pos[kAlignWaves][kMaxExperts];   // counts, then positions
  __shared__ int start[kMaxExperts];
  __shared__ int count[kMaxExperts];
  __shared__ int wave_tot[kAlignWaves];
  __shared__ int total_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = (P + kAlignWaves - 1) / kAlignWaves;
  const int f_lo = min(P, wave * chunk);
  const int f_hi = min(P, f_lo + chunk);

  // ids of kBatch rounds are loaded together (the rounds would otherwise
  // wait on one load each)
  constexpr int kBatch = 8;
  auto load_batch = [&](int base, int (&v)[kBatch]) {
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int f = base + 64 * r + lane;
      v[r] = (f < f_hi) ? ids[f] : -1;
    }
  };

  // the wave's first batch of ids is in flight while it clears its own
  // counters (only this wave touches them until the barrier after step 1,
  // and its LDS accesses take effect in program order)
  int v0[kBatch];
  load_batch(f_lo, v0);
  for (int i = lane; i < E; i += 64) pos[wave][i] = 0;

  // 1. per-wave histograms; a wave whose range fits one batch keeps its
  // ids in registers for step 3
  const bool one_batch = f_hi - f_lo <= 64 * kBatch;
  for (int base = f_lo; base < f_hi; base += 64 * kBatch) {
    int v[kBatch];
    if (base == f_lo) {
#pragma unroll
      for (int r = 0; r < kBatch; ++r) v[r] = v0[r];
    } else {
      load_batch(base, v);
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r)
      if (v[r] >= 0 && v[r] < E) atomicAdd(&pos[wave][v[r]], 1);
  }
  __syncthreads();

  // 2. segment starts (thread e owns expert e and keeps its 16 wave counts
  // in registers), then per-wave positions
  int c = 0;
  int hc[kAlignWaves];
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      hc[w] = pos[w][tid];
      c += hc[w];
    }
    count[tid] = c;
  }
  const int padded = (tid < E) ? ((c + B - 1) / B) * B : 0;
  const int incl = wave_incl_scan(padded);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int wprefix = 0;
  for (int w = 0; w < wave; ++w) wprefix += wave_tot[w];
  if (tid < E) {
    const int s0 = wprefix + incl - padded;
    start[tid] = s0;
    int run = s0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      pos[w][tid] = run;
      run += hc[w];
    }
  }
  if (tid == kAlignThreads - 1) total_sh = wprefix + incl;
  __syncthreads();
  const int total = total_sh;

  // 3. stable placement, each wave through its own range (ids from the
  // registers of step 1 when they fit one batch); the expert ids need
  // nbits bits, one ballot each
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 1;
  for (int base0 = f_lo; base0 < f_hi; base0 += 64 * kBatch) {
    int v[kBatch];
    if (one_batch) {
#pragma unroll
      for (int r = 0; r < kBatch; ++r) v[r] = v0[r];
    } else {
      load_batch(base0, v);
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int f = base0 + 64 * r + lane;
      if (base0 + 64 * r >= f_hi) break;               // wave-uniform: past the range
      const int e = (v[r] >= 0 && v[r] < E) ? v[r] : -1;
      const bool valid = e >= 0;
      uint64_t match = ballot64(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool b = valid && ((e >> bit) & 1);
        const uint64_t ones = ballot64(b);
        match &= ((e >> bit) & 1) ? ones : ~ones;
      }
      const int rank = __popcll(match & lt_mask);
      int p = 0;
      if (valid) p = pos[wave][e] + rank;
      // every lane has read its position (same wave, program order) before
      // the expert's first lane advances it
      if (valid && rank == 0) pos[wave][e] += __popcll(match);
      if (valid) sorted_ids[p] = f;
    }
  }

  // 4. padding slots inside segments, the tail, and the block map
  if (tid < E) {
    const int s0 = start[tid];
    const int cnt = count[tid];
    const int pe = ((cnt + B - 1) / B) * B;
    for (int q = s0 + cnt; q < s0 + pe; ++q) sorted_ids[q] = P;
    for (int b = s0 / B; b < (s0 + pe) / B; ++b) expert_ids[b] = tid;
  }
  for (int q = total + tid; q < cap; q += kAlignThreads) sorted_ids[q] = P;
  for (int b = total / B + tid; b < cap / B; b += kAlignThreads) expert_ids[b] = -1;
  if (tid == 0) ntpp[0] = total;
}

hipError_t launch_align(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t B,
                        int64_t cap, int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                        hipStream_t st) {
  hipLaunchKernelGGL(k_align, dim3(1), dim3(kAlignThreads), 0, st, ids, (int)(T * k), (int)E,
                     (int)B, (int)cap, sorted_ids, expert_ids, ntpp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ route --
// One wave per token.  Round j picks the j-th expert: the wave maximum of
// the logits not yet taken (v_max_f32 in each lane, then two DPP quad
// swaps, the two DPP mirrors within each 16-lane row, v_permlane16_swap and
// v_permlane32_swap across rows: every lane ends with the maximum), then
// the lowest expert index holding that value (one ballot per candidate
// slot, slots in index order).  v_max_f32 returns the other operand when
// one is NaN, so NaN logits and taken experts never win while any expert
// with a number is left; -0 equals +0, so equal logits tie on the index.
// Lane j keeps pick j; the weights are exp(l_j - l_0) / sum over the k
// picks, which equals the softmax over all experts renormalised to the
// picked set.  If fewer than k experts have a number, the remaining picks
// are the lowest untaken indices (distinct; unspecified by the ABI).
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_fmax(float a) {
  const float b =
      __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), CTRL, 0xF, 0xF, false));
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_fmax(float a) {
  a = dpp_fmax<0xB1>(a);     // quad_perm [1, 0, 3, 2]
  a = dpp_fmax<0x4E>(a);     // quad_perm [2, 3, 0, 1]
  a = dpp_fmax<0x141>(a);    // row_half_mirror: the other quad of each 8 lanes
  a = dpp_fmax<0x140>(a);    // row_mirror: the other 8 lanes of each row
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a),
                                                    false, false);   // rows (0, 1), (2, 3)
    a = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a),
                                                    false, false);   // rows (0, 1) with (2, 3)
    a = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return a;
}

// wave-wide sum, every lane ends with it (same ladder as wave_fmax)
__device__ __forceinline__ float wave_fsum(float a) {
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, false));
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, false));
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x141, 0xF, 0xF, false));
  a += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x140, 0xF, 0xF, false));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a),
                                                    false, false);
    a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a),
                                                    false, false);
    a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return a;
}

}  // namespace

// NPER: candidates per lane (E <= 64 NPER); candidate i of lane l is expert l + 64 i
template <int NPER>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int32_t* __restrict__ ids,
                                               float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole waves: every lane of a live wave takes part below
  const float* row = logits + (int64_t)t * E;
  const float qnan = __uint_as_float(0x7FC00000u);
  float v[NPER];
  uint32_t live = 0;    // bit i: candidate i is an expert not yet taken
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    const float x = (e < E) ? row[e] : qnan;
    v[i] = (x != x) ? qnan : x;    // any NaN becomes a quiet one, which v_max_f32 skips
    live |= (e < E) ? (1u << i) : 0u;
  }
  int my_id = 0;
  float my_val = 0.0f;
  for (int j = 0; j < k; ++j) {
    float m = qnan;
#pragma unroll
    for (int i = 0; i < NPER; ++i) m = fmaxf(m, ((live >> i) & 1u) ? v[i] : qnan);
    m = wave_fmax(m);
    int win = -1;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint64_t b = __ballot(((live >> i) & 1u) && v[i] == m);
      if (win < 0 && b) win = 64 * i + (int)__builtin_ctzll(b);
    }
    if (win < 0) {        // no expert with a number left: lowest untaken index
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        const uint64_t b = __ballot((live >> i) & 1u);
        if (win < 0 && b) win = 64 * i + (int)__builtin_ctzll(b);
      }
    }
    if (lane == (win & 63)) live &= ~(1u << (win >> 6));
    if (lane == j) {
      my_id = win;
      my_val = m;
    }
  }
  // lane j < k holds pick j; l_0 (the largest) from lane 0
  const float l0 = __shfl(my_val, 0);
  const float ex = (lane < k) ? expf(my_val - l0) : 0.0f;
  const float sum = wave_fsum(ex);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    wts[(int64_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                        float* w, hipStream_t st) {
  const dim3 g((unsigned)((T + 3) / 4)), b(256);
  if (E <= 64)
    hipLaunchKernelGGL(k_route<1>, g, b, 0, st, logits, (int)T, (int)E, (int)k, ids, w);
  else if (E <= 128)
    hipLaunchKernelGGL(k_route<2>, g, b, 0, st, logits, (int)T, (int)E, (int)k, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_route<4>, g, b, 0, st, logits, (int)T, (int)E, (int)k, ids, w);
  else if (E <= 384)
    hipLaunchKernelGGL(k_route<6>, g, b, 0, st, logits, (int)T, (int)E, (int)k, ids, w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_route<8>, g, b, 0, st, logits, (int)T, (int)E, (int)k, ids, w);
  else
    hipLaunchKernelGGL(k_route<16>, g, b, 0, st, logits, (int)T, (int)E, (int)k, ids, w);
  return hipGetLastError();
}

// --------------------------------------------------------------- silu_mul --
__global__ __launch_bounds__(256) void k_silu_mul(const uint32_t* __restrict__ H1,
                                                  uint32_t* __restrict__ A, int64_t R,
                                                  int64_t I2) {
  // I2 = I / 2 bf16 pairs per output row; input rows hold 2 * I2 pairs
  const int64_t n = R * I2;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / I2;
    const int64_t c = i - r * I2;
    const uint32_t g = H1[r * 2 * I2 + c];
    const uint32_t u = H1[r * 2 * I2 + I2 + c];
    const float g0 = bf16_lo(g), g1 = bf16_hi(g);
    const float a0 = silu_mul(g0, bf16_lo(u));
    const float a1 = silu_mul(g1, bf16_hi(u));
    A[i] = pk_bf16(a0, a1);
  }
}

hipError_t launch_silu_mul(const uint16_t* H1, uint16_t* A, int64_t R, int64_t I,
                           hipStream_t st) {
  const int64_t n = R * (I / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint32_t*)H1, (uint32_t*)A, R, I / 2);
  return hipGetLastError();
}

// ---------------------------------------------------------------- moe_sum --
__global__ __launch_bounds__(256) void k_moe_sum(const uint32_t* __restrict__ H2,
                                                 const float* __restrict__ w,
                                                 uint32_t* __restrict__ Out, int64_t T, int k,
                                                 int64_t H2p) {
  const int64_t n = T * H2p;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / H2p;
    const int64_t c = i - t * H2p;
    float s0 = 0.0f, s1 = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float wj = w ? w[t * k + j] : 1.0f;
      const uint32_t hv = H2[(t * k + j) * H2p + c];
      s0 = __builtin_fmaf(wj, bf16_lo(hv), s0);
      s1 = __builtin_fmaf(wj, bf16_hi(hv), s1);
    }
    Out[i] = pk_bf16(s0, s1);
  }
}

// Vector path: one workgroup row per token (grid y), 8 bf16 per thread with
// 16-byte loads and stores; the same per-element sum order as k_moe_sum.
__global__ __launch_bounds__(256) void k_moe_sum8(const u32x4* __restrict__ H2,
                                                  const float* __restrict__ w,
                                                  u32x4* __restrict__ Out, int64_t T, int k,
                                                  int64_t H8) {
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < H8;
         c += (int64_t)gridDim.x * 256) {
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      // the rows of 8 pairs are loaded together, then summed in pair order
      for (int j0 = 0; j0 < k; j0 += 8) {
        u32x4 hv[8];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = j0 + u;
          hv[u] = j < k ? H2[(t * k + j) * H8 + c] : u32x4{0u, 0u, 0u, 0u};
          wj[u] = j < k ? (w ? w[t * k + j] : 1.0f) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j0 + u >= k) break;
          const uint32_t d[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s[2 * q] = __builtin_fmaf(wj[u], bf16_lo(d[q]), s[2 * q]);
            s[2 * q + 1] = __builtin_fmaf(wj[u], bf16_hi(d[q]), s[2 * q + 1]);
          }
        }
      }
      Out[t * H8 + c] = u32x4{pk_bf16(s[0], s[1]), pk_bf16(s[2], s[3]), pk_bf16(s[4], s[5]),
                              pk_bf16(s[6], s[7])};
    }
  }
}

hipError_t launch_moe_sum(const uint16_t* H2, const float* w, uint16_t* Out, int64_t T, int32_t k,
                          int64_t H, hipStream_t st) {
  if (H % 8 == 0 && ((uintptr_t)H2 & 15) == 0 && ((uintptr_t)Out & 15) == 0) {
    const int64_t H8 = H / 8;
    const int64_t bx = (H8 + 255) / 256;
    const int64_t by = T < 65535 ? T : 65535;
    hipLaunchKernelGGL(k_moe_sum8, dim3((unsigned)bx, (unsigned)by), dim3(256), 0, st,
                       (const u32x4*)H2, w, (u32x4*)Out, T, (int)k, H8);
    return hipGetLastError();
  }
  const int64_t n = T * (H / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_moe_sum, dim3((unsigned)blocks), dim3(256), 0, st, (const uint32_t*)H2, w,
                     (uint32_t*)Out, T, (int)k, H / 2);
  return hipGetLastError();
}

}  // namespace w4
