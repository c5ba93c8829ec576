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
//     counters: counts do not depend on order);
//  2. exclusive scan of the padded counts -> segment starts; then, per
//     expert, a scan over the waves in wave order turns the wave's count
//     into the position where its first pair of that expert goes;
//  3. every wave walks its range in order, 64 pairs per round: the lanes
//     with the same expert are found with ten ballots (one per bit of the
//     id), giving each lane its rank among equal lanes before it; the
//     round's first lane of each expert then advances the wave's position
//     for that expert.  No barrier between rounds: positions are private to
//     the wave, read and advanced in program order;
//  4. padding slots, the tail and the block -> expert map are written by
//     disjoint threads, so no location is written twice.
constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 1024;

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

  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&pos[0][0])[i] = 0;
  __syncthreads();

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

  // 1. per-wave histograms
  for (int base = f_lo; base < f_hi; base += 64 * kBatch) {
    int v[kBatch];
    load_batch(base, v);
#pragma unroll
    for (int r = 0; r < kBatch; ++r)
      if (v[r] >= 0 && v[r] < E) atomicAdd(&pos[wave][v[r]], 1);
  }
  __syncthreads();

  // 2. segment starts (thread e owns expert e), then per-wave positions
  int c = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) c += pos[w][tid];
    count[tid] = c;
  }
  const int padded = (tid < E) ? ((c + B - 1) / B) * B : 0;
  int incl = padded;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
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
      const int n = pos[w][tid];
      pos[w][tid] = run;
      run += n;
    }
  }
  if (tid == kAlignThreads - 1) total_sh = wprefix + incl;
  __syncthreads();
  const int total = total_sh;

  // 3. stable placement, each wave through its own range
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base0 = f_lo; base0 < f_hi; base0 += 64 * kBatch) {
    int v[kBatch];
    load_batch(base0, v);
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int f = base0 + 64 * r + lane;
      const int e = (v[r] >= 0 && v[r] < E) ? v[r] : -1;
      const bool valid = e >= 0;
      uint64_t match = ballot64(valid);
#pragma unroll
      for (int bit = 0; bit < 10; ++bit) {
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
// One wave per token: repeated wave-wide argmax picks the k experts in
// descending logit order (ties: lower index); the weights are
// exp(l_j - l_0) / sum_i exp(l_i - l_0) over the picked logits, which equals
// the softmax over all experts renormalised to the picked set.
//
// Each candidate is one 64-bit key that orders like (logit, -index): the
// high word maps the fp32 logit to an unsigned integer of the same order
// (sign set: all bits flipped; else the sign bit set), the low word is
// ~index (-0 counts as +0).  A removed pick and a NaN logit get key 0, below every real key
// (-inf included), so they are never picked again while any expert is left.
// The wave maximum of the keys takes two DPP quad swaps and the two DPP
// mirrors within each 16-lane row, then v_permlane16_swap and
// v_permlane32_swap across rows: no LDS round trip.
namespace {

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  const uint32_t u = __float_as_uint(v + 0.0f);   // -0 -> +0: equal logits tie on the index
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (v != v) ? 0ull : ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t a) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)a, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(a >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t b = ((uint64_t)hi << 32) | lo;
  return b > a ? b : a;
}

__device__ __forceinline__ uint64_t wave_max_key(uint64_t a) {
  a = dpp_max<0xB1>(a);     // quad_perm [1, 0, 3, 2]
  a = dpp_max<0x4E>(a);     // quad_perm [2, 3, 0, 1]
  a = dpp_max<0x141>(a);    // row_half_mirror: the other quad of each 8 lanes
  a = dpp_max<0x140>(a);    // row_mirror: the other 8 lanes of each row
  {
    // rows (0, 1) and (2, 3): each lane meets the same lane of the paired row
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)a, (uint32_t)a, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(a >> 32), (uint32_t)(a >> 32),
                                                    false, false);
    const uint64_t x = ((uint64_t)h[0] << 32) | l[0], y = ((uint64_t)h[1] << 32) | l[1];
    a = x > y ? x : y;
  }
  {
    // rows (0, 1) with (2, 3)
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)a, (uint32_t)a, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(a >> 32), (uint32_t)(a >> 32),
                                                    false, false);
    const uint64_t x = ((uint64_t)h[0] << 32) | l[0], y = ((uint64_t)h[1] << 32) | l[1];
    a = x > y ? x : y;
  }
  return a;
}

}  // namespace

// NPER: candidates per lane (E <= 64 NPER)
template <int NPER>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int32_t* __restrict__ ids,
                                               float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole waves: every lane of a live wave takes part below
  const float* row = logits + (int64_t)t * E;
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? route_key(row[e], e) : 0ull;
  }
  float picked[16];
  int picked_id[16];
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_key(best);
    const int bi = (int)~(uint32_t)best;
    picked[j] = key_value(best);
    picked_id[j] = bi;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + 64 * i == bi) key[i] = 0ull;
  }
  if (lane == 0) {
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += expf(picked[j] - picked[0]);
    for (int j = 0; j < k; ++j) {
      ids[(int64_t)t * k + j] = picked_id[j];
      wts[(int64_t)t * k + j] = expf(picked[j] - picked[0]) / sum;
    }
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
      for (int j = 0; j < k; ++j) {
        const float wj = w ? w[t * k + j] : 1.0f;
        const u32x4 hv = H2[(t * k + j) * H8 + c];
        const uint32_t d[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s[2 * q] = __builtin_fmaf(wj, bf16_lo(d[q]), s[2 * q]);
          s[2 * q + 1] = __builtin_fmaf(wj, bf16_hi(d[q]), s[2 * q + 1]);
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
