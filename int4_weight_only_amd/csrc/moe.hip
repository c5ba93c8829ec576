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
// thousand to a few tens of thousands, and must be stable and exact).
//  1. histogram of experts (LDS atomics: the counts do not depend on order);
//  2. exclusive scan of the padded counts -> segment starts;
//  3. stable placement, 1024 pairs per round: inside a wave the lanes with
//     the same expert are found with ten ballots (one per bit of the id),
//     giving each lane its rank among equal lanes before it; a per-expert
//     prefix over the 16 waves (in wave order, in LDS) and a running count
//     per expert place the round after all earlier rounds;
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
  __shared__ int count[kMaxExperts];
  __shared__ int start[kMaxExperts];
  __shared__ int running[kMaxExperts];
  __shared__ int wave_base[kAlignWaves][kMaxExperts];
  __shared__ int wave_tot[kAlignWaves];
  __shared__ int total_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < kMaxExperts; e += kAlignThreads) {
    count[e] = 0;
    running[e] = 0;
  }
  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads)
    (&wave_base[0][0])[i] = 0;
  __syncthreads();

  // 1. histogram
  for (int f = tid; f < P; f += kAlignThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&count[e], 1);
  }
  __syncthreads();

  // 2. exclusive scan of padded counts (thread e owns expert e)
  int padded = 0;
  if (tid < E) padded = ((count[tid] + B - 1) / B) * B;
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
  if (tid < E) start[tid] = wprefix + incl - padded;
  if (tid == kAlignThreads - 1) total_sh = wprefix + incl;
  __syncthreads();
  const int total = total_sh;

  // 3. stable placement
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < P; base += kAlignThreads) {
    const int f = base + tid;
    int e = -1;
    if (f < P) {
      const int v = ids[f];
      if (v >= 0 && v < E) e = v;
    }
    const bool valid = e >= 0;
    uint64_t match = ballot64(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool b = valid && ((e >> bit) & 1);
      const uint64_t ones = ballot64(b);
      match &= ((e >> bit) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(match & lt_mask);
    const bool leader = valid && rank == 0;
    if (leader) wave_base[wave][e] = __popcll(match);
    __syncthreads();
    if (tid < E) {
      int run = running[tid];
#pragma unroll
      for (int w = 0; w < kAlignWaves; ++w) {
        // only entries some lane of wave w leads are rewritten (and that
        // leader clears them after placement); absent experts stay 0
        const int c = wave_base[w][tid];
        if (c != 0) wave_base[w][tid] = run;
        run += c;
      }
      running[tid] = run;
    }
    __syncthreads();
    if (valid) sorted_ids[start[e] + wave_base[wave][e] + rank] = f;
    // same wave, program order: every lane has read its base before the
    // leader clears the entry for the next round
    if (leader) wave_base[wave][e] = 0;
  }

  // 4. padding slots inside segments, the tail, and the block map
  if (tid < E) {
    const int s0 = start[tid];
    const int c = count[tid];
    const int pe = ((c + B - 1) / B) * B;
    for (int p = s0 + c; p < s0 + pe; ++p) sorted_ids[p] = P;
    for (int b = s0 / B; b < (s0 + pe) / B; ++b) expert_ids[b] = tid;
  }
  for (int p = total + tid; p < cap; p += kAlignThreads) sorted_ids[p] = P;
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
constexpr int kRouteMaxPerLane = kMaxExperts / 64;

__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int32_t* __restrict__ ids,
                                               float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? row[e] : -__builtin_inff();
  }
  float picked[16];
  int picked_id[16];
  for (int j = 0; j < k; ++j) {
    // lane-local best (first index wins on ties: i ascending = index ascending)
    float best = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > best || (v[i] == best && e < bi))) {
        best = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    picked[j] = best;
    picked_id[j] = bi;
    // remove the pick
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i)
      if (lane + 64 * i == bi) v[i] = -__builtin_inff();
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
  const int64_t blocks = (T + 3) / 4;
  hipLaunchKernelGGL(k_route, dim3((unsigned)blocks), dim3(256), 0, st, logits, (int)T, (int)E,
                     (int)k, ids, w);
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
    const float a0 = g0 / (1.0f + expf(-g0)) * bf16_lo(u);
    const float a1 = g1 / (1.0f + expf(-g1)) * bf16_hi(u);
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

hipError_t launch_moe_sum(const uint16_t* H2, const float* w, uint16_t* Out, int64_t T, int32_t k,
                          int64_t H, hipStream_t st) {
  const int64_t n = T * (H / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_moe_sum, dim3((unsigned)blocks), dim3(256), 0, st, (const uint32_t*)H2, w,
                     (uint32_t*)Out, T, (int)k, H / 2);
  return hipGetLastError();
}

}  // namespace w4
