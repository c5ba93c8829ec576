// W4A16 product for small M (decode): Y[M, N] = X[M, K] * dequant(W)^T.
//
// Method: "INT4 QAT end-to-end for RL" §4 (INT4 weights are dequantized in
// registers and multiplied against BF16 activations on BF16 matrix units);
// "Quantization basics: from FP32 to INT4" §2.1 (w' = q * s) and the
// tutorial's opening remark that decode reads every weight once per token,
// so this path is bound by HBM bandwidth.
//
// Mapping (MI355X): a workgroup owns RT*16 consecutive weight rows n and
// all of M; its WAVES waves split K into contiguous ranges of 128-element
// chunks.  In a chunk, lane l = (r = l % 16, kq = l / 16) loads one whole
// 32-element group (16 bytes: four packed words) of weight row r and its
// bf16 scale: a 16-row tile is one fully used 1 KB load per chunk.  Word j
// of every lane feeds MFMA j of the chunk (v_mfma_f32_16x16x32_bf16), so
// each MFMA contracts a permuted set of 32 k; the activation operand uses
// the same permutation (lane (m, kq) loads X[m, 32 g + 8 j .. + 7]), which
// leaves the sum unchanged.  The weight row tile is the A operand, the
// activation rows the B operand: D[n][m], fp32 accumulation.  Each wave
// issues the weight loads of CPW chunks before touching them, to keep
// enough bytes in flight per CU; the activations (at most 32 x K bf16)
// come from L2.  The per-wave partial sums are combined in LDS in wave
// order (deterministic), converted to bf16 once, and stored coalesced.
#include "common.h"

namespace w4 {

template <int MT, int RT, int WAVES, int CPW>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(const uint16_t* __restrict__ X,
                                                     const uint32_t* __restrict__ Wq,
                                                     const uint16_t* __restrict__ S,
                                                     uint16_t* __restrict__ Y, int M, int N,
                                                     int K) {
  constexpr int ROWS = RT * 16;
  constexpr int PAD = 4;
  __shared__ __attribute__((aligned(16))) float part[WAVES][MT * 16][ROWS + PAD];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kq = lane >> 4;
  const int n0 = blockIdx.x * ROWS;
  const int G = K >> 5;                 // groups per row
  const int C = (G + 3) >> 2;           // 128-element chunks
  const int kw = K >> 3;                // packed words per row

  // contiguous chunk range of this wave
  const int c_lo = (int)(((int64_t)C * wave) / WAVES);
  const int c_hi = (int)(((int64_t)C * (wave + 1)) / WAVES);

  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = c_lo; c0 < c_hi; c0 += CPW) {
    u32x4 wv[CPW][RT];
    float sc[CPW][RT];
    // issue every weight load of this pass first
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int g = 4 * (c0 + cc) + kq;
      const bool gv = (c0 + cc < c_hi) && (g < G);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = n0 + rt * 16 + r16;
        if (gv && row < N) {
          wv[cc][rt] = *(const u32x4*)(Wq + (int64_t)row * kw + 4 * g);
          sc[cc][rt] = bf16f(S[(int64_t)row * G + g]);
        } else {
          wv[cc][rt] = u32x4{0u, 0u, 0u, 0u};
          sc[cc][rt] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int g = 4 * (c0 + cc) + kq;
      const bool gv = (c0 + cc < c_hi) && (g < G);
      u32x4 xv[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r16;
        if (gv && m < M) {
          const u32x4* xp = (const u32x4*)(X + (int64_t)m * K + 32 * g);
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[mt][j] = xp[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[mt][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float s = sc[cc][rt];
        const float m8s = -8.0f * s;
        const u32x4 w = wv[cc][rt];
        const u32x4 a0 = dequant8(w.x, s, m8s);
        const u32x4 a1 = dequant8(w.y, s, m8s);
        const u32x4 a2 = dequant8(w.z, s, m8s);
        const u32x4 a3 = dequant8(w.w, s, m8s);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[rt][mt] = mfma16(a0, xv[mt][0], acc[rt][mt]);
          acc[rt][mt] = mfma16(a1, xv[mt][1], acc[rt][mt]);
          acc[rt][mt] = mfma16(a2, xv[mt][2], acc[rt][mt]);
          acc[rt][mt] = mfma16(a3, xv[mt][3], acc[rt][mt]);
        }
      }
    }
  }

  // lane holds D[4*kq + i][r16] of each (rt, mt) tile: weight row
  // rt*16 + 4*kq + i, activation row mt*16 + r16
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *(f32x4*)&part[wave][mt * 16 + r16][rt * 16 + 4 * kq] = acc[rt][mt];
  __syncthreads();

  constexpr int OUT = MT * 16 * ROWS;
  for (int idx = threadIdx.x; idx < OUT; idx += WAVES * 64) {
    const int m = idx / ROWS;
    const int n = idx - m * ROWS;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += part[w][m][n];
    if (m < M && n0 + n < N) Y[(int64_t)m * N + n0 + n] = to_bf16(sum);
  }
}

template <int MT, int RT, int WAVES, int CPW>
static hipError_t run_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                           int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t blocks = (N + RT * 16 - 1) / (RT * 16);
  hipLaunchKernelGGL((k_gemv<MT, RT, WAVES, CPW>), dim3((unsigned)blocks), dim3(WAVES * 64), 0,
                     st, X, (const uint32_t*)Wq, S, Y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* X, const int32_t* Wq, const uint16_t* S, uint16_t* Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 16) return run_gemv<1, 2, 8, 4>(X, Wq, S, Y, M, N, K, st);
  return run_gemv<2, 2, 8, 4>(X, Wq, S, Y, M, N, K, st);
}

}  // namespace w4
