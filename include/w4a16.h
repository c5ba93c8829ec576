/*
 * w4a16.h -- C ABI of libw4a16.so, INT4 weight-only quantization and the
 * W4A16 matrix multiply on AMD Instinct MI355X (gfx950).
 *
 * Method sources (cited by page title and section):
 *  [QB]  "Quantization basics: from FP32 to INT4" (量化基础：从 FP32 到 INT4
 *        的压缩艺术, wsisp.com tutorial): §1.3 INT4 grid [-8, 7]; §2.1 affine
 *        map and its inverse; §2.2 symmetric scale s = max|x| / q_max;
 *        §2.4 error bound; §3 per-group granularity; §5 round must be a real
 *        round (half-to-even), not a truncating cast.
 *  [RL]  "INT4 QAT end-to-end for RL" (SGLang RL / slime / Miles write-up):
 *        §2.1 fake quantization in the training forward pass; §3.2 real
 *        quantization at weight update, 8 INT4 packed per INT32 (Fig. 4);
 *        §4 W4A16 inference, moe_align_block_size, fused MoE and gating.
 *  [TAG] "Quantization-aware training" tag summary (量化感知训练, reportify):
 *        [11] one scale per 1 x 32 group; [32] two 4-bit weights per byte;
 *        [35] block size picked from the token count and expert spread.
 *
 * Conventions for every entry point
 *  - All tensors are row-major and contiguous, in device memory (pointers
 *    from hipMalloc or a framework allocator on the current device).
 *  - bfloat16 values are passed as their 16-bit patterns (uint16_t).
 *  - The caller owns all memory; the library allocates and frees nothing.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; no call synchronizes or reads back.
 *  - Arguments are validated before anything is enqueued; on any error the
 *    outputs are left untouched and a nonzero status is returned.
 *  - Pointers marked "16-byte aligned" must be; others need their natural
 *    alignment.  Inputs and outputs must not overlap unless stated.
 *  - Sizes are int64_t; a size of 0 is a valid no-op where stated.
 *  - Calls are deterministic: the same inputs give bitwise-identical outputs
 *    (no floating-point atomics; reductions in a fixed order).
 *  - Weight layout: Wq int32 [N, K/8]: nibble j (bits 4j..4j+3) of word w of
 *    row n holds the two's-complement INT4 code of element k = 8w + j.
 *    Scales S bf16 [N, K/32]: one per 32 consecutive k of a row.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define W4_OK               0
#define W4_ERR_NULL         1  /* a required pointer is NULL */
#define W4_ERR_SHAPE        2  /* a size is negative or K % 32 != 0, etc. */
#define W4_ERR_MISALIGNED   3  /* a pointer lacks the required alignment */
#define W4_ERR_UNSUPPORTED  4  /* valid but outside what the kernels cover */
#define W4_ERR_HIP          5  /* a HIP launch failed; see w4_last_hip_error */

/* Human-readable name of a status code (static string, never NULL). */
const char* w4_status_string(int status);

/* The hipError_t of the last failed launch on the calling thread (0 if
 * none).  Thread-local; reset by no call except a later failure. */
int w4_last_hip_error(void);

/* Library version string. */
const char* w4_version(void);

/*
 * w4_quantize_pack -- symmetric group-wise INT4 quantization + packing.
 * [QB] §2.2 (z = 0, s = max|w| / 7), [TAG] [11] (1 x 32 groups), [RL] §3.2
 * (eight codes per INT32).
 *
 *   for each row n and group g of 32 consecutive k:
 *     amax = max |W[n, 32g .. 32g+31]|                       (exact)
 *     S[n, g] = bf16_rne( fp32(amax) / 7 )                   (IEEE fp32 div)
 *     q = S == 0 ? 0 : clamp( rint_half_even( fp32(w) / fp32(S) ), -8, 7 )
 *     Wq packs q along k as described in the header comment.
 *
 * W   bf16 [N, K], 16-byte aligned, finite values (NaN/Inf: undefined codes).
 * Wq  int32 [N, K/8] output, 16-byte aligned.
 * S   bf16 [N, K/32] output, 2-byte aligned.
 * K % 32 == 0, N >= 0, K >= 0 (N*K == 0 is a no-op).
 * Outputs are bit-exact with the plain definition above.
 */
int w4_quantize_pack(const uint16_t* W, int64_t N, int64_t K,
                     int32_t* Wq, uint16_t* S, void* stream);

/*
 * w4_fake_quant -- QAT forward quantize-dequantize ([RL] §2.1).
 *   W_fq[n, k] = bf16_rne( q[n, k] * S[n, k/32] )
 * with q and S exactly as w4_quantize_pack computes them; the fp32 product
 * is exact, so W_fq equals the dequantized packed weights bit for bit.
 * W, W_fq bf16 [N, K], 16-byte aligned.  W_fq == W (in place) is allowed;
 * any other overlap is not.  K % 32 == 0.
 */
int w4_fake_quant(const uint16_t* W, int64_t N, int64_t K,
                  uint16_t* W_fq, void* stream);

/*
 * w4_quantize_pack_asym -- asymmetric (zero-point) group-wise INT4
 * quantization + packing ([QB] §2.1 affine map, §2.3 asymmetric scale and
 * zero point; [TAG] [11] 1 x 32 groups).  Unsigned grid [0, 15]; the range
 * is widened to contain 0 (the zero-point bullet of [QB] §2.1: 0 is on
 * the grid).  For each row n and group g:
 *   lo = min(0, min w), hi = max(0, max w)                    (exact)
 *   S[n, g] = bf16_rne( fp32(hi - lo) / 15 )                  (fp32 sub, IEEE div)
 *   Z[n, g] = S == 0 ? 0 : clamp( rint_half_even(0 - lo / S), 0, 15 )
 *   q = S == 0 ? 0 : clamp( rint_half_even(w / S) + Z, 0, 15 )
 *   Wq packs the unsigned q along k (nibble j of word w holds k = 8w + j).
 * W bf16 [N, K], 16-byte aligned, finite, with every group's hi - lo
 * finite in fp32 (otherwise the codes are undefined).  Wq int32 [N, K/8],
 * 16-byte aligned.  S bf16 [N, K/32], 2-byte aligned.  Z uint8 [N, K/32].
 * K % 32 == 0.  Bit-exact with the definition above.
 */
int w4_quantize_pack_asym(const uint16_t* W, int64_t N, int64_t K,
                          int32_t* Wq, uint16_t* S, uint8_t* Z, void* stream);

/*
 * w4_fake_quant_asym -- QAT forward with the asymmetric grid:
 *   W_fq[n, k] = bf16_rne( (q[n, k] - Z[n, k/32]) * S[n, k/32] )
 * with q, S, Z as w4_quantize_pack_asym computes them (the fp32 product is
 * exact).  Layout, alignment and in-place rules as w4_fake_quant.
 */
int w4_fake_quant_asym(const uint16_t* W, int64_t N, int64_t K,
                       uint16_t* W_fq, void* stream);

/*
 * w4_dequant -- packed codes back to bf16 weights ([RL] §4 dequantization,
 * the values the products multiply; [RL] §2.1: the same values fake
 * quantization gives, so restoring a bf16 copy of packed weights needs no
 * source weights):
 *   W[n, k] = bf16_rne( q[n, k] * S[n, k/32] )   (the fp32 product is exact)
 * Wq int32 [N, K/8] (4-byte aligned), S bf16 [N, K/32], W bf16 [N, K]
 * output, 16-byte aligned, not overlapping the inputs.  K % 32 == 0; N or
 * K == 0 is a no-op.  Bit-exact: w4_dequant(w4_quantize_pack(W)) equals
 * w4_fake_quant(W).
 */
int w4_dequant(const int32_t* Wq, const uint16_t* S, int64_t N, int64_t K,
               uint16_t* W, void* stream);

/*
 * w4_dequant_asym -- the same for zero-point codes ([QB] §2.1 inverse map):
 *   W[n, k] = bf16_rne( (q[n, k] - Z[n, k/32]) * S[n, k/32] )
 * with q the unsigned nibbles of Wq and Z uint8 [N, K/32] in [0, 15].
 * w4_dequant_asym(w4_quantize_pack_asym(W)) equals w4_fake_quant_asym(W).
 */
int w4_dequant_asym(const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                    int64_t N, int64_t K, uint16_t* W, void* stream);

/*
 * w4a16_gemm -- Y = X * dequant(Wq, S)^T ([RL] §4: INT4 weights, BF16
 * activations, dequantized in registers, BF16 matrix cores, fp32
 * accumulation).
 *   Y[m, n] = bf16_rne( sum_k X[m, k] * bf16_rne(q[n, k] * S[n, k/32]) )
 * accumulated in fp32 (order unspecified but fixed).
 * X  bf16 [M, K], 16-byte aligned.   Wq int32 [N, K/8], 16-byte aligned.
 * S  bf16 [N, K/32].                 Y  bf16 [M, N] output, 4-byte aligned.
 * K % 32 == 0; M, N >= 0 (M*N == 0 is a no-op); K == 0 writes zeros.
 * Small M (<= 32, K <= 2^24) runs the decode kernel, larger M the tiled
 * MFMA kernel, which needs X and Wq each below 2 GiB (32-bit buffer
 * offsets): W4_ERR_UNSUPPORTED otherwise.  Both kernels multiply the
 * weights of the definition, bf16_rne(q * s), at every M and K.  Scales
 * must stay below 2^118 (weights below about 2e36): the dequant step of
 * both kernels overflows beyond.
 */
int w4a16_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
               uint16_t* Y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * w4a16_gemm_asym -- the same product with zero-point weights ([QB] §2.1
 * inverse map x_hat = (q - z) s, §2.3 asymmetric quantization; [RL] §4
 * for the mixed-precision product):
 *   Y[m, n] = bf16_rne( sum_k X[m, k] * w'[n, k] )
 *   w'[n, k] = bf16_rne( (q[n, k] - Z[n, k/32]) * S[n, k/32] )   (exact product)
 * with q the unsigned nibbles of Wq, as w4_quantize_pack_asym writes them.
 * Z uint8 [N, K/32], values in [0, 15] (other values: results undefined).
 * Layout, alignment, size limits, dispatch and accumulation as w4a16_gemm;
 * both kernels multiply the rounded w' above.  Scales below 2^118, as in
 * w4a16_gemm.
 */
int w4a16_gemm_asym(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                    const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                    void* stream);

/*
 * Kernel-order code layout ([RL] §4: after loading INT4 weights the
 * inference engine converts them into the layout its kernel reads, and
 * restores the original layout before new weights are loaded).  Per [N, K]
 * matrix: ceil(N/32) x ceil(K/64) blocks of 1 KB; block (r, c) starts at
 * byte 1024 * (r * ceil(K/64) + c); its 16-byte unit u (u = 0..63) holds
 * the 16 bytes of group 2c + u/32 (32 codes, as in the canonical word
 * layout) of row 32r + u%32.  Units of rows >= N or groups >= K/32 are
 * zero.  E matrices (stacked experts) are stored one after the other.
 * Scales and zero points keep their [N, K/32] layout.  The products read
 * each step's codes of 32 rows as one contiguous kilobyte.
 *
 * w4_repacked_words -- int32 words of one matrix in kernel order:
 *   ceil(N/32) * ceil(K/64) * 256.  -1 on invalid sizes.
 */
int64_t w4_repacked_words(int64_t N, int64_t K);

/*
 * w4_repack -- canonical codes Wq [E, N, K/8] -> kernel order
 * Wt [E * w4_repacked_words(N, K)] (padding units written as zero).
 * w4_restore -- the inverse: kernel order -> canonical (padding ignored).
 * Both are pure permutations of 16-byte units: w4_restore(w4_repack(Wq))
 * equals Wq bit for bit.  Symmetric and zero-point codes alike.  Wq and Wt
 * 16-byte aligned, not overlapping; K % 32 == 0; E, N or K == 0 is a no-op.
 */
int w4_repack(const int32_t* Wq, int64_t E, int64_t N, int64_t K, int32_t* Wt,
              void* stream);
int w4_restore(const int32_t* Wt, int64_t E, int64_t N, int64_t K, int32_t* Wq,
               void* stream);

/*
 * w4_repacked_group_elems -- elements of one [N, K/32] per-group array
 *   (scales or zero points) in kernel order: ceil(N/16) * ceil(K/256) * 128.
 *   -1 on invalid sizes.
 *
 * w4_repack_groups -- per-group values A [E, N, K/32] (elem_bytes = 2: bf16
 * scales; 1: uint8 zero points) -> kernel order At
 * [E * w4_repacked_group_elems(N, K)]: per matrix, ceil(N/16) x ceil(K/256)
 * blocks of 128 elements, block (r, c) at element 128 (r ceil(K/256) + c),
 * element 8 i + j of a block = row 16 r + i, group 8 c + j; elements past N
 * or K/32 are written as zero.  The products then read a wave's eight
 * values of 16 consecutive rows as one contiguous piece.
 * w4_restore_groups -- the inverse (padding ignored).  Pure permutations:
 * w4_restore_groups(w4_repack_groups(A)) equals A bit for bit.  Buffers
 * aligned to elem_bytes, not overlapping; K % 32 == 0; elem_bytes other
 * than 1 or 2 is unsupported; E, N or K == 0 is a no-op.
 */
int64_t w4_repacked_group_elems(int64_t N, int64_t K);
int w4_repack_groups(const void* A, int32_t elem_bytes, int64_t E, int64_t N, int64_t K, void* At,
                     void* stream);
int w4_restore_groups(const void* At, int32_t elem_bytes, int64_t E, int64_t N, int64_t K, void* A,
                      void* stream);

/*
 * w4a16_gemm_tiled -- w4a16_gemm (Z == NULL) or w4a16_gemm_asym (Z given)
 * with the codes, the scales and the zero points in kernel order: Wt from
 * w4_repack, S and Z from w4_repack_groups (E = 1; w4_repacked_group_elems
 * values each).  Same definition, arguments, limits and dispatch; the
 * results equal those of the canonical-layout call bit for bit.
 */
int w4a16_gemm_tiled(const uint16_t* X, const int32_t* Wt, const uint16_t* S,
                     const uint8_t* Z, uint16_t* Y, int64_t M, int64_t N, int64_t K,
                     void* stream);

/*
 * w4a16_moe_gemm_tiled, w4a16_moe_gemm_swiglu_tiled -- the grouped
 * products (symmetric with Z == NULL, zero-point with Z given) with every
 * expert's codes, scales and zero points in kernel order (Wt from w4_repack,
 * S and Z from w4_repack_groups, E experts each).  Definitions, arguments
 * and limits as w4a16_moe_gemm(_asym) and w4a16_moe_gemm_swiglu(_asym);
 * results equal the canonical-layout calls bit for bit.
 */
int w4a16_moe_gemm_tiled(const uint16_t* X, const int32_t* Wt, const uint16_t* S,
                         const uint8_t* Z, const int32_t* sorted_token_ids,
                         const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                         const float* topk_weights, uint16_t* Y, int64_t T, int32_t k,
                         int32_t E, int64_t N, int64_t K, int32_t B, int32_t x_row_div,
                         void* stream);
int w4a16_moe_gemm_swiglu_tiled(const uint16_t* X, const int32_t* Wt, const uint16_t* S,
                                const uint8_t* Z, const int32_t* sorted_token_ids,
                                const int32_t* expert_ids,
                                const int32_t* num_tokens_post_padded, uint16_t* A, int64_t T,
                                int32_t k, int32_t E, int64_t I, int64_t K, int32_t B,
                                int32_t x_row_div, void* stream);

/*
 * w4_dequant_t -- the dequantized weight, transposed ([RL] §2.1: the QAT
 * forward multiplies W' = fake_quant(W); with the straight-through
 * estimator the input gradient is dX = dY W', which w4_bf16_gemm_nt
 * computes from this W'^T):
 *   WT[k, n] = bf16_rne( q[n, k] * S[n, k/32] )            (Z == NULL)
 *   WT[k, n] = bf16_rne( (q[n, k] - Z[n, k/32]) * S[n, k/32] )   (Z given)
 * the values of w4_dequant(_asym), bit for bit.  Wq int32 [N, K/8]
 * (4-byte aligned), S bf16 [N, K/32], Z uint8 [N, K/32] or NULL, WT bf16
 * [K, N] output, 16-byte aligned.  K % 32 == 0; N or K == 0 is a no-op.
 */
int w4_dequant_t(const int32_t* Wq, const uint16_t* S, const uint8_t* Z,
                 int64_t N, int64_t K, uint16_t* WT, void* stream);

/*
 * w4_bf16_gemm_nt -- C = A B^T for bf16 matrices with fp32 accumulation
 * (the QAT input gradient dX = dY W' with A = dY [M, N_w], B = W'^T from
 * w4_dequant_t; [RL] §2.1):
 *   C[m, n] = bf16_rne( sum_k A[m, k] * B[n, k] )    (order fixed)
 * A bf16 [M, K], B bf16 [N, K], both 16-byte aligned; C bf16 [M, N],
 * 2-byte aligned.  K % 8 == 0 (W4_ERR_SHAPE otherwise); K == 0 writes
 * zeros; A and B each below 2 GiB (W4_ERR_UNSUPPORTED otherwise).
 */
int w4_bf16_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M,
                    int64_t N, int64_t K, void* stream);

/*
 * w4_bf16_transpose -- AT = A^T with zero rows appended ([RL] §2.1: the QAT
 * weight gradient dW = dY^T X is w4_bf16_gemm_nt(dY^T, X^T), whose operands
 * need their shared dimension contiguous and a multiple of 8):
 *   AT[c, r] = A[r, c]  (r < R),   AT[c, r] = 0  (R <= r < RP)
 * A bf16 [R, C], AT bf16 [C, RP] output, both 2-byte aligned and not
 * overlapping.  RP >= R (W4_ERR_SHAPE otherwise); C == 0 or RP == 0 is a
 * no-op.  Bit-exact (a copy).
 */
int w4_bf16_transpose(const uint16_t* A, int64_t R, int64_t C, int64_t RP, uint16_t* AT,
                      void* stream);

/*
 * w4_pick_block_size -- alignment block size from the token count and the
 * expert count ([TAG] [35]):  B = min(64, max(16, next_pow2(ceil(T*k/E)))).
 * Returns 0 if T < 0, k < 1 or E < 1.
 */
int32_t w4_pick_block_size(int64_t T, int32_t k, int32_t E);

/*
 * w4_moe_align_capacity -- length of sorted_token_ids that
 * moe_align_block_size fills: round_up(T*k + E*(B-1), B).  Returns -1 on
 * invalid arguments.  expert_ids holds capacity / B entries.
 */
int64_t w4_moe_align_capacity(int64_t T, int32_t k, int32_t E, int32_t B);

/*
 * moe_align_block_size -- merge and align each expert's token set
 * ([RL] §4, [TAG] [35]).
 * topk_ids int32 [T, k] (pair f = t*k + j routes to expert topk_ids[t, j];
 * ids outside [0, E) are skipped).  Outputs, over their whole capacity:
 *   sorted_token_ids int32 [cap]: experts in ascending order; inside an
 *       expert its pairs f in ascending order, then the sentinel T*k up to
 *       a multiple of B; after the last segment, the sentinel.
 *   expert_ids int32 [cap/B]: the expert of each block, -1 past the end.
 *   num_tokens_post_padded int32 [1]: total padded length (multiple of B).
 * 1 <= k, 1 <= E <= 1024, 1 <= B <= 1024, T*k + E*B < 2^31.  T == 0 is
 * valid (all sentinels, total 0).  Bit-exact; deterministic.
 */
int moe_align_block_size(const int32_t* topk_ids, int64_t T, int32_t k,
                         int32_t E, int32_t B, int32_t* sorted_token_ids,
                         int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         void* stream);

/*
 * w4a16_moe_gemm -- grouped W4A16 GEMM over aligned expert blocks
 * ([RL] §4 fused MoE).  For every block b < num_tokens_post_padded / B
 * with e = expert_ids[b] in [0, E), and every slot holding a pair
 * f = sorted_token_ids[b*B + i] < T*k:
 *   Y[f, :] = bf16_rne( X[f / x_row_div, :] * dequant(Wq[e], S[e])^T
 *                       (* topk_weights[f] if topk_weights != NULL) )
 * Rows of Y not named by a valid slot are not written.
 * X   bf16 [rows, K] with rows = (T*k) / x_row_div (x_row_div = k for the
 *     gate_up projection of token rows, 1 for the down projection of pair
 *     rows), 16-byte aligned.
 * Wq  int32 [E, N, K/8], S bf16 [E, N, K/32] (experts stacked), Wq 16-byte
 *     aligned.  Y bf16 [T*k, N], 4-byte aligned.
 * sorted_token_ids / expert_ids / num_tokens_post_padded: as produced by
 * moe_align_block_size with the same T, k, E, B (device memory; the count
 * is read on the device, never by the host).
 * topk_weights float32 [T*k] or NULL.  K % 32 == 0, N >= 1, B in [1, 1024],
 * x_row_div in {1, k}.  X and one expert's Wq each below 2 GiB (32-bit
 * buffer offsets), else W4_ERR_UNSUPPORTED.  Scales below 2^118 (the
 * dequant step overflows beyond).
 */
int w4a16_moe_gemm(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded,
                   const float* topk_weights, uint16_t* Y, int64_t T,
                   int32_t k, int32_t E, int64_t N, int64_t K, int32_t B,
                   int32_t x_row_div, void* stream);

/*
 * w4a16_moe_gemm_swiglu -- the gate_up projection with the SwiGLU of
 * w4_silu_mul fused into its epilogue (one more step of the MoE operator
 * fusion of [RL] §4; the activation is a reading, as for w4_silu_mul).  Wq / S hold
 * 2I weight rows per expert: rows [0, I) gate, [I, 2I) up.  For every
 * valid slot (as in w4a16_moe_gemm, topk weights not applied):
 *   g = bf16_rne(X[f / x_row_div, :] * dequant(W_e[0:I])^T)
 *   u = bf16_rne(X[f / x_row_div, :] * dequant(W_e[I:2I])^T)
 *   A[f, i] = bf16_rne( silu(g[i]) * u[i] )
 * so A equals w4_silu_mul(w4a16_moe_gemm(...)) bit for bit, without the
 * [T*k, 2I] intermediate.  X, Wq, S, the alignment arrays, B and x_row_div
 * as for w4a16_moe_gemm with N = 2I; A bf16 [T*k, I], 4-byte aligned;
 * I >= 1.  Rows of A not named by a valid slot are not written.
 */
int w4a16_moe_gemm_swiglu(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                          const int32_t* sorted_token_ids, const int32_t* expert_ids,
                          const int32_t* num_tokens_post_padded, uint16_t* A, int64_t T,
                          int32_t k, int32_t E, int64_t I, int64_t K, int32_t B,
                          int32_t x_row_div, void* stream);

/*
 * w4a16_moe_gemm_asym, w4a16_moe_gemm_swiglu_asym -- the two grouped
 * products with zero-point experts ([QB] §2.1 inverse map x_hat = (q - z) s,
 * §2.3 asymmetric quantization; [RL] §4 fused MoE):  every dequantized
 * weight is  w'[n, k] = bf16_rne( (q[n, k] - Z[e, n, k/32]) * S[e, n, k/32] )
 * (exact product) with q the unsigned nibbles of Wq[e], as
 * w4_quantize_pack_asym writes them per expert.  Z uint8 [E, N, K/32]
 * (N = 2I for the SwiGLU form), values in [0, 15] (other values: results
 * undefined).  Every other argument, rule and limit as in w4a16_moe_gemm /
 * w4a16_moe_gemm_swiglu; Z == NULL is W4_ERR_NULL.
 */
int w4a16_moe_gemm_asym(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                        const uint8_t* Z, const int32_t* sorted_token_ids,
                        const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                        const float* topk_weights, uint16_t* Y, int64_t T, int32_t k,
                        int32_t E, int64_t N, int64_t K, int32_t B, int32_t x_row_div,
                        void* stream);
int w4a16_moe_gemm_swiglu_asym(const uint16_t* X, const int32_t* Wq, const uint16_t* S,
                               const uint8_t* Z, const int32_t* sorted_token_ids,
                               const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                               uint16_t* A, int64_t T, int32_t k, int32_t E, int64_t I,
                               int64_t K, int32_t B, int32_t x_row_div, void* stream);

/*
 * w4_silu_mul -- SwiGLU between the expert projections (a reading: the
 * pages name the gate_up / down pair but not the activation):
 *   A[r, i] = bf16_rne( silu(H1[r, i]) * H1[r, I + i] ),  silu(v) = v/(1+e^-v)
 * H1 bf16 [R, 2I], A bf16 [R, I], both 4-byte aligned; I even.
 */
int w4_silu_mul(const uint16_t* H1, uint16_t* A, int64_t R, int64_t I,
                void* stream);

/*
 * w4_moe_sum -- top-k combine:
 *   Out[t, :] = bf16_rne( sum_{j = 0..k-1, in order} w[t, j] * H2[t*k + j, :] )
 * in fp32, with w = topk_weights, or w = 1 when topk_weights is NULL.
 * H2 bf16 [T*k, H], Out bf16 [T, H], 4-byte aligned; H even.
 */
int w4_moe_sum(const uint16_t* H2, const float* topk_weights, uint16_t* Out,
               int64_t T, int32_t k, int64_t H, void* stream);

/*
 * w4_moe_route -- softmax top-k routing (fused gating, [RL] §4 / [TAG] [35]):
 *   p = softmax(logits[t, :]); pick the k largest logits (ties: lower
 *   expert index first), ordered by descending logit; weights are the
 *   picked p renormalised to sum to 1 (= softmax over the picked logits).
 * logits float32 [T, E]; topk_ids int32 [T, k]; topk_weights float32 [T, k].
 * 1 <= k <= min(E, 16), 1 <= E <= 1024, T < 2^31.  fp32 arithmetic.
 * -inf logits (masked experts) sort last, by index, and the k ids of a
 * token are always distinct; NaN logits are never picked (a row with fewer
 * than k non-NaN logits gets unspecified ids).
 */
int w4_moe_route(const float* logits, int64_t T, int32_t E, int32_t k,
                 int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * w4_moe_combine_workspace_words -- int32 words of the arrival counters
 * that w4a16_moe_gemm_combine needs for T tokens, top-k, E experts, N
 * output columns and block size B: one per token and weight-row tile of the
 * grouped product (T * ceil(N / 128) or T * ceil(N / 256), as the tile the
 * product picks).  -1 on invalid arguments.
 */
int64_t w4_moe_combine_workspace_words(int64_t T, int32_t k, int32_t E, int64_t N,
                                       int32_t B);

/*
 * w4a16_moe_gemm_combine -- the grouped down product with the top-k
 * combine fused ([RL] §4, deep fusion of the MoE operators; [TAG] [35]).
 * In one launch:
 *   H2 = w4a16_moe_gemm(A, Wq, S, ..., x_row_div = 1, topk_weights = NULL)
 *   Out[t, :] = bf16( sum over j = 0..k-1 in order, fp32 fused multiply-add,
 *                     of topk_weights[t, j] * H2[t*k + j, :] )
 * -- bit for bit what w4a16_moe_gemm followed by w4_moe_sum give.  Pairs
 * whose topk_ids entry lies outside [0, E) take no part in the sum; a token
 * none of whose pairs lies in [0, E) is not written.
 * A bf16 [T*k, K] (the SwiGLU output); Wq / S the experts' codes and scales
 * as w4a16_moe_gemm (tiled == 0) or in the kernel-order layouts of
 * w4_repack / w4_repack_groups (tiled != 0); sorted_token_ids, expert_ids,
 * num_tokens_post_padded from moe_align_block_size over topk_ids int32
 * [T, k]; topk_weights float32 [T, k]; H2 bf16 [T*k, N] (written: the
 * unweighted rows); Out bf16 [T, N].
 * workspace: int32 [w4_moe_combine_workspace_words(T, k, E, N, B)],
 * caller-owned device memory, 4-byte aligned, all zero before the call;
 * the call leaves it all zero.  Each workgroup counts its rows' tokens in
 * once its rows are stored, and the one that completes a token's count
 * writes that token's columns, so the result does not depend
 * on the order in which workgroups run.  Calls that share a workspace must
 * not overlap in time.  The rows of H2 are written and read back with
 * agent-coherent accesses (through the L2 of each XCD), so no cache
 * write-back or invalidate is needed between workgroups.  Limits and errors
 * as w4a16_moe_gemm (symmetric codes), plus k <= 16 (W4_ERR_UNSUPPORTED)
 * and NULL topk_ids / topk_weights / Out / workspace: W4_ERR_NULL.
 */
int w4a16_moe_gemm_combine(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                           const int32_t* sorted_token_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded,
                           const int32_t* topk_ids, const float* topk_weights,
                           uint16_t* H2, uint16_t* Out, int64_t T, int32_t k,
                           int32_t E, int64_t N, int64_t K, int32_t B, int32_t tiled,
                           int32_t* workspace, void* stream);

/*
 * w4a16_moe_gemm_combine_noalloc -- w4a16_moe_gemm_combine without the
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The arrival counters live in a fixed array of the library:
 * 2^18 int32 (1 MiB) per GPU, held until the process ends, zero when the
 * library loads and left zero by every call.  A layer needing more
 * counters than that (w4_moe_combine_workspace_words(T, k, E, N, B) >
 * 262144) returns W4_ERR_UNSUPPORTED with nothing enqueued.  The call
 * allocates nothing and calls no allocating routine; on its first use on a
 * device it looks up that device's copy of the array.  All calls on one GPU
 * share the counters: calls that overlap in time on one GPU (unordered
 * streams, or several host threads) race and give undefined results.
 * Outputs, other limits and errors as w4a16_moe_gemm_combine.
 */
int w4a16_moe_gemm_combine_noalloc(const uint16_t* A, const int32_t* Wq, const uint16_t* S,
                                   const int32_t* sorted_token_ids,
                                   const int32_t* expert_ids,
                                   const int32_t* num_tokens_post_padded,
                                   const int32_t* topk_ids, const float* topk_weights,
                                   uint16_t* H2, uint16_t* Out, int64_t T, int32_t k,
                                   int32_t E, int64_t N, int64_t K, int32_t B,
                                   int32_t tiled, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
