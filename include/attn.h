/*
 * attn.h -- C ABI of the MI355X (gfx950) tiled exact attention forward.
 *
 * The operation (cited from the public pages this library implements):
 *   O = softmax(Q K^T * scale) V, computed tile by tile with an online
 *   softmax (running row maximum and row sum, rescaling of the output
 *   accumulator) so that the N x N score matrix never reaches HBM, plus the
 *   per-row log-sum-exp of the scaled scores.
 *   - operation: "FlashAttention-4 no Blackwell B200: pipelining de kernels
 *     e o que FP4 realmente muda", section "Por que o Blackwell exige mais do
 *     que multiplicações rápidas"; exactness: dev.to "FlashAttention-4 em
 *     Blackwell B200", section 6 (FAQ, question 2);
 *   - tiling and online softmax: same dev.to page, section 1 and the
 *     simulator of section 4; "FlashAttention 4: Atenção Mais Rápida e
 *     Eficiente em Memória para LLMs", sections "Introdução" and
 *     "Reescalonamento Softmax Online Mais Inteligente" (threshold-gated
 *     rescale);
 *   - argument convention (bfloat16 [batch][seq][heads][head_dim] tensors,
 *     softmax_scale, causal flag, no dropout): "FlashAttention-3: Pipeline
 *     Assíncrono com Warp Specialization, WGMMA e FP8 no Hopper e
 *     Blackwell", section "Implementando FlashAttention-3 em produção";
 *   - FP8 E4M3 operands with fp32 accumulation: same page, section
 *     "Estabilidade em FP8: Algoritmo de 2 Passos e Incoherent Processing".
 *
 * Definition, per batch b, head h and query row i (j runs over the visible
 * keys: all j, or j <= i when causal):
 *   s_ij  = scale * sum_c q[b][i][h][c] * k[b][j][h][c]
 *   o[b][i][h][:] = sum_j exp(s_ij - m_i) v[b][j][h][:] / sum_j exp(s_ij - m_i),
 *                   m_i = max_j s_ij
 *   lse[b][h][i]  = ln sum_j exp(s_ij)       (natural logarithm)
 *
 * Conventions shared by every entry point
 *   - Layout: q, k, v, o are contiguous row-major [B][N][H][d]; lse is
 *     contiguous fp32 [B][H][N].  Query and key sequences have the same
 *     length N (square attention); with causal = 1 query i sees keys 0..i.
 *   - Any N >= 1 is accepted; ragged tails are masked, never truncated.
 *   - Pointers are DEVICE pointers owned by the caller, who keeps them alive
 *     until the work queued on `stream` has completed.  The library
 *     allocates nothing, frees nothing and never synchronises; each call
 *     only enqueues one kernel on `stream` (0 = the null stream).
 *   - Errors are detected on the host before any HIP call; nothing is
 *     launched when a call returns an error.  The functions are stateless
 *     and thread-safe.
 *   - Inputs must be finite; results for inf/NaN inputs are unspecified.
 *   - o must not alias q, k or v.
 */
#ifndef ATTN_H
#define ATTN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG 1 /* null pointer, B/H/N <= 0, causal not 0/1, non-finite scale, size overflow */
#define ATTN_ERR_UNSUPPORTED 2 /* head_dim not in {64, 128}, pointer not 16-byte aligned */
#define ATTN_ERR_HIP 3         /* the HIP runtime reported an error at launch */

/*
 * attn_fwd -- bfloat16 attention forward.
 *   q, k, v : bf16 [B][N][H][d], device, read only.
 *   o       : bf16 [B][N][H][d], device, written (round-to-nearest-even).
 *   lse     : fp32 [B][H][N], device, written.
 *   B, H, N : batch, heads, sequence length, each >= 1.
 *   d       : head dimension, 64 or 128.
 *   causal  : 0 = every key visible, 1 = key j visible to query i iff j <= i.
 *   scale   : multiplies Q K^T (finite; 1/sqrt(d) in the usual case).
 *   stream  : HIP stream to enqueue on.
 * Arithmetic: bf16 MFMA products with fp32 accumulation; softmax in fp32
 * with base-2 exponentials (log2(e) folded into the scale); probabilities
 * rounded to bf16 for the P.V product.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_fp8 -- OCP FP8 E4M3 ("e4m3fn", max 448) attention forward.
 *   q, k, v   : e4m3fn codes [B][N][H][d], device, read only.  The real
 *               input value is code * descale[b*H + h].
 *   o         : bf16 [B][N][H][d], device, written.
 *   lse       : fp32 [B][H][N], device, written (of the dequantised scores).
 *   descale_q, descale_k, descale_v : fp32 [B*H], device, one factor per
 *               (batch, head), read by the kernel (never by the host).
 *   B, H, N, d, causal, scale, stream : as for attn_fwd.
 * Arithmetic: e4m3 MFMA products with fp32 accumulation; the descales are
 * folded into the score scale and the output normalisation; probabilities
 * are rounded to e4m3 for the P.V product.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 const float* descale_q, const float* descale_k, const float* descale_v,
                 int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/* Static, human-readable name of a status code ("ATTN_OK", ...). */
const char* attn_status_string(int status);

/* Library version string (static). */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
