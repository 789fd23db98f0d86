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
 *     allocates nothing, frees nothing and never synchronises.  The
 *     single-pass forwards (attn_fwd, attn_fwd_fp8 and their grouped-query
 *     and variable-length forms) enqueue exactly one kernel on `stream`
 *     (0 = the null stream); attn_fwd_fp8_2pass enqueues two, attn_bwd
 *     three and attn_fp8_quantize four, in order on the same stream.
 *   - Argument errors (ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED) are
 *     detected on the host before any HIP call; nothing is launched then.
 *     ATTN_ERR_HIP reports a failed launch: for a multi-kernel entry point
 *     the kernels enqueued before the failing one stay enqueued and may have
 *     written part of the outputs (or the workspace), which are then
 *     unspecified.  The functions are stateless and thread-safe.
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
#define ATTN_ERR_INVALID_ARG 1 /* null pointer, B/H/N <= 0, H not a multiple of H_kv, causal not 0/1,
                                  non-finite scale, size overflow, inconsistent varlen sizes */
#define ATTN_ERR_UNSUPPORTED 2 /* head_dim not in {64, 128}, pointer not 16-byte aligned (fp32 arrays:
                                  4-byte), H * head_dim > 2^24, grid over 2^31 - 1 work-groups */
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

/*
 * Grouped-query and variable-length forms.  Grouped-query attention (GQA;
 * MQA when H_kv = 1) lets several query heads share one key/value head, and
 * variable-length batches pack sequences of different lengths without
 * padding: "FlashAttention 4: Atenção Mais Rápida e Eficiente em Memória
 * para LLMs", sections "Principais Conclusões" and "Compatibilidade e status
 * atual", where both are listed as missing forward-pass features of the
 * page's kernel.  The arithmetic is that of attn_fwd / attn_fwd_fp8; only
 * which K/V rows a query row sees changes:
 *   - query head h (0 <= h < H) reads K/V head h / (H / H_kv); H must be a
 *     multiple of H_kv (H_kv = H is plain multi-head attention);
 *   - in a variable-length batch every sequence is a separate attention
 *     problem: its queries see only its own keys (and with causal = 1 only
 *     keys 0..i of the same sequence for its query i).
 *
 * attn_fwd_gqa -- bf16, fixed length.
 *   q, o   : bf16 [B][N][H][d];   k, v : bf16 [B][N][H_kv][d];
 *   lse    : fp32 [B][H][N].  Other arguments as for attn_fwd.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int H_kv, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_varlen -- bf16, variable-length batch packed along the token axis.
 *   q, o        : bf16 [total][H][d];   k, v : bf16 [total][H_kv][d];
 *   lse         : fp32 [H][total] (row of query token t of head h at h*total + t);
 *   cu_seqlens  : int32 [B+1], DEVICE, read by the kernel: sequence b owns
 *                 token rows cu_seqlens[b] .. cu_seqlens[b+1]-1; the caller
 *                 guarantees 0 = cu[0] <= cu[1] <= ... <= cu[B] = total and
 *                 cu[b+1] - cu[b] <= max_seqlen.  A sequence whose offsets
 *                 break this (negative, decreasing, past total, longer than
 *                 max_seqlen) is skipped -- its rows of o and lse are not
 *                 written -- and no memory outside the tensors is touched.
 *                 Empty sequences are allowed.
 *   B           : number of sequences, >= 1;
 *   total       : token rows in the packed tensors, >= 0 (0: nothing is
 *                 launched, the tensor pointers are not checked);
 *   max_seqlen  : an upper bound on the sequence lengths, 1 <= max_seqlen <=
 *                 total; the grid is sized from it.
 *   H, H_kv, d, causal, scale, stream : as for attn_fwd_gqa.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int B, int total, int max_seqlen, int H, int H_kv,
                    int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fwd_fp8_gqa -- OCP FP8 E4M3 form of attn_fwd_gqa.
 *   q : e4m3fn [B][N][H][d];  k, v : e4m3fn [B][N][H_kv][d];  o : bf16; lse : fp32 [B][H][N].
 *   descale_q : fp32 [B*H] (index b*H + h);
 *   descale_k, descale_v : fp32 [B*H_kv] (index b*H_kv + hk), device.
 */
int attn_fwd_fp8_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                     const float* descale_q, const float* descale_k, const float* descale_v,
                     int B, int H, int H_kv, int N, int d, int causal, float scale,
                     hipStream_t stream);

/*
 * attn_fwd_fp8_2pass -- attn_fwd_fp8_gqa in the two-pass form of
 * "FlashAttention-3: Pipeline Assíncrono com Warp Specialization, WGMMA e
 * FP8 no Hopper e Blackwell", section "Estabilidade em FP8: Algoritmo de 2
 * Passos e Incoherent Processing": a first pass computes every row's exact
 * maximum score (fp32 accumulation of the e4m3 products) and stores it in
 * lse; a second pass exponentiates against that fixed maximum and
 * multiplies by V with a static scale on P (p' = 2^8 p, rounded to e4m3),
 * with no running maximum and no rescale.  Same arguments, layouts,
 * results (o, lse) and errors as attn_fwd_fp8_gqa; lse also carries the
 * row maxima between the two kernels, which are enqueued on `stream` in
 * order.  It costs about one and a half times the single pass.
 */
int attn_fwd_fp8_2pass(const void* q, const void* k, const void* v, void* o, float* lse,
                       const float* descale_q, const float* descale_k, const float* descale_v,
                       int B, int H, int H_kv, int N, int d, int causal, float scale,
                       hipStream_t stream);

/*
 * attn_fwd_fp8_varlen -- OCP FP8 E4M3 form of attn_fwd_varlen.
 *   q : e4m3fn [total][H][d];  k, v : e4m3fn [total][H_kv][d];  o : bf16 [total][H][d];
 *   lse : fp32 [H][total];  descales per (sequence b, head) as for attn_fwd_fp8_gqa.
 */
int attn_fwd_fp8_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* descale_q, const float* descale_k, const float* descale_v,
                        const int* cu_seqlens, int B, int total, int max_seqlen, int H, int H_kv,
                        int d, int causal, float scale, hipStream_t stream);

/*
 * attn_bwd -- bfloat16 backward pass: the gradients of attn_fwd's output O
 * with respect to q, k and v, given the upstream gradient dO.  The backward
 * pass is named as the forward kernel's counterpart (needed for training) by
 * "FlashAttention 4: Atenção Mais Rápida e Eficiente em Memória para LLMs",
 * section "Principais Conclusões", and "FlashAttention-4 no Blackwell B200
 * ...", section "Redução de tráfego no backward".  With P = softmax(scale
 * Q K^T) (masked as in the forward):
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 * P is recomputed tile by tile from lse; no N x N matrix reaches HBM.
 *   q, k, v, o, dout : bf16 [B][N][H][d], device, read only; o and lse are
 *                      the outputs of attn_fwd for the same q, k, v, causal
 *                      and scale.
 *   lse              : fp32 [B][H][N], device, read only.
 *   dq, dk, dv       : bf16 [B][N][H][d], device, written.
 *   delta            : fp32 [B][H][N], device, caller-owned workspace (the
 *                      library allocates nothing); written with D.
 *   B, H, N, d, causal, scale, stream : as for attn_fwd.
 * Three kernels are enqueued on `stream` in order: D, dQ, then dK and dV;
 * the results are deterministic (no atomics).  Errors as for attn_fwd; null
 * dout/dq/dk/dv/delta is ATTN_ERR_INVALID_ARG.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* delta,
             int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * attn_fp8_quantize -- bfloat16 attention input -> OCP FP8 E4M3 codes and a
 * per-(batch, head) descale, the input format of the FP8 entry points, with
 * the optional random Hadamard rotation of "FlashAttention-3: Pipeline
 * Assíncrono com Warp Specialization, WGMMA e FP8 no Hopper e Blackwell",
 * section "Estabilidade em FP8: Algoritmo de 2 Passos e Incoherent
 * Processing" (incoherent processing: a random orthogonal Hadamard matrix
 * spreads outliers over all dimensions).  With M = diag(s) H_d / sqrt(d)
 * (s the random signs, H_d the Sylvester Hadamard matrix), rotating Q and K
 * with the same signs leaves Q K^T unchanged; V is quantised unrotated.
 *   x         : bf16 [B][N][H][d], device, read only, finite values.
 *   codes     : e4m3fn [B][N][H][d], device, written (its first
 *               4 * B * H * ceil(N / 128) bytes hold per-work-group partial
 *               maxima until the codes overwrite them).
 *   descale   : fp32 [B][H], device, written (also used as the per-head
 *               maximum while the call runs).
 *   sign_bits : device, d/32 words, bit i of the words = sign of column i
 *               (1: negate); NULL = no rotation.
 * Per (b, h): y = x diag(s) H_d (binary32 fast Walsh-Hadamard butterfly,
 * strides 1, 2, ..., d/2) or y = x; amax = max |y|; ds = amax / 448;
 * code = e4m3(clamp(y / ds, +-448)) rounded to nearest even (ds = 0 divides
 * by 1); descale = ds, or ds / sqrt(d) rounded to binary32 with the
 * rotation, so that code * descale approximates x M.  Every decision is
 * taken in binary32 and the codes are bit-reproducible.
 * d is 64 or 128.  Four kernels are enqueued on `stream`; calls that share
 * descale must not overlap.  Errors: null x/codes/descale, B, N or H <= 0:
 * ATTN_ERR_INVALID_ARG; other d, x or codes not 16-byte aligned, descale or
 * sign_bits not 4-byte aligned, more than 2^31 - 1 work-groups:
 * ATTN_ERR_UNSUPPORTED; a launch failure: ATTN_ERR_HIP.
 */
int attn_fp8_quantize(const void* x, void* codes, float* descale, const unsigned* sign_bits,
                      int B, int N, int H, int d, hipStream_t stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and results, with the D workspace
 * in a static device array of the library instead of a caller's `delta`.
 *   Arguments as for attn_bwd, without `delta`.
 *   Limit: B * H * N <= ATTN_BWD_NOALLOC_MAX_ROWS (16 MiB of fp32 rows per
 *   GPU, held from the library's load until the process ends); larger calls
 *   return ATTN_ERR_UNSUPPORTED and launch nothing.
 *   `stream` must belong to the current device (else ATTN_ERR_INVALID_ARG).
 *   The first call on a device looks the array's device address up
 *   (hipGetSymbolAddress); no call allocates or frees memory.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams or host threads) race and must be serialised by
 *   the caller.  Nothing in the array needs to start at zero (each call
 *   writes every row it reads before reading it).
 *   Errors: null pointers, B/H/N <= 0 -> ATTN_ERR_INVALID_ARG; the limit ->
 *   ATTN_ERR_UNSUPPORTED (both before any HIP call); the rest as attn_bwd.
 */
#define ATTN_BWD_NOALLOC_MAX_ROWS (1 << 22)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv,
                     int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/* Static, human-readable name of a status code ("ATTN_OK", ...). */
const char* attn_status_string(int status);

/* Library version string (static). */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
