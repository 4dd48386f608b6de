/*
 * fa.h - C ABI of an MI355X (gfx950) exact-attention library: fused forward, backward by
 * recomputation, and split-KV decoding, for bfloat16 tensors on one GPU.
 *
 * What is computed (page "Bellek Duvarının Fiziği: Standart Attention'dan FlashAttention'a",
 * section "Attention'ın Cebiri"; notation of "FlashAttention'ı Anlamak Bölüm 1", section 0.2):
 *     S = scale * Q K^T + M,   P = row-softmax(S),   O = P V,
 * with M_ij = 0 where key j is visible to query i and -inf elsewhere. Without `causal` every key
 * is visible. With `causal`, key j is visible to query i iff j <= i + (N_k - N_q): the page's
 * "query i sees keys j <= i" (section "Maskeleme ve Dropout"), aligned so that the queries are
 * the last N_q positions of the key sequence when N_q < N_k.
 *
 * Layout. Every tensor is a device pointer to a contiguous row-major array:
 *     q, o, dout, dq      [B, H, N_q, d]   bf16
 *     k, v, dk, dv        [B, H, N_k, d]   bf16
 *     lse                 [B, H, N_q]      fp32, natural log: lse_i = ln sum_j exp(S_ij)
 * bf16 values are passed as their 16-bit patterns (fa_bf16). V, O, dO and dV share d with Q
 * and K everywhere except the fa_fwd_dv / fa_bwd_dv entry points, which give them a width d_v
 * of their own; K and V have H_kv heads instead of H in the grouped-query entry points; the
 * entry points with an additive bias, per-sequence lengths, dropout or FP8 say what they add.
 *
 * Ownership. The caller owns every buffer. The library never allocates, frees or synchronises
 * and keeps no mutable global state, so calls are reentrant (the one exception, a per-GPU
 * device array used by fa_decode_noalloc, is described there). Inputs are read only; outputs
 * are fully overwritten; outputs must not alias inputs or each other.
 *
 * Streams. Every call only enqueues kernels on `stream` (0 = the null stream) and returns.
 *
 * Errors. All arguments are validated before anything is enqueued; on any error nothing is
 * enqueued and no output is touched. A failed launch returns FA_ERR_HIP. Faults during kernel
 * execution surface at the caller's next synchronisation of the stream.
 *
 * Common constraints: B, H, N_q, N_k >= 1; d in {64, 128}; B*H*N_q and B*H*N_k below 2^31;
 * one head's rows of any tensor below 2^31 bytes (the kernels address a head through 32-bit
 * buffer offsets); pointers 16-byte aligned; scale finite and > 0; causal requires N_q <= N_k
 * (so no row is empty). A violation returns FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_ALIGN,
 * FA_ERR_SCALE or FA_ERR_CAUSAL before anything is enqueued.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t fa_bf16; /* bfloat16 bit pattern */

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,     /* a size < 1, or an index range too large */
  FA_ERR_HEADDIM = 3,   /* d not in {64, 128} */
  FA_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  FA_ERR_CAUSAL = 5,    /* causal with N_q > N_k */
  FA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than the queried size */
  FA_ERR_SCALE = 7,     /* scale not finite or not > 0 */
  FA_ERR_ARG = 8,       /* another argument out of range (decode: N_q != 1, bad split count) */
  FA_ERR_HIP = 9        /* a kernel launch failed */
} fa_status;

/* Human-readable name of a status code; never NULL. */
const char* fa_status_string(fa_status s);

/*
 * Forward pass: O and the per-row log-sum-exp L.
 * Page "Bellek Duvarının Fiziği", sections "Online Softmax" and "Forward geçişin iskeleti":
 * Q is split into row blocks, K/V are streamed block by block through on-chip memory, the row
 * maximum and sum are kept as running statistics, and the N_q x N_k score and probability
 * matrices are never written to HBM. Section "Geri Yayılım": L is the one statistic per row that
 * the backward pass needs to rebuild P.
 *   q [B,H,N_q,d], k/v [B,H,N_k,d] in; o [B,H,N_q,d] bf16 and lse [B,H,N_q] fp32 out.
 */
fa_status fa_fwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                 int B, int H, int N_q, int N_k, int d, float scale, int causal,
                 hipStream_t stream);

/* Bytes of device workspace fa_bwd needs: two fp32 row vectors [B, H, N_q], D = rowsum(dO * O)
 * and the log-sum-exp in base-2 units, each padded to 16 bytes. */
size_t fa_bwd_workspace_bytes(int B, int H, int N_q, int N_k, int d);

/*
 * Backward pass by recomputation: gradients of O with respect to Q, K, V given dO.
 * Page "Bellek Duvarının Fiziği", section "Geri Yayılım": P is rebuilt block by block as
 * exp(S - L) from the stored L, D = rowsum(dO * O) is taken from the forward output, and the
 * softmax gradient identity dS = P * (dP - D) gives dQ = scale dS K, dK = scale dS^T Q,
 * dV = P^T dO.
 *   q, k, v, o (forward output), lse (forward output), dout = dO in;
 *   dq [B,H,N_q,d], dk, dv [B,H,N_k,d] bf16 out.
 *   workspace: device memory of at least fa_bwd_workspace_bytes(...) bytes, 16-byte aligned,
 *   owned by the caller, clobbered by the call.
 */
fa_status fa_bwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                 const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int H, int N_q, int N_k, int d, float scale, int causal,
                 hipStream_t stream);

/*
 * The three phases fa_bwd runs, exposed so that a caller can schedule or time them separately.
 * Same layouts, workspace and validation as fa_bwd; they must run in this order on one stream,
 * since the later two read what the first writes into the workspace:
 *   fa_bwd_preprocess: D = rowsum(dO * O) ("Geri Yayılım": D is taken from the forward output)
 *                      and lse / scale, both negated, into the workspace; uses o, lse, dout;
 *   fa_bwd_dkdv:       dK and dV; uses q, k, v, dout and the workspace;
 *   fa_bwd_dq:         dQ; uses q, k, v, dout and the workspace.
 */
fa_status fa_bwd_preprocess(const fa_bf16* o, const float* lse, const fa_bf16* dout,
                            void* workspace, size_t workspace_bytes, int B, int H, int N_q,
                            int N_k, int d, hipStream_t stream);
fa_status fa_bwd_dkdv(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v,
                      const fa_bf16* dout, fa_bf16* dk, fa_bf16* dv, void* workspace,
                      size_t workspace_bytes, int B, int H, int N_q, int N_k, int d, float scale,
                      int causal, hipStream_t stream);
fa_status fa_bwd_dq(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* dout,
                    fa_bf16* dq, void* workspace, size_t workspace_bytes, int B, int H, int N_q,
                    int N_k, int d, float scale, int causal, hipStream_t stream);

/* ---- V with its own head dimension -------------------------------------------------------------
 *
 * "FlashAttention'ı Anlamak Bölüm 1", notation 0.2: V in R^{N_k x d_v}, so O in R^{N_q x d_v},
 * while Q, K have d columns. Layouts as for fa_fwd / fa_bwd with d_v columns for v, o, dout and
 * dv: v, dv [B,H,N_k,d_v], o, dout [B,H,N_q,d_v]. d, d_v in {64, 128} (else FA_ERR_HEADDIM);
 * d_v = d is the same as fa_fwd / fa_bwd. The backward's workspace is fa_bwd_workspace_bytes.
 */
fa_status fa_fwd_dv(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                    int B, int H, int N_q, int N_k, int d, int d_v, float scale, int causal,
                    hipStream_t stream);
fa_status fa_bwd_dv(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                    const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k, int d,
                    int d_v, float scale, int causal, hipStream_t stream);

/* ---- Grouped query heads in the forward and backward passes ------------------------------------
 *
 * Page "Bellek Duvarının Fiziği", section "Duvarın Ötesi: KV Cache, Uzun Bağlam ve Yaklaşık
 * Attention" names query heads that share key/value heads (GQA/MQA) without defining them; the
 * definition used here is the decode's (below): H query heads, H_kv key/value heads, H a multiple
 * of H_kv (else FA_ERR_ARG), query head h attends with key/value head h / (H / H_kv). Layouts as
 * for fa_fwd / fa_bwd except k, v, dk, dv [B,H_kv,N_k,d]; dk and dv of a key/value head are the
 * sums of the gradients its H / H_kv query heads send to it, formed in a fixed order without
 * atomics (a dK/dV workgroup of a key/value head visits its query heads in turn).
 * H_kv = H is fa_fwd / fa_bwd. When the K/V heads times the 128-key tiles are too few to fill
 * the GPU (fewer than 2048), the dK/dV pass runs one workgroup per query head instead and keeps
 * fp32 partial rows in the workspace that a second kernel sums over each group, in head order;
 * fa_bwd_gqa_workspace_bytes (0 for invalid sizes) covers both cases.
 */
size_t fa_bwd_gqa_workspace_bytes(int B, int H, int H_kv, int N_q, int N_k, int d);
fa_status fa_fwd_gqa(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                     int B, int H, int H_kv, int N_q, int N_k, int d, float scale, int causal,
                     hipStream_t stream);
fa_status fa_bwd_gqa(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                     const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                     void* workspace, size_t workspace_bytes, int B, int H, int H_kv, int N_q,
                     int N_k, int d, float scale, int causal, hipStream_t stream);

/* ---- Additive bias on the scores --------------------------------------------------------------
 *
 * "FlashAttention'ı Anlamak Bölüm 1", notation 0.2: S = Q K^T / sqrt(d) + B with B an optional
 * mask or bias. Here S = scale Q K^T + bias (the bias is not multiplied by the scale), on top of
 * the causal mask when causal != 0. bias: bf16, element (b, h, i, j) at
 * bias[b bias_stride_b + h bias_stride_h + i bias_stride_q + j] (strides in elements, >= 0,
 * multiples of 8; 0 broadcasts, e.g. one [N_q, N_k] bias for all batches and heads, or a
 * per-key bias with bias_stride_q = 0); 16-byte aligned; entries finite or -inf (a mask). A row
 * whose scores are all -inf gets o = 0, lse = -inf and zero dq. The backward treats the bias as
 * a constant (no gradient is formed for it). Errors as for fa_fwd / fa_bwd, plus FA_ERR_ARG for
 * negative or unaligned strides and FA_ERR_SHAPE if one head's bias spans 2^30 elements or more.
 */
fa_status fa_fwd_bias(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                      float* lse, const fa_bf16* bias, int64_t bias_stride_b,
                      int64_t bias_stride_h, int64_t bias_stride_q, int B, int H, int N_q, int N_k,
                      int d, float scale, int causal, hipStream_t stream);
fa_status fa_bwd_bias(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                      const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                      fa_bf16* dv, const fa_bf16* bias, int64_t bias_stride_b,
                      int64_t bias_stride_h, int64_t bias_stride_q, void* workspace,
                      size_t workspace_bytes, int B, int H, int N_q, int N_k, int d, float scale,
                      int causal, hipStream_t stream);

/* ---- FP8 forward with incoherent processing ---------------------------------------------------
 *
 * Page "FlashAttention-3 (TR)", on using FP8 while reducing the quantization error: Q and K are
 * multiplied by a random orthogonal matrix (random signs times a Hadamard matrix), which spreads
 * outlier coordinates and leaves Q K^T unchanged, then quantized to FP8; the FlashAttention-3
 * paragraph of "Bellek Duvarının Fiziği" adds block-wise scaling. Here:
 *   - M = diag(sigma) H_d / sqrt(d) (H_d Sylvester-Hadamard); sigma_i = -1 iff bit i of the
 *     Philox-4x32-10 output for counter (0, 0, 0, 0) and key (seed mod 2^32, seed div 2^32) is
 *     set (bit i mod 32 of word i div 32). incoherent = 0 skips the rotation (plain FP8).
 *   - FP8 = OCP E4M3 (largest finite 448). Scales: Q per 32 rows, K per 64 rows, V per head,
 *     scale = max|x| / 448 (1 if all zero), code = E4M3(clamp(x / scale, -448, 448)), rounded to
 *     nearest even, all in fp32 (the rotation by the fast Walsh-Hadamard butterfly, spans 1, 2,
 *     4, ..., d/2, then times 1/sqrt(d) rounded to fp32).
 *   - S = scale (dequantized Q)(dequantized K)^T on FP8 matrix cores; P = exp(S - m) quantized as
 *     E4M3(2^8 P) for the P V product on FP8 matrix cores, m the running row maximum (moved
 *     whenever a score exceeds it by more than 0.5 in log2 units); o = sum P^ V^ / sum P, bf16;
 *     lse = ln sum exp(S) of the dequantized scores, fp32.
 * Inputs q, k, v are bf16 as for fa_fwd (d in {64, 128}); causal needs N_q <= N_k.
 * workspace: device, 16-byte aligned, at least fa_fwd_fp8_workspace_bytes(); after the call it
 * holds, at 256-byte aligned offsets in this order: the E4M3 codes of Q [B,H,N_q,d] and of K
 * [B,H,N_k,d] (after the rotation), of V transposed [B,H,d,N_kp] (N_kp = N_k rounded up to a
 * multiple of 64, padding zero), the fp32 scales of Q [B,H,ceil(N_q/32)] and of K
 * [B,H,ceil(N_k/64)], the per-64-key maxima of |V| [B,H,ceil(N_k/64)] and the V scales [B,H].
 * Errors as for fa_fwd, plus FA_ERR_WORKSPACE.
 */
size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N_q, int N_k, int d);
fa_status fa_fwd_fp8(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                     float* lse, int B, int H, int N_q, int N_k, int d, float scale, int causal,
                     int incoherent, uint64_t seed, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* ---- Dropout on the attention probabilities ---------------------------------------------------
 *
 * [MW] "Maskeleme ve Dropout": dropout acts on P; since P is never stored, neither is the mask:
 * the kernels regenerate it from a seed and an offset, in the forward and again in the backward.
 * Output: o = (P * Z / (1 - p_drop)) V, with P the softmax of fa_fwd and Z the keep mask; lse is
 * that of the scores (the softmax is normalised before dropout), as fa_fwd writes it.
 * The mask: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key (seed mod 2^32,
 * seed div 2^32); the call with counter (j / 8, i, b*H + h, offset) yields eight 16-bit numbers
 * for keys 8 (j/8) .. 8 (j/8) + 7 of query row i (key j: output word (j mod 8) / 2, low half for
 * even j); (i, j) is kept iff its number is below t = floor((1 - p_drop) 65536) (double
 * precision). p_drop in [0, 1) (else FA_ERR_ARG); p_drop = 0 is exactly fa_fwd / fa_bwd.
 * Callers give each dropout layer and step its own (seed, offset) pair, and pass the forward's
 * pair to the backward. Other arguments and errors as for fa_fwd / fa_bwd.
 */
fa_status fa_fwd_dropout(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                         float* lse, int B, int H, int N_q, int N_k, int d, float scale,
                         int causal, float p_drop, uint64_t seed, uint32_t offset,
                         hipStream_t stream);
fa_status fa_bwd_dropout(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                         const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                         fa_bf16* dv, void* workspace, size_t workspace_bytes, int B, int H,
                         int N_q, int N_k, int d, float scale, int causal, float p_drop,
                         uint64_t seed, uint32_t offset, hipStream_t stream);

/* ---- Variable-length batches ------------------------------------------------------------------
 *
 * Batches whose sequences have different lengths, kept in the padded layouts above: sequence b
 * uses its first seq_lens_q[b] query rows and first seq_lens_k[b] key rows of the [B, H, N_q, d]
 * and [B, H, N_k, d] tensors (device int32 arrays [B]; values are clamped to [0, N_q] and
 * [0, N_k]). The pages do not define batching ([MW] "Attention'ın Cebiri" defines one sequence);
 * each sequence here is that definition on its own lengths, with the causal alignment of the
 * "Maskeleme ve Dropout" reading applied per sequence: key j visible to query i iff
 * j <= i + seq_lens_k[b] - seq_lens_q[b]. A query row past its sequence's length, or one that
 * sees no key (causal with seq_lens_q[b] > seq_lens_k[b]), gets o = 0 and lse = -inf; the
 * backward gives zero gradients for padding rows and keys and for rows that see no key.
 * Rows and keys past a sequence's lengths are never read, so the padding may hold any bit
 * pattern (NaN included). Because the lengths live on the device, causal is accepted for any
 * N_q, N_k.
 * seq_lens_q, seq_lens_k: 4-byte aligned; other arguments as for fa_fwd / fa_bwd (the backward
 * uses the same workspace size, fa_bwd_workspace_bytes).
 */
fa_status fa_fwd_varlen(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                        float* lse, const int32_t* seq_lens_q, const int32_t* seq_lens_k,
                        int B, int H, int N_q, int N_k, int d, float scale, int causal,
                        hipStream_t stream);
fa_status fa_bwd_varlen(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                        const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk,
                        fa_bf16* dv, const int32_t* seq_lens_q, const int32_t* seq_lens_k,
                        void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k,
                        int d, float scale, int causal, hipStream_t stream);

/* ---- Variable lengths, grouped K/V heads and dropout, together -------------------------------
 *
 * One call with any subset of three options, each meaning what its own entry point above
 * documents (the training step of a batch of packed sequences needs all three at once, [MW]
 * "Maskeleme ve Dropout" and "Duvarın Ötesi: KV Cache, Uzun Bağlam ve Yaklaşık Attention"):
 *   seq_lens_q, seq_lens_k  per-sequence lengths in the padded layout, as fa_fwd_varlen (device
 *                           int32 [B], 4-byte aligned); both NULL: every sequence is N_q x N_k
 *                           (one NULL and not the other: FA_ERR_ARG);
 *   H_kv                    key/value heads, as fa_fwd_gqa: k, v, dk, dv [B, H_kv, N_k, d], H a
 *                           multiple of H_kv (else FA_ERR_ARG); H_kv = H: one per query head;
 *   p_drop, seed, offset    dropout on P, as fa_fwd_dropout; p_drop = 0: none. The keep mask of
 *                           (i, j) is drawn for query head b H + h and the row and key indices of
 *                           the padded layout, which are the sequence's own indices.
 * Without lengths causal needs N_q <= N_k (FA_ERR_CAUSAL); with them any N_q, N_k. The backward
 * needs the forward's (seq_lens, H_kv, p_drop, seed, offset) and a workspace of at least
 * fa_bwd_ext_workspace_bytes(B, H, H_kv, N_q, N_k, d) bytes (0 for invalid sizes); with grouped
 * K/V heads this includes the fp32 partial rows of fa_bwd_gqa's small-grid mode, which the dK/dV
 * pass also uses whenever lengths are given (a workgroup per whole group would make the longest
 * sequences' workgroups set the time). A bias and d_v != d are not among the options. Other
 * arguments and errors as for fa_fwd / fa_bwd.
 */
fa_status fa_fwd_ext(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                     const int32_t* seq_lens_q, const int32_t* seq_lens_k, int B, int H, int H_kv,
                     int N_q, int N_k, int d, float scale, int causal, float p_drop,
                     uint64_t seed, uint32_t offset, hipStream_t stream);
size_t fa_bwd_ext_workspace_bytes(int B, int H, int H_kv, int N_q, int N_k, int d);
fa_status fa_bwd_ext(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                     const float* lse, const fa_bf16* dout, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                     const int32_t* seq_lens_q, const int32_t* seq_lens_k, void* workspace,
                     size_t workspace_bytes, int B, int H, int H_kv, int N_q, int N_k, int d,
                     float scale, int causal, float p_drop, uint64_t seed, uint32_t offset,
                     hipStream_t stream);

/* The split count fa_decode uses when called with num_splits = 0. */
int fa_decode_num_splits(int B, int H, int N_k, int d);

/* Bytes of device workspace fa_decode needs for a split count (0 = the automatic choice):
 * per (b, h, split) one fp32 partial output row of d values and one fp32 log-sum-exp. */
size_t fa_decode_workspace_bytes(int B, int H, int N_k, int d, int num_splits);

/*
 * Decode step (Flash-Decoding): one query row per (b, h) against a long KV cache.
 * Page "Bellek Duvarının Fiziği", section "Decode Aşaması: Flash-Decoding": the keys are split
 * into C chunks processed in parallel, each producing its own local (max, sum, output) triple,
 * and one reduction merges them with the online-softmax rescaling identity.
 *   q [B,H,1,d], k/v [B,H,N_k,d] in; o [B,H,1,d] bf16 and lse [B,H,1] fp32 out.
 *   N_q must be 1. With one query row the bottom-right causal mask hides nothing, so `causal`
 *   is accepted and changes nothing. num_splits: 0 = automatic, else 1..min(N_k, 1024).
 *   workspace: at least fa_decode_workspace_bytes(B, H, N_k, d, num_splits) bytes, 16-byte
 *   aligned, owned by the caller, clobbered by the call.
 */
fa_status fa_decode(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int N_q, int N_k, int d, float scale, int causal,
                    int num_splits, hipStream_t stream);

/* ---- Decode without allocation ----------------------------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. fa_decode_noalloc is fa_decode (same arguments except
 * the workspace, same kernels, same results bit for bit at the same split count) with the
 * per-split partials in a device array that the library holds, one per GPU, until the process
 * ends: FA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB). A call whose fa_decode_workspace_bytes(B, H,
 * N_k, d, splits) exceeds it returns FA_ERR_WORKSPACE before anything is enqueued (pass a smaller
 * num_splits, or use fa_decode). The call allocates nothing; its first call on a device looks up
 * that device's array (FA_ERR_HIP if that fails), on the device that runs `stream`.
 * Calls on one GPU share its array, which keeps the last call's partials: calls ordered on one
 * stream are fine, calls that may overlap in time on one GPU (other streams, other threads)
 * race and give undefined results.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fa_status fa_decode_noalloc(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                            float* lse, int B, int H, int N_q, int N_k, int d, float scale,
                            int causal, int num_splits, hipStream_t stream);

/* ---- Decode with grouped-query heads, over a paged or a contiguous KV cache --------------------
 *
 * Page "Bellek Duvarının Fiziği", section "Duvarın Ötesi: KV Cache, Uzun Bağlam ve Yaklaşık
 * Attention": at inference the KV cache is the second IO front, attacked by a paged cache
 * (PagedAttention) and by query heads that share K/V heads (GQA/MQA); section "Decode Aşaması:
 * Flash-Decoding" pairs Flash-Decoding with the paged cache. The pages name these methods without
 * defining them; the definitions used here:
 *   * grouped query heads: H query heads, H_kv key/value heads, H a multiple of H_kv; query head
 *     h attends with key/value head h / (H / H_kv) (H_kv = H: multi-head, H_kv = 1: multi-query);
 *   * paged cache: K and V live in fixed-size blocks of block_size positions,
 *       k_cache, v_cache   [num_blocks, H_kv, block_size, d]   bf16
 *     and sequence b's position j sits in block block_table[b, j / block_size] at row
 *     j % block_size;
 *       block_table        [B, max_blocks_per_seq]  int32, entries in [0, num_blocks)
 *       seq_lens           [B]                      int32, 1 <= seq_lens[b] <= max_blocks_per_seq * block_size
 *   * each (b, h) computes O = softmax(scale * q K_b^T) V_b over its seq_lens[b] positions, with
 *       q, o   [B, H, d] bf16 (one query row per head),   lse [B, H] fp32 (natural log).
 * Device-side arguments (block table entries, sequence lengths) cannot be validated before the
 * launch: block ids outside [0, num_blocks) read as zero rows, lengths are clamped to
 * [0, max_blocks_per_seq * block_size], and a row with no position gets o = 0, lse = -inf.
 * block_size must be a power of two (1 .. 4096).
 */

/* The split count fa_decode_gqa uses when called with num_splits = 0. */
int fa_decode_gqa_num_splits(int B, int H, int H_kv, int N_k, int d);

/* Bytes of device workspace fa_decode_gqa needs (0 = the automatic split count): per (b, h,
 * split) one fp32 partial output row of d values and one fp32 log-sum-exp. */
size_t fa_decode_gqa_workspace_bytes(int B, int H, int H_kv, int N_k, int d, int num_splits);

/* Split-KV decode with grouped query heads over a contiguous cache (same grouping as above, no
 * block table, every sequence N_k positions long):
 *   q [B,H,1,d], k/v [B,H_kv,N_k,d] bf16 in; o [B,H,1,d] bf16 and lse [B,H,1] fp32 out;
 *   query head h reads K/V head h / (H / H_kv). num_splits: 0 = automatic, else
 *   1 .. min(N_k, 1024); split c covers positions [c * chunk, (c + 1) * chunk) with
 *   chunk = ceil(N_k / num_splits). All pointers and the workspace 16-byte aligned.
 * Errors as for fa_decode; FA_ERR_ARG also for H not a multiple of H_kv. */
fa_status fa_decode_gqa(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                        float* lse, void* workspace, size_t workspace_bytes, int B, int H,
                        int H_kv, int N_k, int d, float scale, int num_splits,
                        hipStream_t stream);

/* The split count fa_decode_paged uses when called with num_splits = 0. */
int fa_decode_paged_num_splits(int B, int H, int H_kv, int max_blocks_per_seq, int block_size,
                               int d);

/* Bytes of device workspace fa_decode_paged needs (0 = the automatic split count): per (b, h,
 * split) one fp32 partial output row of d values and one fp32 log-sum-exp. */
size_t fa_decode_paged_workspace_bytes(int B, int H, int H_kv, int max_blocks_per_seq,
                                       int block_size, int d, int num_splits);

/* Split-KV decode over the paged cache. num_splits: 0 = automatic, else 1 .. min(1024,
 * max_blocks_per_seq * block_size); split c of a sequence covers positions
 * [c * chunk, (c + 1) * chunk) with chunk = ceil(max_blocks_per_seq * block_size / num_splits).
 * q, k_cache, v_cache, o and workspace 16-byte aligned; block_table, seq_lens, lse 4-byte aligned.
 * Errors as for fa_decode; FA_ERR_ARG also for H not a multiple of H_kv, a block_size that is
 * not a power of two, or a split count out of range. */
fa_status fa_decode_paged(const fa_bf16* q, const fa_bf16* k_cache, const fa_bf16* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, fa_bf16* o,
                          float* lse, void* workspace, size_t workspace_bytes, int B, int H,
                          int H_kv, int d, int block_size, int num_blocks, int max_blocks_per_seq,
                          float scale, int num_splits, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
