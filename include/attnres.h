/*
 * attnres.h -- C ABI of libattnres, the MI355X (gfx950) implementation of the
 * Attention Residuals (AttnRes) depth aggregation.
 *
 * The operation (cited by page title and section):
 *   "DepthBench reading notes" (arXiv 2609.32534 notes), sec. 2.3 "Full
 *   AttnRes": for one token, with v_0 the embedding and v_i the raw output of
 *   sublayer i, a read with learned pseudo-query w scores every earlier source
 *   by e_i = w^T RMSNorm(v_i) (no 1/sqrt(d), temperature 1), takes a softmax
 *   over depth and returns z = sum_i a_i v_i over the raw values.
 *   "LLMRes" post (wln20), section "Kimi AttnRes": the same read with the
 *   query independent of the input, keys = values = earlier outputs, and the
 *   Block variant: additive sums inside a block, attention over block
 *   summaries.
 *   DataCamp "Attention Residuals explained", block section and the
 *   "two-phase computation" bullet: a Block read attends over the embedding,
 *   the completed block summaries and the running partial sum of the current
 *   block; phase 1 batches the reads of a block over the frozen sources,
 *   phase 2 merges the partial sum with an online softmax.
 *
 * Conventions used by every entry point:
 *   hist   [n_hist][T][d]  history rows: row 0 is the embedding, row i >= 1 the
 *                          output of sublayer i; d fastest, tokens next.
 *   w      [n_q][d] fp32   pseudo-queries of the reads this call computes; row j
 *                          belongs to read l = q_begin + j.  Any per-read gain of
 *                          the key RMSNorm is folded into w by the caller
 *                          (w * g), since r(x) (g o x) . w = r(x) x . (g o w).
 *   read l sees history rows 0..l: read 0 returns the embedding, read n_hist-1
 *                          is the final (LM-head) read over everything.
 *   RMSNorm of a key x:    r(x) = 1 / sqrt(sum_k x_k^2 / d + eps), unit gain.
 *   out    [n_q][T][d]     h_l for each read of the call.
 *   lse    [n_q][T] fp32   log-sum-exp of the read's scores (for the backward);
 *                          may be NULL.
 *   Block size S counts sublayer outputs: block c (c >= 1) is rows
 *   (c-1)S+1 .. cS.  Read l with m = floor(l/S) sees v_0, the block sums
 *   b_1..b_m, and the partial sum p_l = v_{mS+1} + ... + v_l when l mod S != 0.
 *   Block sums and partial sums are kept in fp32, never rounded to bf16.
 *
 * Memory and execution:
 *   * All tensor pointers are device pointers owned by the caller; the library
 *     allocates no device memory and keeps no state between calls apart from
 *     the thread-local error string, the dynamic-LDS limit of its LDS-staged
 *     kernels, which it raises to the device maximum once per kernel and
 *     device (never lowered), and a cache of how many workgroups of each
 *     persistent kernel a device holds at once (queried once).  The
 *     backward's scratch is caller-supplied.
 *   * d must be a multiple of 8 (8 <= d <= 4096); hist, out, dout, dhist and w
 *     must be 16-byte aligned, lse / rinv / dw 4-byte aligned.
 *   * T < 2^22 tokens and n_hist * T * d <= 2^40 elements per call
 *     (ATTNRES_ERR_UNSUPPORTED beyond: one launch counts its work-items in
 *     32 bits).  Tokens are independent, so larger inputs are split by
 *     tokens across calls (the backward's dw then sums over the calls).
 *   * Calls validate every argument on the host before any launch and return
 *     synchronously on error; on success the work is enqueued on `stream`
 *     (asynchronous).  Outputs must not alias inputs.
 *   * T == 0 or n_q == 0 is a valid empty call: nothing is launched.
 *   * NaN / Inf inputs propagate; they are not checked.
 *   * Thread-safe: calls share no mutable state apart from the one-time LDS
 *     limit and workgroup-count cache above, both set under a lock.
 *
 * Status: every entry point returns an attnres_status; attnres_last_error()
 * gives a human-readable detail of the last failure on the calling thread.
 */
#ifndef ATTNRES_H_
#define ATTNRES_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attnres_dtype {
    ATTNRES_F32 = 0,
    ATTNRES_BF16 = 1
} attnres_dtype;

typedef enum attnres_status {
    ATTNRES_OK = 0,
    ATTNRES_ERR_INVALID_ARG = 1, /* a size, index, null pointer or dtype is wrong */
    ATTNRES_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels handle     */
    ATTNRES_ERR_ALIGN = 3,       /* d % 8 != 0 or a pointer is misaligned         */
    ATTNRES_ERR_WORKSPACE = 4,   /* backward workspace missing or too small       */
    ATTNRES_ERR_HIP = 5          /* a HIP launch or runtime call failed           */
} attnres_status;

typedef enum attnres_variant {
    ATTNRES_FULL = 0,
    ATTNRES_BLOCK = 1
} attnres_variant;

/*
 * Full AttnRes forward ("DepthBench reading notes" sec. 2.3; "LLMRes",
 * "Kimi AttnRes"): for j in [0, n_q) and every token, read l = q_begin + j
 * over history rows 0..l.
 *
 *   hist, hist_dtype   [n_hist][T][d], F32 or BF16
 *   w                  [n_q][d] fp32
 *   q_begin, n_q       reads l = q_begin .. q_begin + n_q - 1 (q_begin + n_q <= n_hist)
 *   eps                RMSNorm epsilon (>= 0)
 *   rinv               optional [n_hist][T] fp32 cache of r(v_i) per (row, token).
 *                      Rows i < rinv_valid_rows are read from it and trusted;
 *                      rows rinv_valid_rows <= i < q_begin + n_q are computed in
 *                      the same pass and written to it, so a model that calls
 *                      read by read (q_begin = l, n_q = 1, rinv_valid_rows = l)
 *                      normalises every history row exactly once.  NULL: all
 *                      scales are computed on the fly (rinv_valid_rows must be 0).
 *   out, out_dtype     [n_q][T][d], F32 or BF16 (rounded once, to nearest even)
 *   lse                optional [n_q][T] fp32
 *   norm_gain, normed  optional fused pre-norm of each output, the sublayer's
 *                      branch input RMSNorm_pre,l(h_l) ("DepthBench reading
 *                      notes" sec. 2.3, the f_l equation): normed [n_q][T][d]
 *                      (out_dtype) = norm_gain[j] * h * r(h), with r as for
 *                      the keys, taken from the fp32 h before its rounding;
 *                      norm_gain [n_q][d] fp32, or NULL for unit gain.
 *                      normed NULL: no pre-norm (norm_gain ignored).
 *   alpha              optional weight probe [n_q][n_hist][T] fp32 (tokens
 *                      fastest): alpha[j][x][t] is the softmax weight of the
 *                      read's source x in source order (Full: rows 0..l);
 *                      entries past the read's source count are 0.  The data
 *                      behind the pages' weight maps ("DepthBench reading
 *                      notes", the AttnRes weight figures); a probe, not a
 *                      fast path (one lane per token writes it).
 */
int attnres_full_fwd(const void* hist, attnres_dtype hist_dtype, int64_t n_hist,
                     int64_t T, int64_t d, const float* w, int64_t q_begin,
                     int64_t n_q, float eps, float* rinv, int64_t rinv_valid_rows,
                     void* out, attnres_dtype out_dtype, float* lse,
                     const float* norm_gain, void* normed, float* alpha,
                     hipStream_t stream);

/*
 * Input-dependent query (the ablation in "Kimi K3 notes 2", sec. 6: a d x d
 * projection of the current hidden state replaces the learned per-read
 * query).  q[j][t] = W[j] x[j][t], i.e. q_k = sum_i W[j][k][i] x[j][t][i].
 *   x  [n_q][T][d] bf16: the hidden state each read projects from (for read
 *      l of a history, the newest row v_l: pass hist + l*T*d)
 *   W  [n_q][d][d] bf16, row-major (output index first)
 *   q  [n_q][T][d] fp32 (overwritten)
 * Other dtypes return ATTNRES_ERR_UNSUPPORTED.  d % 8 == 0, d <= 4096,
 * 16-byte aligned pointers.
 */
int attnres_query_proj(const void* x, attnres_dtype x_dtype, int64_t n_q, int64_t T, int64_t d,
                       const void* W, attnres_dtype w_dtype, float* q, hipStream_t stream);

/*
 * Full AttnRes forward with a query per (read, token) -- the same aggregation
 * as attnres_full_fwd, scored with q[j][t] (from attnres_query_proj or any
 * caller) instead of one w[j] per read.  Arguments as in attnres_full_fwd with
 * q [n_q][T][d] fp32 in place of w (16-byte aligned); no pre-norm or weight
 * probe.
 */
int attnres_full_fwd_q(const void* hist, attnres_dtype hist_dtype, int64_t n_hist, int64_t T,
                       int64_t d, const float* q, int64_t q_begin, int64_t n_q, float eps,
                       float* rinv, int64_t rinv_valid_rows, void* out, attnres_dtype out_dtype,
                       float* lse, hipStream_t stream);

/*
 * Block AttnRes forward, two-phase ("DepthBench reading notes" sec. 2.5;
 * "LLMRes", Block paragraph; DataCamp, block section and "two-phase
 * computation"): reads l = q_begin .. q_begin + n_q - 1 with block size S
 * (S >= 1; S = 1 is Full AttnRes).  The raw history is read once; block sums
 * and the partial sum are built on chip in fp32.  Arguments as in
 * attnres_full_fwd, without the rinv cache and the pre-norm; alpha (optional,
 * [n_q][n_hist][T]) holds the weights of v_0, b_1 .. b_m and, when the read
 * has one, the partial sum, in that order.
 */
int attnres_block_fwd(const void* hist, attnres_dtype hist_dtype, int64_t n_hist,
                      int64_t T, int64_t d, int64_t S, const float* w,
                      int64_t q_begin, int64_t n_q, float eps, void* out,
                      attnres_dtype out_dtype, float* lse, float* alpha,
                      hipStream_t stream);

/*
 * Block AttnRes forward with a query per (read, token) (the input-dependent
 * query of "Kimi K3 notes 2", sec. 6, applied to the Block read of
 * "DepthBench reading notes" sec. 2.5): the same reads as attnres_block_fwd,
 * scored with q[j][t] ([n_q][T][d] fp32, 16-byte aligned; from
 * attnres_query_proj or any caller) instead of one w[j] per read.  No weight
 * probe.  Other arguments and requirements as attnres_block_fwd.
 */
int attnres_block_fwd_q(const void* hist, attnres_dtype hist_dtype, int64_t n_hist,
                        int64_t T, int64_t d, int64_t S, const float* q,
                        int64_t q_begin, int64_t n_q, float eps, void* out,
                        attnres_dtype out_dtype, float* lse, hipStream_t stream);

/*
 * Block AttnRes in model order, phase 1 (DataCamp, "two-phase computation":
 * the reads of one block group share the frozen sources and are batched;
 * block reading of "DepthBench reading notes" sec. 2.5).  Called when history
 * row m*S arrives (m = n_src - 1), i.e. when block m is complete (m = 0: the
 * embedding v_0), before sublayer m*S + 1 runs:
 *   1. forms the new source  blocks[m] = partial + v  in fp32 (partial may be
 *      NULL: the new source is v alone -- v_0, or any block when S = 1);
 *   2. for the n_reads reads l = m*S .. m*S + n_reads - 1 of the group
 *      (n_reads <= S; fewer at the end of the history), scores the frozen
 *      sources blocks[0 .. m] with the read's query w[k] and writes
 *      o[k] = sum_c alpha_c blocks[c] (alpha the softmax over the frozen
 *      sources only, fp32) and lse1[k] = log sum_c exp(s_c);
 *   3. read m*S sees no partial sum, so its output h = o[0] is also written to
 *      out0 (out_dtype, rounded once; may be NULL) and its lse to lse0 (may
 *      be NULL); normed0 (out_dtype, may be NULL) receives its pre-norm
 *      norm_gain0 * h * r(h) as in attnres_full_fwd (norm_gain0 [d] or NULL).
 *   blocks  [n_src][T][d] fp32, caller-owned state across calls: rows
 *           0 .. n_src-2 must hold the earlier sources; row n_src-1 is written.
 *   v       [T][d] history row m*S (v_dtype); partial [T][d] fp32 or NULL.
 *   w       [n_reads][d] fp32; o [n_reads][T][d] fp32; lse1 [n_reads][T] fp32.
 *   rs      [n_src][T] fp32 RMS scales r(b_c), or NULL (then all are computed
 *           here): rows 0 .. n_src-2 must hold the values of earlier calls;
 *           row n_src-1 is written.
 * Requirements as attnres_block_fwd; 1 <= n_src <= 13, 1 <= n_reads <= 64.
 */
int attnres_block_phase1(float* blocks, int64_t n_src, int64_t T, int64_t d,
                         const void* v, attnres_dtype v_dtype, const float* partial,
                         const float* w, int64_t n_reads, float eps, float* rs,
                         float* o, float* lse1, void* out0, attnres_dtype out_dtype,
                         float* lse0, const float* norm_gain0, void* normed0,
                         hipStream_t stream);

/*
 * Block AttnRes in model order, phase 2 (DataCamp, "two-phase computation":
 * the partial sum of the current block is merged online): for read l with
 * l mod S != 0, after sublayer l has produced history row v:
 *   partial = (first_in_block ? 0 : partial) + v        (fp32, in place)
 *   s_p = r(partial) (w . partial),  M = max(lse1, s_p)
 *   h = (e^(lse1 - M) o + e^(s_p - M) partial) / (e^(lse1 - M) + e^(s_p - M))
 *   lse = M + log(e^(lse1 - M) + e^(s_p - M))
 * with o, lse1 the read's phase-1 results.  first_in_block is 1 for the first
 * row after a block boundary (l mod S == 1).
 *   v [T][d] (v_dtype); partial [T][d] fp32 in/out; w [d] fp32;
 *   o [T][d] fp32; lse1 [T] fp32; out [T][d] out_dtype; lse [T] fp32 or NULL;
 *   normed [T][d] out_dtype or NULL: the pre-norm norm_gain * h * r(h) of
 *   the output as in attnres_full_fwd (norm_gain [d] fp32 or NULL).
 * Requirements as attnres_block_fwd.
 */
int attnres_block_phase2(const void* v, attnres_dtype v_dtype, int64_t T, int64_t d,
                         float* partial, int first_in_block, const float* w,
                         const float* o, const float* lse1, float eps, void* out,
                         attnres_dtype out_dtype, float* lse, const float* norm_gain,
                         void* normed, hipStream_t stream);

/*
 * The two model-order phases with a query per token (the input-dependent
 * query of "Kimi K3 notes 2", sec. 6).  The pages name the price of that
 * query: read l's query is a projection of v_l, which exists only once
 * sublayer l has run, so the reads of a block group can no longer be scored
 * ahead in one batch -- the serial access the pages describe.  A model
 * therefore calls, for each read l with m = floor(l/S):
 *   l mod S == 0:  attnres_block_phase1_q with v = row l (closing block m,
 *                  n_src = m + 1), n_reads = 1, q = q_l: out0 receives h_l;
 *   otherwise:     attnres_block_phase1_q with v = NULL (no block closed;
 *                  all n_src = m + 1 sources are read from blocks, rs holds
 *                  all their scales or is NULL), n_reads = 1, q = q_l, into
 *                  o / lse1; then attnres_block_phase2_q with row l, q_l and
 *                  that o / lse1.
 *   attnres_block_phase1_q: arguments as attnres_block_phase1 with
 *     q [n_reads][T][d] fp32 in place of w; v may be NULL (then partial must
 *     be NULL and nothing is written to blocks or rs); no pre-norm.
 *   attnres_block_phase2_q: arguments as attnres_block_phase2 with q [T][d]
 *     fp32 in place of w; no pre-norm.
 */
int attnres_block_phase1_q(float* blocks, int64_t n_src, int64_t T, int64_t d,
                           const void* v, attnres_dtype v_dtype, const float* partial,
                           const float* q, int64_t n_reads, float eps, float* rs,
                           float* o, float* lse1, void* out0, attnres_dtype out_dtype,
                           float* lse0, hipStream_t stream);
int attnres_block_phase2_q(const void* v, attnres_dtype v_dtype, int64_t T, int64_t d,
                           float* partial, int first_in_block, const float* q,
                           const float* o, const float* lse1, float eps, void* out,
                           attnres_dtype out_dtype, float* lse, hipStream_t stream);

/*
 * Backward of attnres_full_fwd (variant ATTNRES_FULL) or attnres_block_fwd
 * (ATTNRES_BLOCK, block size S) for the reads q_begin .. q_begin + n_q - 1.
 * The pages state no gradient; this is the derivative of the forward
 * (keys and values are the same tensors, so each row gets a value-path and a
 * score-path term; block and partial sums pass their gradient to every row
 * they contain).  Gradients are of sum(out * dout).
 *
 *   (no lse argument: the softmax of each read is renormalised over its own
 *   recomputed scores, so a read with one source gets weight exactly 1)
 *   dout, dout_dtype   [n_q][T][d], F32 or BF16
 *   dhist, dhist_dtype [n_hist][T][d], F32 or BF16
 *   accumulate         0: dhist and dw are overwritten (rows no read of the
 *                      call sees get zero gradient).  1: the call's gradients
 *                      are added, dhist += ... and dw += ..., so a model that
 *                      runs the backward per group of reads (the schedule of
 *                      DataCamp's "two-phase computation") or per token range
 *                      sums the pieces in place; needs an F32 dhist
 *                      (ATTNRES_ERR_INVALID_ARG otherwise), and leaves rows no
 *                      read sees unchanged.
 *   dw                 [n_q][d] fp32 (summed over tokens in a fixed order, so
 *                      results are bitwise reproducible)
 *   workspace          device scratch of at least attnres_bwd_workspace_bytes()
 *                      bytes, 256-byte aligned; contents on entry are ignored
 * The per-read coefficients of a token are formed in one workgroup's LDS;
 * when a call's sources do not fit (Full with more than about 1600 rows), or
 * when n_hist * n_q exceeds about 8 million (the coefficients of 32 tokens
 * then pass 1 GiB), it returns ATTNRES_ERR_UNSUPPORTED.
 */
int attnres_bwd(attnres_variant variant, int64_t S, const void* hist,
                attnres_dtype hist_dtype, int64_t n_hist, int64_t T, int64_t d,
                const float* w, int64_t q_begin, int64_t n_q, float eps,
                const void* dout, attnres_dtype dout_dtype,
                void* dhist, attnres_dtype dhist_dtype, int accumulate, float* dw,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attnres_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments and results as attnres_bwd; the workspace is a static device
 * array of attnres_bwd_noalloc_max_workspace() bytes (64 MiB) that the
 * library holds on every GPU it runs on until the process ends.  A call
 * whose attnres_bwd_workspace_bytes() exceeds it returns
 * ATTNRES_ERR_UNSUPPORTED (split such calls by tokens).  The call allocates
 * nothing; the first call on a device looks the array's address up once.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (two streams, two threads) race and must be serialised by the
 * caller.
 */
int attnres_bwd_noalloc(attnres_variant variant, int64_t S, const void* hist,
                        attnres_dtype hist_dtype, int64_t n_hist, int64_t T, int64_t d,
                        const float* w, int64_t q_begin, int64_t n_q, float eps,
                        const void* dout, attnres_dtype dout_dtype,
                        void* dhist, attnres_dtype dhist_dtype, int accumulate, float* dw,
                        hipStream_t stream);

/* Bytes of the static workspace attnres_bwd_noalloc uses. */
size_t attnres_bwd_noalloc_max_workspace(void);

/* Bytes of workspace attnres_bwd needs for these sizes (0 on invalid sizes). */
size_t attnres_bwd_workspace_bytes(attnres_variant variant, int64_t S, int64_t n_hist,
                                   int64_t T, int64_t d, int64_t q_begin, int64_t n_q);

/*
 * Block index table (host only, no GPU work): for each read l = q_begin + j,
 * writes out[3j + 0] = m = floor(l / S) (completed blocks),
 * out[3j + 1] = first row of the partial sum (mS + 1),
 * out[3j + 2] = one past its last row (l + 1; empty when equal to out[3j + 1]).
 * `out` is host memory of 3 * n_q int32.
 */
int attnres_block_index_table(int64_t n_hist, int64_t S, int64_t q_begin, int64_t n_q,
                              int32_t* out);

/* Static description of a status code. */
const char* attnres_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* attnres_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H_ */
