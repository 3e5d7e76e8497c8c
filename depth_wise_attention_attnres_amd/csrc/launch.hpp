// launch.hpp -- internal interface between the C-ABI front end and the
// kernel launchers.  Not installed; callers use include/attnres.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attnres.h"

namespace attnres {

constexpr int kMaxD = 4096;
// Tokens per call.  A dispatch counts work-items per grid dimension in 32
// bits, and the widest launches hold 1024 work-items per token (the backward's
// dhist at d = 4096: 16 slices x 64 lanes; the batched and Block forwards: up
// to 512), so T stays below 2^22.  Tokens are independent: larger inputs are
// split by the caller.
constexpr int64_t kMaxTokens = ((int64_t)1 << 22) - 1;
// Block reads whose source count (v_0 + completed blocks) is at most this keep
// their sources in registers (two-phase kernel); more blocks use the
// streaming kernel, which forms block sums on the fly per read.
constexpr int kBlockMaxRegSources = 13;

struct FwdParams {
    const void* hist;  // [n_hist][T][d]
    const float* w;    // [n_q][d]
    float* rinv;       // [n_hist][T] or null
    void* out;         // [n_q][T][d]
    float* lse;        // [n_q][T] or null
    const float* norm_gain;  // [n_q][d] or null (unit gain)
    void* normed;      // [n_q][T][d] pre-norm of the outputs, or null
    float* alpha;      // [n_q][n_hist][T] softmax weights in source order, or null
    const float* qtok; // [n_q][T][d] per-token queries (then w is unused), or null
    int64_t T;
    int d;             // width, multiple of 8
    int nc;            // d / 8 chunks
    int n_hist;
    int q_begin;
    int n_q;
    int rinv_valid;    // rows of rinv trusted on entry
    int S;             // block size (Block reads only)
    attnres_dtype hist_dt;
    attnres_dtype out_dt;
    float eps;
    float inv_d;
};
typedef FwdParams FullFwdParams;
typedef FwdParams BlockFwdParams;

hipError_t launch_full_fwd(const FullFwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                           hipStream_t stream);
// Full reads of a call with many reads over a bf16 history with bf16 outputs,
// every row staged in LDS, both contractions on the matrix cores
bool full_batch_mfma_applies(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt);
hipError_t launch_full_batch_mfma(const FwdParams& p, hipStream_t stream);
// For a call that kernel cannot take whole (more history rows than it stages):
// the most leading reads it can take (their rows 0 .. q_begin + n - 1 fit),
// or 0 (the whole call fits, or no prefix of at least its minimum does)
int full_batch_mfma_prefix(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt);
hipError_t launch_block_fwd(const BlockFwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                            hipStream_t stream);
// Full reads of a call with many reads, served from the token's rows staged in
// LDS (full_batch.hip): whether the call qualifies, and the launch
bool full_batch_applies(const FwdParams& p, attnres_dtype hist_dt);
hipError_t launch_full_batch(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                             hipStream_t stream);
// Block reads of a call with many reads, one wave per half block group
// (block_batch.hip): whether the call qualifies, and the launch
bool block_batch_applies(const FwdParams& p, attnres_dtype hist_dt);
hipError_t launch_block_batch(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                              hipStream_t stream);
// streaming Block kernel (one pass over rows 0..l per read, sums formed on the fly)
hipError_t launch_block_stream(const BlockFwdParams& p, hipStream_t stream);

// Backward workspace layout (byte offsets; every region 256-byte aligned).
struct BwdLayout {
    int64_t nh8;       // history rows rounded up to 8 (row length of A1 / A2)
    int64_t nq8;       // reads rounded up to 8 (row length of A2T, zero padded)
    int64_t n_blk;     // v_0 + every block, complete or not
    int64_t nx;        // most sources a read can see
    int64_t n_chunks;  // token chunks of the dw partial sums
    int64_t n_dw_groups;  // chunk groups of the first dw reduction stage
    int64_t off_a1, off_a2, off_a2t, off_c3, off_kappa, off_dwpart, off_wsplit, off_dwstage,
        off_wsplit2;
    int64_t bytes;
};
BwdLayout bwd_layout(int64_t S, int64_t n_hist, int64_t T, int64_t d, int64_t n_q);

struct BwdParams {
    const void* hist;   // [n_hist][T][d]
    const void* dout;   // [n_q][T][d]
    void* dhist;        // [n_hist][T][d]
    const float* w;     // [n_q][d]
    float* dw;          // [n_q][d]
    int64_t T;
    int d, nc, n_hist, q_begin, n_q, S;
    int nh8, nq8, n_blk, nx;
    int accumulate;     // 1: dhist += (fp32 only) and dw += instead of overwriting
    float eps, inv_d;
    attnres_dtype hist_dt, dout_dt, dhist_dt;
    float* ws_a1;       // [T][n_q][nh8]   alpha of the source holding each row
    float* ws_a2;       // [T][n_q][nh8]   ds * r of that source
    float* ws_a2t;      // [T][n_hist][nq8] the same, transposed (reads past n_q are 0)
    float* ws_c3;       // [T][n_blk]      sum over reads of ds r^2 s / d per v_0 / block
    float* ws_kappa;    // [T][n_q]        ds r^2 s / d of each read's partial sum
    float* ws_dwpart;   // [n_chunks][n_q][d]
    float* ws_dwstage;  // [n_dw_groups][n_q][d]
    uint16_t* ws_wsplit;  // [3][n_q][d] bf16: w = hi + mid + lo (matrix-core scores)
    uint16_t* ws_wsplit2;  // [2][n_q][d] bf16: w = hi + mid (matrix-core history gradient)
};
hipError_t launch_bwd(const BwdParams& p, int n_chunks, int n_dw_groups, hipStream_t stream);
// whether some coefficient kernel takes the call (its LDS fits the device)
bool bwd_fits(const BwdParams& p);
// the history gradient on the matrix cores (bwd_dhist_mfma.hip): bf16 history,
// upstream gradient and history gradient; whether the call qualifies, the
// launch, and the size of its w split (bf16 elements)
bool bwd_dhist_mfma_applies(const BwdParams& p);
hipError_t launch_bwd_dhist_mfma(const BwdParams& p, hipStream_t stream);
int64_t bwd_wsplit2_elems(int64_t n_q, int64_t d);
// the per-chunk dw partials on the matrix cores (bwd_dw_mfma.hip): bf16
// history, at most 64 reads; whether the call qualifies, the launch
bool bwd_dw_mfma_applies(const BwdParams& p);
hipError_t launch_bwd_dw_mfma(const BwdParams& p, int chunk_tokens, hipStream_t stream);
// Size of the static device array that serves as the backward's workspace for
// callers that cannot allocate, and its address on the current device (taken
// once per device; bwd_scratch.hip).
constexpr int64_t kBwdScratchBytes = (int64_t)64 << 20;
hipError_t bwd_scratch(void** ptr);
// the backward's per-read coefficients for Block calls with many reads, one
// wave per block group (bwd_group.hip): whether the call qualifies, the launch
bool bwd_scores_group_applies(const BwdParams& p);
hipError_t launch_bwd_scores_group(const BwdParams& p, hipStream_t stream);

// Block AttnRes in model order (block_model.hip)
struct Phase1Params {
    float* blocks;          // [n_src][T][d] fp32; row n_src-1 written (unless v is null)
    const void* v;          // [T][d] history row closing the block, or null: no new
                            // source, all n_src sources are read from blocks
    const float* partial;   // [T][d] fp32 or null
    const float* w;         // [n_reads][d]
    const float* qtok;      // [n_reads][T][d] per-token queries (then w is unused), or null
    float* rs;              // [n_src][T] or null
    float* o;               // [n_reads][T][d] fp32
    float* lse1;            // [n_reads][T]
    void* out0;             // [T][d] or null
    float* lse0;            // [T] or null
    const float* norm_gain0;  // [d] or null
    void* normed0;          // [T][d] or null
    int64_t T;
    int d, nc, n_src, n_reads;
    attnres_dtype v_dt, out_dt;
    float eps, inv_d;
};
struct Phase2Params {
    const void* v;          // [T][d]
    float* partial;         // [T][d] fp32, in place
    const float* w;         // [d]
    const float* qtok;      // [T][d] per-token query (then w is unused), or null
    const float* o;         // [T][d] fp32
    const float* lse1;      // [T]
    void* out;              // [T][d]
    float* lse;             // [T] or null
    const float* norm_gain; // [d] or null
    void* normed;           // [T][d] or null
    int64_t T;
    int d, nc, first;
    attnres_dtype v_dt, out_dt;
    float eps, inv_d;
};
hipError_t launch_block_phase1(const Phase1Params& p, hipStream_t stream);
// q[j][t] = W[j] x[j][t] on the matrix cores (bf16 x and W, fp32 q)
hipError_t launch_query_proj(const void* x, const void* W, float* q, int64_t n_q, int64_t T, int d,
                             hipStream_t stream);
hipError_t launch_block_phase2(const Phase2Params& p, hipStream_t stream);
// zero `bytes` (a multiple of 4) of device memory with a kernel
hipError_t launch_fill_zero(void* dst, int64_t bytes, hipStream_t stream);

// LDS per workgroup of the current device (0 if it cannot be queried)
int device_max_lds();
// Before launching `kernel` with `bytes` of dynamic LDS: raises the kernel's
// limit on the current device to the device maximum, once per (kernel,
// device) for the process (never per call, so concurrent callers cannot lower
// it under each other), and returns hipErrorInvalidValue if `bytes` exceeds
// that maximum.
hipError_t prepare_dynamic_lds(const void* kernel, size_t bytes);
// Workgroups of `threads` threads and `lds` bytes of dynamic LDS that the
// current device holds at once (CUs times workgroups per CU), for persistent
// grids; looked up once per (kernel, device, threads, LDS).
hipError_t resident_workgroups(const void* kernel, int threads, size_t lds, int64_t* slots);

}  // namespace attnres
