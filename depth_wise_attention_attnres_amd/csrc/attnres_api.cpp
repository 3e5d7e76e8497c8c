// attnres_api.cpp -- C-ABI front end of libattnres: argument validation on
// the host (before any HIP call), the Block index table, status strings and
// the thread-local error detail, then dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cinttypes>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "attnres.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return ATTNRES_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dtype(int dt) { return dt == ATTNRES_F32 || dt == ATTNRES_BF16; }

// checks shared by every entry point; returns ATTNRES_OK or an error status
int check_common(const char* fn, const void* hist, int hist_dt, int64_t n_hist, int64_t T,
                 int64_t d, const float* w, int64_t q_begin, int64_t n_q, float eps) {
    if (!valid_dtype(hist_dt)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad hist dtype %d", fn, hist_dt);
    if (n_hist < 1) return fail(ATTNRES_ERR_INVALID_ARG, "%s: n_hist must be >= 1 (got %" PRId64 ")", fn, n_hist);
    if (T < 0) return fail(ATTNRES_ERR_INVALID_ARG, "%s: T must be >= 0 (got %" PRId64 ")", fn, T);
    if (d < 1) return fail(ATTNRES_ERR_INVALID_ARG, "%s: d must be >= 1 (got %" PRId64 ")", fn, d);
    if (q_begin < 0 || n_q < 0 || q_begin + n_q > n_hist)
        return fail(ATTNRES_ERR_INVALID_ARG,
                    "%s: reads [%" PRId64 ", %" PRId64 ") outside the history of %" PRId64 " rows",
                    fn, q_begin, q_begin + n_q, n_hist);
    if (!(eps >= 0.f) || !std::isfinite(eps))
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
    if (d % 8 != 0) return fail(ATTNRES_ERR_ALIGN, "%s: d = %" PRId64 " is not a multiple of 8", fn, d);
    if (d > attnres::kMaxD)
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: d = %" PRId64 " exceeds %d", fn, d, attnres::kMaxD);
    if (n_hist > (int64_t)1 << 20)
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: n_hist = %" PRId64 " too large", fn, n_hist);
    // grids hold up to 1024 work-items per token, in 32 bits
    if (T > attnres::kMaxTokens)
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: T = %" PRId64 " exceeds 2^22 - 1 tokens per call", fn, T);
    // every element offset must fit int64 comfortably
    if (T > ((int64_t)1 << 40) / (n_hist * d))
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: history of %" PRId64 " x %" PRId64 " x %" PRId64 " too large",
                    fn, n_hist, T, d);
    if (T > 0 && n_q > 0) {
        if (hist == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: hist is NULL", fn);
        if (w == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: w is NULL", fn);
        if (!aligned(hist, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: hist is not 16-byte aligned", fn);
        if (!aligned(w, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: w is not 16-byte aligned", fn);
    }
    return ATTNRES_OK;
}

int hip_status(const char* fn, hipError_t e) {
    if (e != hipSuccess)
        return fail(ATTNRES_ERR_HIP, "%s: %s (%s)", fn, hipGetErrorName(e), hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* attnres_status_string(int status) {
    switch (status) {
        case ATTNRES_OK: return "ATTNRES_OK: success";
        case ATTNRES_ERR_INVALID_ARG: return "ATTNRES_ERR_INVALID_ARG: invalid argument";
        case ATTNRES_ERR_UNSUPPORTED: return "ATTNRES_ERR_UNSUPPORTED: size not supported";
        case ATTNRES_ERR_ALIGN: return "ATTNRES_ERR_ALIGN: d % 8 != 0 or misaligned pointer";
        case ATTNRES_ERR_WORKSPACE: return "ATTNRES_ERR_WORKSPACE: workspace missing or too small";
        case ATTNRES_ERR_HIP: return "ATTNRES_ERR_HIP: HIP runtime error";
        default: return "unknown attnres status";
    }
}

const char* attnres_last_error(void) { return g_last_error; }

int attnres_block_index_table(int64_t n_hist, int64_t S, int64_t q_begin, int64_t n_q,
                              int32_t* out) {
    const char* fn = "attnres_block_index_table";
    if (n_hist < 1 || n_hist > INT32_MAX) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad n_hist", fn);
    if (S < 1) return fail(ATTNRES_ERR_INVALID_ARG, "%s: S must be >= 1", fn);
    if (q_begin < 0 || n_q < 0 || q_begin + n_q > n_hist)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: reads outside the history", fn);
    if (n_q > 0 && out == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: out is NULL", fn);
    for (int64_t j = 0; j < n_q; ++j) {
        const int64_t l = q_begin + j;
        const int64_t m = l / S;
        out[3 * j + 0] = (int32_t)m;
        out[3 * j + 1] = (int32_t)(m * S + 1);
        out[3 * j + 2] = (int32_t)(l + 1);
    }
    return ok();
}

namespace {

// w (one query per read) or qtok (one per read and token; w must be NULL)
int full_fwd_impl(const char* fn, const void* hist, attnres_dtype hist_dtype, int64_t n_hist,
                  int64_t T, int64_t d, const float* w, const float* qtok, int64_t q_begin,
                  int64_t n_q, float eps, float* rinv, int64_t rinv_valid_rows, void* out,
                  attnres_dtype out_dtype, float* lse, const float* norm_gain, void* normed,
                  float* alpha, hipStream_t stream) {
    int st = check_common(fn, hist, hist_dtype, n_hist, T, d, qtok != nullptr ? qtok : w, q_begin,
                          n_q, eps);
    if (st != ATTNRES_OK) return st;
    if (!valid_dtype(out_dtype)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad out dtype %d", fn, (int)out_dtype);
    if (rinv_valid_rows < 0 || rinv_valid_rows > n_hist)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: rinv_valid_rows = %" PRId64 " outside [0, n_hist]", fn,
                    rinv_valid_rows);
    if (rinv == nullptr && rinv_valid_rows != 0)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: rinv_valid_rows > 0 needs a rinv cache", fn);
    if (T == 0 || n_q == 0) return ok();
    if (out == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (!aligned(out, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: out is not 16-byte aligned", fn);
    if (lse != nullptr && !aligned(lse, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: lse is not 4-byte aligned", fn);
    if (rinv != nullptr && !aligned(rinv, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: rinv is not 4-byte aligned", fn);
    if (normed != nullptr && !aligned(normed, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: normed is not 16-byte aligned", fn);
    if (normed != nullptr && norm_gain != nullptr && !aligned(norm_gain, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: norm_gain is not 16-byte aligned", fn);
    if (alpha != nullptr && !aligned(alpha, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: alpha is not 4-byte aligned", fn);

    attnres::FullFwdParams p;
    p.alpha = alpha;
    p.qtok = qtok;
    p.hist = hist;
    p.w = w;
    p.rinv = rinv;
    p.out = out;
    p.lse = lse;
    p.norm_gain = normed != nullptr ? norm_gain : nullptr;
    p.normed = normed;
    p.T = T;
    p.d = (int)d;
    p.nc = (int)(d / 8);
    p.n_hist = (int)n_hist;
    p.q_begin = (int)q_begin;
    p.n_q = (int)n_q;
    p.rinv_valid = (int)rinv_valid_rows;
    p.S = 1;
    p.hist_dt = hist_dtype;
    p.out_dt = out_dtype;
    p.eps = eps;
    p.inv_d = 1.0f / (float)d;
    // A call with more history rows than the matrix-core kernel stages: its
    // leading reads (those that see few enough rows) go there, the rest to the
    // kernel that takes the call otherwise.  The first part writes the RMS
    // cache of the rows it reads, which the second then trusts.
    const int n1 = attnres::full_batch_mfma_prefix(p, hist_dtype, out_dtype);
    if (n1 > 0) {
        attnres::FullFwdParams p1 = p;
        p1.n_q = n1;
        hipError_t e = attnres::launch_full_fwd(p1, hist_dtype, out_dtype, stream);
        if (e != hipSuccess) return hip_status(fn, e);
        const size_t out_elem = out_dtype == ATTNRES_BF16 ? 2 : 4;
        p.q_begin += n1;
        p.n_q -= n1;
        p.w = w + (int64_t)n1 * d;
        p.out = static_cast<char*>(out) + (size_t)n1 * (size_t)T * (size_t)d * out_elem;
        if (lse != nullptr) p.lse = lse + (int64_t)n1 * T;
        if (alpha != nullptr) p.alpha = alpha + (int64_t)n1 * n_hist * T;
        if (rinv != nullptr) p.rinv_valid = std::max(p.rinv_valid, p.q_begin);
    }
    return hip_status(fn, attnres::launch_full_fwd(p, hist_dtype, out_dtype, stream));
}

}  // namespace

int attnres_full_fwd(const void* hist, attnres_dtype hist_dtype, int64_t n_hist, int64_t T,
                     int64_t d, const float* w, int64_t q_begin, int64_t n_q, float eps,
                     float* rinv, int64_t rinv_valid_rows, void* out, attnres_dtype out_dtype,
                     float* lse, const float* norm_gain, void* normed, float* alpha,
                     hipStream_t stream) {
    return full_fwd_impl("attnres_full_fwd", hist, hist_dtype, n_hist, T, d, w, nullptr, q_begin,
                         n_q, eps, rinv, rinv_valid_rows, out, out_dtype, lse, norm_gain, normed,
                         alpha, stream);
}

int attnres_full_fwd_q(const void* hist, attnres_dtype hist_dtype, int64_t n_hist, int64_t T,
                       int64_t d, const float* q, int64_t q_begin, int64_t n_q, float eps,
                       float* rinv, int64_t rinv_valid_rows, void* out, attnres_dtype out_dtype,
                       float* lse, hipStream_t stream) {
    return full_fwd_impl("attnres_full_fwd_q", hist, hist_dtype, n_hist, T, d, nullptr, q, q_begin,
                         n_q, eps, rinv, rinv_valid_rows, out, out_dtype, lse, nullptr, nullptr,
                         nullptr, stream);
}

int attnres_query_proj(const void* x, attnres_dtype x_dtype, int64_t n_q, int64_t T, int64_t d,
                       const void* W, attnres_dtype w_dtype, float* q, hipStream_t stream) {
    const char* fn = "attnres_query_proj";
    if (!valid_dtype(x_dtype) || !valid_dtype(w_dtype))
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad dtype", fn);
    if (n_q < 0 || T < 0 || d < 1) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad sizes", fn);
    if (d % 8 != 0) return fail(ATTNRES_ERR_ALIGN, "%s: d = %" PRId64 " is not a multiple of 8", fn, d);
    if (d > attnres::kMaxD) return fail(ATTNRES_ERR_UNSUPPORTED, "%s: d = %" PRId64 " exceeds %d", fn, d, attnres::kMaxD);
    if (x_dtype != ATTNRES_BF16 || w_dtype != ATTNRES_BF16)
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: only bf16 x and W (the matrix-core path)", fn);
    if (T > attnres::kMaxTokens)
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: T = %" PRId64 " exceeds 2^22 - 1 tokens per call", fn, T);
    // one 512-work-item workgroup per 256 x 256 tile, the (read, token tile)
    // groups rounded up to a multiple of 8 (one round per XCD); 32-bit
    // work-item count
    if (8 * ((d + 255) / 256) * ((n_q * ((T + 255) / 256) + 7) / 8) >= ((int64_t)1 << 23))
        return fail(ATTNRES_ERR_UNSUPPORTED, "%s: too many tiles for one launch (n_q x T x d >= 2^39)", fn);
    if (n_q == 0 || T == 0) return ok();
    if (x == nullptr || W == nullptr || q == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(q, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: x, W and q must be 16-byte aligned", fn);
    return hip_status(fn, attnres::launch_query_proj(x, W, q, n_q, T, (int)d, stream));
}

}  // extern "C"

namespace {

// w (one query per read) or qtok (one per read and token; w must be NULL)
int block_fwd_impl(const char* fn, const void* hist, attnres_dtype hist_dtype, int64_t n_hist,
                   int64_t T, int64_t d, int64_t S, const float* w, const float* qtok,
                   int64_t q_begin, int64_t n_q, float eps, void* out, attnres_dtype out_dtype,
                   float* lse, float* alpha, hipStream_t stream) {
    int st = check_common(fn, hist, hist_dtype, n_hist, T, d, qtok != nullptr ? qtok : w, q_begin,
                          n_q, eps);
    if (st != ATTNRES_OK) return st;
    if (S < 1) return fail(ATTNRES_ERR_INVALID_ARG, "%s: S must be >= 1 (got %" PRId64 ")", fn, S);
    if (!valid_dtype(out_dtype)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad out dtype %d", fn, (int)out_dtype);
    if (T == 0 || n_q == 0) return ok();
    if (out == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (!aligned(out, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: out is not 16-byte aligned", fn);
    if (lse != nullptr && !aligned(lse, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: lse is not 4-byte aligned", fn);
    if (alpha != nullptr && !aligned(alpha, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: alpha is not 4-byte aligned", fn);

    attnres::BlockFwdParams p;
    p.alpha = alpha;
    p.qtok = qtok;
    p.hist = hist;
    p.w = w;
    p.rinv = nullptr;
    p.out = out;
    p.lse = lse;
    p.norm_gain = nullptr;
    p.normed = nullptr;
    p.T = T;
    p.d = (int)d;
    p.nc = (int)(d / 8);
    p.n_hist = (int)n_hist;
    p.q_begin = (int)q_begin;
    p.n_q = (int)n_q;
    p.rinv_valid = 0;
    p.S = (int)(S < n_hist ? S : n_hist);  // S >= n_hist behaves like S = n_hist
    p.hist_dt = hist_dtype;
    p.out_dt = out_dtype;
    p.eps = eps;
    p.inv_d = 1.0f / (float)d;
    return hip_status(fn, attnres::launch_block_fwd(p, hist_dtype, out_dtype, stream));
}

}  // namespace

extern "C" {

int attnres_block_fwd(const void* hist, attnres_dtype hist_dtype, int64_t n_hist, int64_t T,
                      int64_t d, int64_t S, const float* w, int64_t q_begin, int64_t n_q,
                      float eps, void* out, attnres_dtype out_dtype, float* lse, float* alpha,
                      hipStream_t stream) {
    return block_fwd_impl("attnres_block_fwd", hist, hist_dtype, n_hist, T, d, S, w, nullptr,
                          q_begin, n_q, eps, out, out_dtype, lse, alpha, stream);
}

int attnres_block_fwd_q(const void* hist, attnres_dtype hist_dtype, int64_t n_hist, int64_t T,
                        int64_t d, int64_t S, const float* q, int64_t q_begin, int64_t n_q,
                        float eps, void* out, attnres_dtype out_dtype, float* lse,
                        hipStream_t stream) {
    return block_fwd_impl("attnres_block_fwd_q", hist, hist_dtype, n_hist, T, d, S, nullptr, q,
                          q_begin, n_q, eps, out, out_dtype, lse, nullptr, stream);
}

}  // extern "C"

namespace {

// w (one query per read) or qtok (per read and token); v may be NULL only
// with qtok (no new source: every source is read from blocks)
int phase1_impl(const char* fn, float* blocks, int64_t n_src, int64_t T, int64_t d, const void* v,
                attnres_dtype v_dtype, const float* partial, const float* w, const float* qtok,
                int64_t n_reads, float eps, float* rs, float* o, float* lse1, void* out0,
                attnres_dtype out_dtype, float* lse0, const float* norm_gain0, void* normed0,
                hipStream_t stream) {
    if (v == nullptr && qtok == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: v is NULL", fn);
    if (v == nullptr && partial != nullptr)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: partial given without a row v to close a block", fn);
    if (n_src < 1 || n_src > attnres::kBlockMaxRegSources)
        return fail(n_src < 1 ? ATTNRES_ERR_INVALID_ARG : ATTNRES_ERR_UNSUPPORTED,
                    "%s: n_src = %" PRId64 " outside 1 .. %d", fn, n_src, attnres::kBlockMaxRegSources);
    if (n_reads < 1 || n_reads > 64)
        return fail(n_reads < 1 ? ATTNRES_ERR_INVALID_ARG : ATTNRES_ERR_UNSUPPORTED,
                    "%s: n_reads = %" PRId64 " outside 1 .. 64", fn, n_reads);
    // v is the new history row (or, without one, the block store is checked in
    // its place); one query row is checked like a read
    int st = check_common(fn, v != nullptr ? v : (const void*)blocks,
                          v != nullptr ? v_dtype : ATTNRES_F32, n_src, T, d,
                          qtok != nullptr ? qtok : w, 0, 1, eps);
    if (st != ATTNRES_OK) return st;
    if (!valid_dtype(out_dtype)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad out dtype %d", fn, (int)out_dtype);
    if (T == 0) return ok();
    if (blocks == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: blocks is NULL", fn);
    if (o == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: o is NULL", fn);
    if (lse1 == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: lse1 is NULL", fn);
    if (!aligned(blocks, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: blocks is not 16-byte aligned", fn);
    if (partial != nullptr && !aligned(partial, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: partial is not 16-byte aligned", fn);
    if (!aligned(o, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: o is not 16-byte aligned", fn);
    if (!aligned(lse1, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: lse1 is not 4-byte aligned", fn);
    if (rs != nullptr && !aligned(rs, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: rs is not 4-byte aligned", fn);
    if (out0 != nullptr && !aligned(out0, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: out0 is not 16-byte aligned", fn);
    if (lse0 != nullptr && !aligned(lse0, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: lse0 is not 4-byte aligned", fn);
    if (normed0 != nullptr && !aligned(normed0, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: normed0 is not 16-byte aligned", fn);
    if (normed0 != nullptr && norm_gain0 != nullptr && !aligned(norm_gain0, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: norm_gain0 is not 16-byte aligned", fn);

    attnres::Phase1Params p;
    p.norm_gain0 = normed0 != nullptr ? norm_gain0 : nullptr;
    p.normed0 = normed0;
    p.blocks = blocks;
    p.v = v;
    p.partial = partial;
    p.w = w;
    p.qtok = qtok;
    p.rs = rs;
    p.o = o;
    p.lse1 = lse1;
    p.out0 = out0;
    p.lse0 = lse0;
    p.T = T;
    p.d = (int)d;
    p.nc = (int)(d / 8);
    p.n_src = (int)n_src;
    p.n_reads = (int)n_reads;
    p.v_dt = v_dtype;
    p.out_dt = out_dtype;
    p.eps = eps;
    p.inv_d = 1.0f / (float)d;
    return hip_status(fn, attnres::launch_block_phase1(p, stream));
}

}  // namespace

extern "C" {

int attnres_block_phase1(float* blocks, int64_t n_src, int64_t T, int64_t d, const void* v,
                         attnres_dtype v_dtype, const float* partial, const float* w,
                         int64_t n_reads, float eps, float* rs, float* o, float* lse1, void* out0,
                         attnres_dtype out_dtype, float* lse0, const float* norm_gain0,
                         void* normed0, hipStream_t stream) {
    return phase1_impl("attnres_block_phase1", blocks, n_src, T, d, v, v_dtype, partial, w,
                       nullptr, n_reads, eps, rs, o, lse1, out0, out_dtype, lse0, norm_gain0,
                       normed0, stream);
}

int attnres_block_phase1_q(float* blocks, int64_t n_src, int64_t T, int64_t d, const void* v,
                           attnres_dtype v_dtype, const float* partial, const float* q,
                           int64_t n_reads, float eps, float* rs, float* o, float* lse1,
                           void* out0, attnres_dtype out_dtype, float* lse0, hipStream_t stream) {
    return phase1_impl("attnres_block_phase1_q", blocks, n_src, T, d, v, v_dtype, partial, nullptr,
                       q, n_reads, eps, rs, o, lse1, out0, out_dtype, lse0, nullptr, nullptr,
                       stream);
}

}  // extern "C"

namespace {

int phase2_impl(const char* fn, const void* v, attnres_dtype v_dtype, int64_t T, int64_t d,
                float* partial, int first_in_block, const float* w, const float* qtok,
                const float* o, const float* lse1, float eps, void* out, attnres_dtype out_dtype,
                float* lse, const float* norm_gain, void* normed, hipStream_t stream) {
    int st = check_common(fn, v, v_dtype, 1, T, d, qtok != nullptr ? qtok : w, 0, 1, eps);
    if (st != ATTNRES_OK) return st;
    if (!valid_dtype(out_dtype)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad out dtype %d", fn, (int)out_dtype);
    if (first_in_block != 0 && first_in_block != 1)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: first_in_block must be 0 or 1", fn);
    if (T == 0) return ok();
    if (partial == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: partial is NULL", fn);
    if (o == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: o is NULL", fn);
    if (lse1 == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: lse1 is NULL", fn);
    if (out == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (!aligned(partial, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: partial is not 16-byte aligned", fn);
    if (!aligned(o, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: o is not 16-byte aligned", fn);
    if (!aligned(lse1, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: lse1 is not 4-byte aligned", fn);
    if (!aligned(out, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: out is not 16-byte aligned", fn);
    if (lse != nullptr && !aligned(lse, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: lse is not 4-byte aligned", fn);
    if (normed != nullptr && !aligned(normed, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: normed is not 16-byte aligned", fn);
    if (normed != nullptr && norm_gain != nullptr && !aligned(norm_gain, 16))
        return fail(ATTNRES_ERR_ALIGN, "%s: norm_gain is not 16-byte aligned", fn);

    attnres::Phase2Params p;
    p.norm_gain = normed != nullptr ? norm_gain : nullptr;
    p.normed = normed;
    p.v = v;
    p.partial = partial;
    p.w = w;
    p.qtok = qtok;
    p.o = o;
    p.lse1 = lse1;
    p.out = out;
    p.lse = lse;
    p.T = T;
    p.d = (int)d;
    p.nc = (int)(d / 8);
    p.first = first_in_block;
    p.v_dt = v_dtype;
    p.out_dt = out_dtype;
    p.eps = eps;
    p.inv_d = 1.0f / (float)d;
    return hip_status(fn, attnres::launch_block_phase2(p, stream));
}

}  // namespace

extern "C" {

int attnres_block_phase2(const void* v, attnres_dtype v_dtype, int64_t T, int64_t d, float* partial,
                         int first_in_block, const float* w, const float* o, const float* lse1,
                         float eps, void* out, attnres_dtype out_dtype, float* lse,
                         const float* norm_gain, void* normed, hipStream_t stream) {
    return phase2_impl("attnres_block_phase2", v, v_dtype, T, d, partial, first_in_block, w,
                       nullptr, o, lse1, eps, out, out_dtype, lse, norm_gain, normed, stream);
}

int attnres_block_phase2_q(const void* v, attnres_dtype v_dtype, int64_t T, int64_t d,
                           float* partial, int first_in_block, const float* q, const float* o,
                           const float* lse1, float eps, void* out, attnres_dtype out_dtype,
                           float* lse, hipStream_t stream) {
    return phase2_impl("attnres_block_phase2_q", v, v_dtype, T, d, partial, first_in_block,
                       nullptr, q, o, lse1, eps, out, out_dtype, lse, nullptr, nullptr, stream);
}

size_t attnres_bwd_workspace_bytes(attnres_variant variant, int64_t S, int64_t n_hist, int64_t T,
                                   int64_t d, int64_t q_begin, int64_t n_q) {
    if (variant != ATTNRES_FULL && variant != ATTNRES_BLOCK) return 0;
    if (variant == ATTNRES_FULL) S = 1;
    if (S < 1 || n_hist < 1 || T < 0 || d < 1 || q_begin < 0 || n_q < 0 || q_begin + n_q > n_hist)
        return 0;
    if (S > n_hist) S = n_hist;
    return (size_t)attnres::bwd_layout(S, n_hist, T, d, n_q).bytes;
}

}  // extern "C"

namespace {

// attnres_bwd and attnres_bwd_noalloc; the latter passes use_scratch and no
// workspace, and takes the static device array instead
int bwd_impl(const char* fn, bool use_scratch, attnres_variant variant, int64_t S,
             const void* hist, attnres_dtype hist_dtype, int64_t n_hist, int64_t T, int64_t d,
             const float* w, int64_t q_begin, int64_t n_q, float eps, const void* dout,
             attnres_dtype dout_dtype, void* dhist, attnres_dtype dhist_dtype, int accumulate,
             float* dw, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (variant != ATTNRES_FULL && variant != ATTNRES_BLOCK)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad variant %d", fn, (int)variant);
    int st = check_common(fn, hist, hist_dtype, n_hist, T, d, w, q_begin, n_q, eps);
    if (st != ATTNRES_OK) return st;
    if (variant == ATTNRES_BLOCK && S < 1)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: S must be >= 1 (got %" PRId64 ")", fn, S);
    if (variant == ATTNRES_FULL) S = 1;
    if (S > n_hist) S = n_hist;  // S >= n_hist behaves like S = n_hist
    if (!valid_dtype(dout_dtype)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad dout dtype", fn);
    if (!valid_dtype(dhist_dtype)) return fail(ATTNRES_ERR_INVALID_ARG, "%s: bad dhist dtype", fn);
    if (accumulate != 0 && accumulate != 1)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: accumulate must be 0 or 1", fn);
    if (accumulate && dhist_dtype != ATTNRES_F32)
        return fail(ATTNRES_ERR_INVALID_ARG, "%s: accumulate needs an fp32 dhist", fn);
    if (T == 0) return ok();
    if (dhist == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: dhist is NULL", fn);
    if (!aligned(dhist, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: dhist is not 16-byte aligned", fn);
    if (n_q > 0) {
        if (dout == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: dout is NULL", fn);
        if (dw == nullptr) return fail(ATTNRES_ERR_INVALID_ARG, "%s: dw is NULL", fn);
        if (!aligned(dout, 16)) return fail(ATTNRES_ERR_ALIGN, "%s: dout is not 16-byte aligned", fn);
        if (!aligned(dw, 4)) return fail(ATTNRES_ERR_ALIGN, "%s: dw is not 4-byte aligned", fn);
    }
    const attnres::BwdLayout L = attnres::bwd_layout(S, n_hist, T, d, n_q);
    if (use_scratch && n_q > 0) {
        if (L.bytes > attnres::kBwdScratchBytes)
            return fail(ATTNRES_ERR_UNSUPPORTED,
                        "%s: needs %" PRId64 " bytes of workspace; the static scratch holds %" PRId64
                        " (split the call by tokens, or use attnres_bwd with a workspace)",
                        fn, L.bytes, attnres::kBwdScratchBytes);
        const hipError_t e = attnres::bwd_scratch(&workspace);
        if (e != hipSuccess) return hip_status(fn, e);
        workspace_bytes = (size_t)attnres::kBwdScratchBytes;
    }
    if (n_q > 0) {
        if (workspace == nullptr || workspace_bytes < (size_t)L.bytes)
            return fail(ATTNRES_ERR_WORKSPACE, "%s: workspace of %zu bytes, %" PRId64 " needed", fn,
                        workspace_bytes, L.bytes);
        if (!aligned(workspace, 256)) return fail(ATTNRES_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
    }

    attnres::BwdParams p;
    p.hist = hist;
    p.dout = dout;
    p.dhist = dhist;
    p.w = w;
    p.dw = dw;
    p.T = T;
    p.d = (int)d;
    p.nc = (int)(d / 8);
    p.n_hist = (int)n_hist;
    p.q_begin = (int)q_begin;
    p.n_q = (int)n_q;
    p.S = (int)S;
    p.nh8 = (int)L.nh8;
    p.nq8 = (int)L.nq8;
    p.n_blk = (int)L.n_blk;
    p.nx = (int)L.nx;
    p.accumulate = accumulate;
    p.eps = eps;
    p.inv_d = 1.0f / (float)d;
    p.hist_dt = hist_dtype;
    p.dout_dt = dout_dtype;
    p.dhist_dt = dhist_dtype;
    char* ws = static_cast<char*>(workspace);
    p.ws_a1 = reinterpret_cast<float*>(ws + L.off_a1);
    p.ws_a2 = reinterpret_cast<float*>(ws + L.off_a2);
    p.ws_a2t = reinterpret_cast<float*>(ws + L.off_a2t);
    p.ws_wsplit = reinterpret_cast<uint16_t*>(ws + L.off_wsplit);
    p.ws_c3 = reinterpret_cast<float*>(ws + L.off_c3);
    p.ws_kappa = reinterpret_cast<float*>(ws + L.off_kappa);
    p.ws_dwpart = reinterpret_cast<float*>(ws + L.off_dwpart);
    p.ws_dwstage = reinterpret_cast<float*>(ws + L.off_dwstage);
    p.ws_wsplit2 = reinterpret_cast<uint16_t*>(ws + L.off_wsplit2);
    if (n_q == 0) {
        // no read: every history row gets a zero gradient (nothing to add)
        if (accumulate) return ok();
        return hip_status(fn, attnres::launch_fill_zero(
                                  dhist, n_hist * T * d * (dhist_dtype == ATTNRES_BF16 ? 2 : 4), stream));
    }
    if (!attnres::bwd_fits(p))
        return fail(ATTNRES_ERR_UNSUPPORTED,
                    "%s: the per-read coefficients of %" PRId64 " sources (%" PRId64
                    " reads) do not fit one workgroup's LDS or one chunk's address range",
                    fn, L.nx, n_q);
    return hip_status(fn, attnres::launch_bwd(p, (int)L.n_chunks, (int)L.n_dw_groups, stream));
}

}  // namespace

extern "C" {

int attnres_bwd(attnres_variant variant, int64_t S, const void* hist, attnres_dtype hist_dtype,
                int64_t n_hist, int64_t T, int64_t d, const float* w, int64_t q_begin, int64_t n_q,
                float eps, const void* dout, attnres_dtype dout_dtype, void* dhist,
                attnres_dtype dhist_dtype, int accumulate, float* dw, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl("attnres_bwd", false, variant, S, hist, hist_dtype, n_hist, T, d, w, q_begin,
                    n_q, eps, dout, dout_dtype, dhist, dhist_dtype, accumulate, dw, workspace,
                    workspace_bytes, stream);
}

int attnres_bwd_noalloc(attnres_variant variant, int64_t S, const void* hist,
                        attnres_dtype hist_dtype, int64_t n_hist, int64_t T, int64_t d,
                        const float* w, int64_t q_begin, int64_t n_q, float eps, const void* dout,
                        attnres_dtype dout_dtype, void* dhist, attnres_dtype dhist_dtype,
                        int accumulate, float* dw, hipStream_t stream) {
    return bwd_impl("attnres_bwd_noalloc", true, variant, S, hist, hist_dtype, n_hist, T, d, w,
                    q_begin, n_q, eps, dout, dout_dtype, dhist, dhist_dtype, accumulate, dw,
                    nullptr, 0, stream);
}

size_t attnres_bwd_noalloc_max_workspace(void) { return (size_t)attnres::kBwdScratchBytes; }

}  // extern "C"
