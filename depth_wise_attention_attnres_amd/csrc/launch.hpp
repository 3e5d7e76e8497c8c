// launch.hpp -- internal interface between the C-ABI front end and the
// kernel launchers.  Not installed; callers use include/attnres.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attnres.h"

namespace attnres {

constexpr int kMaxD = 4096;
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
hipError_t launch_block_fwd(const BlockFwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                            hipStream_t stream);
// streaming Block kernel (one pass over rows 0..l per read, sums formed on the fly)
hipError_t launch_block_stream(const BlockFwdParams& p, hipStream_t stream);

}  // namespace attnres
