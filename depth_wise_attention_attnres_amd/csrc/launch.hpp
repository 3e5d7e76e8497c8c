// launch.hpp -- internal interface between the C-ABI front end and the
// kernel launchers.  Not installed; callers use include/attnres.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attnres.h"

namespace attnres {

constexpr int kMaxD = 4096;

struct FullFwdParams {
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
    float eps;
    float inv_d;
};

hipError_t launch_full_fwd(const FullFwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                           hipStream_t stream);

}  // namespace attnres
