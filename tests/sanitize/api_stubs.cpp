// Host-only stand-ins for the kernel launchers and the two HIP error-string
// functions, so that the C front end (attnres_api.cpp) can be built with
// AddressSanitizer / UndefinedBehaviorSanitizer and driven on a CPU: every
// launcher records that it was reached and returns success.  Test code only.
#include <hip/hip_runtime.h>

#include "launch.hpp"

int g_launches = 0;
alignas(256) static unsigned char g_scratch_stand_in[256];

extern "C" const char* hipGetErrorName(hipError_t) { return "hipErrorStub"; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace attnres {

BwdLayout bwd_layout(int64_t S, int64_t n_hist, int64_t T, int64_t d, int64_t n_q) {
    // sizes only matter to the front end's own comparisons
    BwdLayout L{};
    L.nh8 = (n_hist + 7) / 8 * 8;
    L.nq8 = (n_q + 7) / 8 * 8;
    L.n_blk = 1 + (n_hist - 1 + S - 1) / S;
    L.nx = 1 + (n_hist - 1) / S + 1;
    L.n_chunks = (T + 31) / 32;
    L.n_dw_groups = L.n_chunks < 16 ? L.n_chunks : 16;
    L.bytes = 256 * (1 + T * n_q * L.nh8 * 8 / 256 + n_q * d * 4 / 256);
    return L;
}
hipError_t launch_full_fwd(const FwdParams&, attnres_dtype, attnres_dtype, hipStream_t) { ++g_launches; return hipSuccess; }
// split calls with many reads, so that the split path's offsets run under the sanitizers
int full_batch_mfma_prefix(const FwdParams& p, attnres_dtype, attnres_dtype) {
    return p.n_q >= 32 && p.qtok == nullptr && p.normed == nullptr ? p.n_q / 2 : 0;
}
hipError_t launch_block_fwd(const FwdParams&, attnres_dtype, attnres_dtype, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_query_proj(const void*, const void*, float*, int64_t, int64_t, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_block_phase1(const Phase1Params&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_block_phase2(const Phase2Params&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd(const BwdParams&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fill_zero(void*, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
bool bwd_fits(const BwdParams& p) { return p.nx < 4096; }
hipError_t bwd_scratch(void** ptr) {
    *ptr = g_scratch_stand_in;
    return hipSuccess;
}

}  // namespace attnres
