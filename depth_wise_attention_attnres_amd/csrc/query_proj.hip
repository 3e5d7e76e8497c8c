// query_proj.hip -- the input-dependent query of the AttnRes ablation ("Kimi K3
// notes 2", sec. 6: a d x d projection of the current hidden state replaces
// the learned per-read query): q[j][t] = W[j] x[j][t] for every read j and
// token t.  A dense contraction over d, on the matrix cores:
// v_mfma_f32_32x32x16_bf16, D[32 tokens x 32 outputs] += A B with
//   A[i][k] = x[token t0 + i][k]   (lane j: token j % 32, k = 8 (j / 32) .. + 7)
//   B[k][n] = W[output o0 + n][k]  (lane j: output j % 32, same k)
// so both operands are 16-byte loads contiguous in k.  bf16 x bf16 products
// are exact in fp32; the accumulators are folded into fp32 totals every 16
// steps.  One wave per 32 x 32 tile, four waves (a 64 x 64 tile) per
// workgroup; operands are fetched two steps ahead.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t ld8(const bf16_t* ptr, bool ok) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(ptr);
    return __builtin_bit_cast(bf16x8_t, v);
}
}  // namespace

__global__ __launch_bounds__(256) void query_proj_kernel(const bf16_t* x, const bf16_t* W, float* q,
                                                         int64_t T, int d, int tiles_t, int tiles_o) {
    const int wave = threadIdx.x >> 6, ln = threadIdx.x & 63;
    const int h = ln >> 5, m = ln & 31;
    // blockIdx.x = (read j, token tile, output tile), output tiles fastest so
    // that the workgroups sharing a token tile run together and reuse it in L2
    const int64_t b = blockIdx.x;
    const int to = (int)(b % tiles_o);
    const int64_t rest = b / tiles_o;
    const int tt = (int)(rest % tiles_t);
    const int64_t j = rest / tiles_t;
    const int64_t t0 = (int64_t)tt * 64 + 32 * (wave >> 1);
    const int o0 = to * 64 + 32 * (wave & 1);

    const int64_t tok = t0 + m;
    const bool tok_ok = tok < T;
    const int out = o0 + m;
    const bool out_ok = out < d;
    const bf16_t* xp = x + (j * T + (tok_ok ? tok : 0)) * d + 8 * h;
    const bf16_t* wp = W + (j * d + (out_ok ? out : 0)) * (int64_t)d + 8 * h;

    constexpr int kFold = 16, kPD = 2;
    f32x16 acc, tot;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = tot[r] = 0.f;
    bf16x8_t ra[kPD], rb[kPD];
    const int n_steps = (d + 15) / 16;
    auto fetch = [&](int u, int st) {
        const bool kok = 16 * st + 8 * h < d;  // d % 8 == 0: all eight or none
        ra[u] = ld8(xp + 16 * st, tok_ok && kok);
        rb[u] = ld8(wp + 16 * st, out_ok && kok);
    };
#pragma unroll
    for (int u = 0; u < kPD; ++u)
        if (u < n_steps) fetch(u, u);
    for (int s0 = 0; s0 < n_steps; s0 += kPD) {
#pragma unroll
        for (int u = 0; u < kPD; ++u) {
            const int st = s0 + u;
            if (st >= n_steps) break;
            const bf16x8_t a = ra[u], bb = rb[u];
            if (st + kPD < n_steps) fetch(u, st + kPD);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
            if ((st + 1) % kFold == 0 || st + 1 == n_steps) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    tot[r] += acc[r];
                    acc[r] = 0.f;
                }
            }
        }
    }
    // lane j, register r holds D[i][n = m]: token t0 + i, output o0 + m,
    // i = 8 (r / 4) + 4 h + r % 4
    if (out_ok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t ti = t0 + 8 * (r / 4) + 4 * h + r % 4;
            if (ti < T) q[(j * T + ti) * d + out] = tot[r];
        }
    }
}

hipError_t launch_query_proj(const void* x, const void* W, float* q, int64_t n_q, int64_t T, int d,
                             hipStream_t stream) {
    const int tiles_t = (int)((T + 63) / 64);
    const int tiles_o = (d + 63) / 64;
    const int64_t blocks = n_q * tiles_t * (int64_t)tiles_o;
    hipLaunchKernelGGL(query_proj_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), q, T, d,
                       tiles_t, tiles_o);
    return hipGetLastError();
}

}  // namespace attnres
