// block_model.hip -- Block AttnRes in model order on gfx950: the two phases of
// the pages' two-phase computation as separate calls (DataCamp, "two-phase
// computation"; block reading of "DepthBench reading notes" sec. 2.5).
//
// Phase 1 (once per block group, when block m completes): form the new source
// b_m = partial + v in fp32, then for the group's reads score the frozen
// sources b_0 .. b_m and write each read's normalised weighted sum o and its
// log-sum-exp lse1.  One workgroup per token; lane ln owns the 16-byte chunk
// ln of d and holds every source's chunk in registers, so each source is read
// once per call.  Reads go in chunks of four: per-lane partial dots, summed
// over 16-lane rows with DPP and across rows in LDS (double-buffered, one
// barrier per chunk); every wave then forms the softmax weights of the chunk
// (lane (k, c) = read k, source c) and fetches them with readlane for the
// outputs.
//
// Phase 2 (once per sublayer inside a block): partial += v, score the partial
// sum with the read's query and merge it with (o, lse1) by the log-sum-exp
// rule.  One wave per token, purely streaming.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

// the 8 elements of chunk `off` of a row, as fp32, for any stored dtype
__device__ __forceinline__ void load8(const void* row, attnres_dtype dt, int d, uint32_t chunk,
                                      bool ok, float (&x)[8]) {
    if (dt == ATTNRES_BF16) {
        const rsrc_t r = make_rsrc(row, (uint64_t)d * 2);
        Chunk<bf16_t> c;
        c.load(r, ok ? chunk * 16u : kOOB);
        c.to_float(x);
    } else {
        const rsrc_t r = make_rsrc(row, (uint64_t)d * 4);
        Chunk<float> c;
        c.load(r, ok ? chunk * 32u : kOOB);
        c.to_float(x);
    }
}

__device__ __forceinline__ void store8(void* row, attnres_dtype dt, int d, uint32_t chunk, bool ok,
                                       const float (&x)[8]) {
    if (dt == ATTNRES_BF16) {
        const rsrc_t r = make_rsrc(row, (uint64_t)d * 2);
        store_chunk((bf16_t*)nullptr, r, ok ? chunk * 16u : kOOB, x);
    } else {
        const rsrc_t r = make_rsrc(row, (uint64_t)d * 4);
        store_chunk((float*)nullptr, r, ok ? chunk * 32u : kOOB, x);
    }
}

}  // namespace

template <int NSRC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void block_phase1_kernel(Phase1Params p) {
    constexpr int CR = 4;                    // reads per chunk: one 16-lane row each
    constexpr int kSq = CR * NSRC;           // LDS slot of source c's squared norm: kSq + c
    constexpr int kVals = CR * NSRC + NSRC;
    static_assert(NSRC <= 16, "one lane per source in a 16-lane row");
    const int tid = threadIdx.x;
    const int row_slots = blockDim.x / 16, row_slot = tid >> 4;
    const int lane = tid & 63, kk = lane >> 4, cc = lane & 15;
    const int64_t t = blockIdx.x;
    const int64_t row_elems = p.T * (int64_t)p.d;
    const bool ok = tid < p.nc;
    const uint32_t chunk = (uint32_t)tid;
    const int m = p.n_src - 1;  // index of the new source (the last frozen one when v is null)
    const bool fresh = p.v != nullptr;  // a new source is formed here
    extern __shared__ float lds[];  // [2][kVals][row_slots], then [row_slots] for the pre-norm

    // ---- sources: the frozen ones, then the new one formed here -----------
    float src[NSRC][8];
#pragma unroll
    for (int c = 0; c < NSRC; ++c) {
        if (c < m || (c == m && !fresh)) {
            load8(p.blocks + c * row_elems + t * p.d, ATTNRES_F32, p.d, chunk, ok, src[c]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) src[c][e] = 0.f;
        }
    }
    if (fresh) {
        float x[8];
        load8(static_cast<const char*>(p.v) + t * p.d * (p.v_dt == ATTNRES_BF16 ? 2 : 4), p.v_dt, p.d,
              chunk, ok, x);
        if (p.partial != nullptr) {
            float q[8];
            load8(p.partial + t * p.d, ATTNRES_F32, p.d, chunk, ok, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = q[e] + x[e];
        }
#pragma unroll
        for (int c = 0; c < NSRC; ++c)
            if (c == m)
#pragma unroll
                for (int e = 0; e < 8; ++e) src[c][e] = x[e];
        store8(p.blocks + m * row_elems + t * p.d, ATTNRES_F32, p.d, chunk, ok, x);
    }

    float rsv = 0.f;  // RMS scale of source cc (every wave keeps its own copy)
    int buf = 0;
    for (int k0 = 0; k0 < p.n_reads; k0 += CR) {
        const int n = p.n_reads - k0 < CR ? p.n_reads - k0 : CR;
        float* part = lds + buf * kVals * row_slots;
        // ---- per-lane dots, summed over 16-lane rows, into LDS -------------
#pragma unroll
        for (int k = 0; k < CR; ++k) {
            if (k < n) {
                float wv[8];
                const float* wrow = p.qtok != nullptr ? p.qtok + ((int64_t)(k0 + k) * p.T + t) * p.d
                                                      : p.w + (int64_t)(k0 + k) * p.d;
                load8(wrow, ATTNRES_F32, p.d, chunk, ok, wv);
                float v[NSRC];
#pragma unroll
                for (int c = 0; c < NSRC; ++c) {
                    float dp = 0.f;
                    if (c <= m)
#pragma unroll
                        for (int e = 0; e < 8; ++e) dp = fmaf(wv[e], src[c][e], dp);
                    v[c] = dp;
                }
#pragma unroll
                for (int c = 0; c < NSRC; ++c)
                    if (c <= m) v[c] = tg_sum<16>(v[c]);
#pragma unroll
                for (int c = 0; c < NSRC; ++c)
                    if (c <= m) part[(k * NSRC + c) * row_slots + row_slot] = v[c];
            }
        }
        if (k0 == 0) {  // squared norms of the sources whose scale is not cached
#pragma unroll
            for (int c = 0; c < NSRC; ++c) {
                if (c <= m && (p.rs == nullptr || (c == m && fresh))) {
                    float sq = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) sq = fmaf(src[c][e], src[c][e], sq);
                    sq = tg_sum<16>(sq);
                    part[(kSq + c) * row_slots + row_slot] = sq;
                }
            }
        }
        __syncthreads();

        // ---- softmax weights of the chunk, in every wave ----------------------
        auto total = [&](int idx) {
            const f32x4* q = reinterpret_cast<const f32x4*>(part + idx * row_slots);
            float s = 0.f;
            for (int r = 0; r < row_slots / 4; ++r) {
                const f32x4 a = q[r];
                s += a[0];
                s += a[1];
                s += a[2];
                s += a[3];
            }
            return s;
        };
        if (k0 == 0 && cc <= m) {
            if (p.rs != nullptr && (cc < m || !fresh))
                rsv = p.rs[(int64_t)cc * p.T + t];
            else
                rsv = fast_rsqrt(fmaf(total(kSq + cc), p.inv_d, p.eps));
            if (p.rs != nullptr && fresh && cc == m && kk == 0 && tid == lane)
                p.rs[(int64_t)m * p.T + t] = rsv;
        }
        const bool live = kk < n && cc <= m;
        const float s2 = live ? rsv * total(kk * NSRC + cc) * kLog2e : -INFINITY;
        const float M = tg_max<16>(s2);
        const float e = live ? fast_exp2(s2 - M) : 0.f;
        const float Z = tg_sum<16>(e);
        const float coef = e / Z;
        if (kk < n && cc == 0 && tid == lane) {  // wave 0 stores the log-sum-exp
            const float l1 = (M + fast_log2(Z)) * kLn2;
            p.lse1[(int64_t)(k0 + kk) * p.T + t] = l1;
            if (k0 + kk == 0 && p.lse0 != nullptr) p.lse0[t] = l1;
        }
        buf ^= 1;

        // ---- outputs -----------------------------------------------------------
#pragma unroll
        for (int k = 0; k < CR; ++k) {
            if (k < n) {
                float o[8];
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) o[e2] = 0.f;
#pragma unroll
                for (int c = 0; c < NSRC; ++c) {
                    if (c <= m) {
                        const float a = __int_as_float(
                            __builtin_amdgcn_readlane(__float_as_int(coef), 16 * k + c));
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) o[e2] = fmaf(a, src[c][e2], o[e2]);
                    }
                }
                store8(p.o + (int64_t)(k0 + k) * row_elems + t * p.d, ATTNRES_F32, p.d, chunk, ok, o);
                if (k0 + k == 0 && p.out0 != nullptr)
                    store8(static_cast<char*>(p.out0) + t * p.d * (p.out_dt == ATTNRES_BF16 ? 2 : 4),
                           p.out_dt, p.d, chunk, ok, o);
                if (k0 + k == 0 && p.normed0 != nullptr) {  // uniform: every thread takes it
                    float* red = lds + 2 * kVals * row_slots;
                    float ss = 0.f;
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) ss = fmaf(o[e2], o[e2], ss);
                    ss = tg_sum<16>(ss);
                    red[row_slot] = ss;
                    __syncthreads();
                    float tot = 0.f;
                    for (int r = 0; r < row_slots; ++r) tot += red[r];
                    const float rn = fast_rsqrt(fmaf(tot, p.inv_d, p.eps));
                    float g[8];
                    if (p.norm_gain0 != nullptr) {
                        load8(p.norm_gain0, ATTNRES_F32, p.d, chunk, ok, g);
                    } else {
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) g[e2] = 1.f;
                    }
                    float y[8];
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) y[e2] = g[e2] * (o[e2] * rn);
                    store8(static_cast<char*>(p.normed0) + t * p.d * (p.out_dt == ATTNRES_BF16 ? 2 : 4),
                           p.out_dt, p.d, chunk, ok, y);
                }
            }
        }
    }
}

// one wave per token, NCH chunks of 8 elements per lane
template <int NCH>
__global__ __launch_bounds__(256) void block_phase2_kernel(Phase2Params p) {
    const int ln = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= p.T) return;  // whole waves leave together
    const int vb = p.v_dt == ATTNRES_BF16 ? 2 : 4;
    const int ob = p.out_dt == ATTNRES_BF16 ? 2 : 4;
    const void* v_row = static_cast<const char*>(p.v) + t * p.d * vb;
    float* part_row = p.partial + t * p.d;
    const float* o_row = p.o + t * p.d;
    void* out_row = static_cast<char*>(p.out) + t * p.d * ob;

    float x[NCH][8], o[NCH][8];
    float dot = 0.f, sq = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const uint32_t ch = (uint32_t)(c * 64 + ln);
        const bool ok = (int)ch < p.nc;
        load8(v_row, p.v_dt, p.d, ch, ok, x[c]);
        if (!p.first) {
            float q[8];
            load8(part_row, ATTNRES_F32, p.d, ch, ok, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[c][e] = q[e] + x[c][e];
        }
        float wv[8];
        load8(p.qtok != nullptr ? p.qtok + t * p.d : p.w, ATTNRES_F32, p.d, ch, ok, wv);
        load8(o_row, ATTNRES_F32, p.d, ch, ok, o[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dot = fmaf(wv[e], x[c][e], dot);
            sq = fmaf(x[c][e], x[c][e], sq);
        }
        store8(part_row, ATTNRES_F32, p.d, ch, ok, x[c]);
    }
    dot = tg_sum<64>(dot);
    sq = tg_sum<64>(sq);
    const float sp = fast_rsqrt(fmaf(sq, p.inv_d, p.eps)) * dot * kLog2e;  // log2 units
    const float l1 = p.lse1[t] * kLog2e;
    const float M = fmaxf(l1, sp);
    const float A = fast_exp2(l1 - M), B = fast_exp2(sp - M);
    const float inv = 1.0f / (A + B);
    const float a = A * inv, b = B * inv;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const uint32_t ch = (uint32_t)(c * 64 + ln);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[c][e] = fmaf(a, o[c][e], b * x[c][e]);  // o now holds h
            ss = fmaf(o[c][e], o[c][e], ss);
        }
        store8(out_row, p.out_dt, p.d, ch, (int)ch < p.nc, o[c]);
    }
    if (p.lse != nullptr && ln == 0) p.lse[t] = (M + fast_log2(A + B)) * kLn2;
    if (p.normed != nullptr) {  // fused pre-norm of the output (uniform branch)
        ss = tg_sum<64>(ss);
        const float rn = fast_rsqrt(fmaf(ss, p.inv_d, p.eps));
        void* n_row = static_cast<char*>(p.normed) + t * p.d * ob;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t ch = (uint32_t)(c * 64 + ln);
            float g[8];
            if (p.norm_gain != nullptr) {
                load8(p.norm_gain, ATTNRES_F32, p.d, ch, (int)ch < p.nc, g);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) g[e] = 1.f;
            }
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = g[e] * (o[c][e] * rn);
            store8(n_row, p.out_dt, p.d, ch, (int)ch < p.nc, y);
        }
    }
}

hipError_t launch_block_phase1(const Phase1Params& p, hipStream_t stream) {
    const int nw = p.nc <= 64 ? 1 : p.nc <= 128 ? 2 : p.nc <= 256 ? 4 : 8;
    auto lds = [&](int nsrc) { return sizeof(float) * (2 * (size_t)(4 * nsrc + nsrc) + 1) * 4 * nw; };
    if (p.n_src <= 5)
        hipLaunchKernelGGL(block_phase1_kernel<5>, dim3((unsigned)p.T), dim3(64 * nw), lds(5), stream, p);
    else if (p.n_src <= 9)
        hipLaunchKernelGGL(block_phase1_kernel<9>, dim3((unsigned)p.T), dim3(64 * nw), lds(9), stream, p);
    else
        hipLaunchKernelGGL(block_phase1_kernel<13>, dim3((unsigned)p.T), dim3(64 * nw), lds(13), stream, p);
    return hipGetLastError();
}

hipError_t launch_block_phase2(const Phase2Params& p, hipStream_t stream) {
    const unsigned blocks = (unsigned)((p.T + 3) / 4);
    switch ((p.nc + 63) / 64) {
        case 1: hipLaunchKernelGGL(block_phase2_kernel<1>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 2: hipLaunchKernelGGL(block_phase2_kernel<2>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 3: hipLaunchKernelGGL(block_phase2_kernel<3>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 4: hipLaunchKernelGGL(block_phase2_kernel<4>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 5: hipLaunchKernelGGL(block_phase2_kernel<5>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 6: hipLaunchKernelGGL(block_phase2_kernel<6>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 7: hipLaunchKernelGGL(block_phase2_kernel<7>, dim3(blocks), dim3(256), 0, stream, p); break;
        case 8: hipLaunchKernelGGL(block_phase2_kernel<8>, dim3(blocks), dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attnres
