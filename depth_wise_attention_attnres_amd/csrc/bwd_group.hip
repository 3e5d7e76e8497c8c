// bwd_group.hip -- the per-read coefficients of the Block AttnRes backward for
// calls with many reads, one wave per block group, on gfx950.
//
// For each token and read l with sources x (v_0, the block sums b_1..b_m and,
// when l mod S != 0, the partial sum p_l), the backward needs the softmax
// weights alpha_x, the gradient dots a_x = g_l . x, delta = sum_x alpha_x a_x
// and ds_x = alpha_x (a_x - delta); from them the coefficient tables the
// dhist and dw kernels consume (see bwd.hip): A1 = alpha and A2 = ds r of the
// source holding each row (row-major and transposed), C3 = sum over reads of
// ds r^2 s / d per frozen source, kappa = ds r^2 s / d of each read's partial
// sum.  The streaming kernel in bwd.hip re-forms the sources from the rows
// once per pass of a few reads; here, as in the Block forward for many reads
// (block_batch.hip), one workgroup per token forms the frozen fp32 sources
// once into LDS and each wave takes whole block groups, streaming the group's
// rows again for the partial sums and reading each read's dout row once.
// C3 is summed over reads in read order from a per-read LDS table, so the
// result does not depend on which wave took which group.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

constexpr int kBgWaves = 8;
constexpr int kBgMinReads = 16;
constexpr int kBgMaxSources = 13;  // v_0 + completed blocks a read of the call sees

// LDS: sources [nb][srow] fp32, their RMS scales [nbp], per-read C3 [n_q][nbp],
// counter.  A source row holds, per 64-lane chunk group c2, two planes of
// [64 lanes][4 floats] (elements 0-3 and 4-7 of each lane's 8): a lane's
// 16-byte reads are then 16 bytes apart across the wave, free of bank
// conflicts (8 contiguous floats per lane would put lanes 8 apart on the same
// banks).
__host__ __device__ inline int bg_nbp(int nb) { return (nb + 3) & ~3; }
__host__ __device__ inline int bg_srow(int nc) { return (nc + 63) / 64 * 512; }
__host__ __device__ inline int64_t bg_lds_bytes(int nb, int nc, int n_q) {
    return (int64_t)nb * bg_srow(nc) * 4 + (int64_t)bg_nbp(nb) * 4 + (int64_t)n_q * bg_nbp(nb) * 4 + 16;
}
// the two planes of lane ln's 8 elements of chunk group c2 in a source row
__device__ __forceinline__ void bg_src_read(const float* row, int c2, int ln, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + (2 * c2) * 256 + 4 * ln);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + (2 * c2 + 1) * 256 + 4 * ln);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        x[q] = a[q];
        x[4 + q] = b[q];
    }
}

struct BgLane {
    bool live[4];
    uint32_t h_off[4], g_off[4], w_off[4];
};

// The reads la..lb of block group G (la >= G S).
template <typename TG, int NCH, int G>
__device__ __forceinline__ void bg_group(const BwdParams& p, const float* src, const float* rsv,
                                         float* c3r, int nbp, const bf16_t* hist_tok, const TG* dout_tok,
                                         int64_t t, int ln, const BgLane& q, int la, int lb) {
    constexpr int kW = G + 1;       // frozen sources
    constexpr int kV = 2 * kW + 3;  // w.x and g.x per frozen source; w.p, g.p, p.p
    const int d = p.d, S = p.S;
    const int64_t row_elems = p.T * (int64_t)d;
    const int g0 = G * S;

    float part[NCH][8];
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[c2][e] = 0.f;
    auto add_row = [&](const Chunk<bf16_t> (&r)[NCH]) {
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
            float x[8];
            r[c2].to_float(x);
#pragma unroll
            for (int e = 0; e < 8; ++e) part[c2][e] += x[e];
        }
    };
    auto issue_row = [&](Chunk<bf16_t> (&r)[NCH], int i) {
        const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, (uint64_t)d * 2);
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) r[c2].load(rr, q.h_off[c2]);
    };
    // rows g0+1 .. la-1 of the partial sum before the first read, four at a time
    for (int i0 = g0 + 1; i0 < la; i0 += 4) {
        Chunk<bf16_t> cb[4][NCH];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u < la) issue_row(cb[u], i0 + u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u < la) add_row(cb[u]);
    }
    Chunk<bf16_t> rl[NCH];  // row l of the current read, in flight
    if (la > g0) issue_row(rl, la);
    Chunk<float> wq[NCH];   // query and upstream gradient of the current read, in flight
    Chunk<TG> gq[NCH];
    auto issue_wg = [&](int l) {
        const int lq = l - p.q_begin;
        const rsrc_t wr = make_rsrc(p.w + (int64_t)lq * d, (uint64_t)d * 4);
        const rsrc_t gr = make_rsrc(dout_tok + (int64_t)lq * row_elems, (uint64_t)d * sizeof(TG));
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
            wq[c2].load(wr, q.w_off[c2]);
            gq[c2].load(gr, q.g_off[c2]);
        }
    };
    issue_wg(la);

    for (int l = la; l <= lb; ++l) {
        const int lq = l - p.q_begin;
        float wv[NCH][8], gv[NCH][8];
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
            wq[c2].to_float(wv[c2]);
            gq[c2].to_float(gv[c2]);
        }
        const bool has_p = l > g0;
        if (has_p) add_row(rl);
        if (l < lb) issue_row(rl, l + 1);

        float v[kV];
#pragma unroll
        for (int j = 0; j < kV; ++j) v[j] = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
            if (!q.live[c2]) continue;
#pragma unroll
            for (int c = 0; c < kW; ++c) {
                float x[8];
                bg_src_read(src + c * NCH * 512, c2, ln, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[c] = fmaf(wv[c2][e], x[e], v[c]);
                    v[kW + c] = fmaf(gv[c2][e], x[e], v[kW + c]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[2 * kW] = fmaf(wv[c2][e], part[c2][e], v[2 * kW]);
                v[2 * kW + 1] = fmaf(gv[c2][e], part[c2][e], v[2 * kW + 1]);
                v[2 * kW + 2] = fmaf(part[c2][e], part[c2][e], v[2 * kW + 2]);
            }
        }
        if (l < lb) issue_wg(l + 1);
        float tot[kV];
        wave_totals<0, kV>(v, tot, ln);

        // sources of the read in order: v_0, b_1..b_G, then the partial sum
        float s[kW + 1], a[kW + 1], r[kW + 1];
#pragma unroll
        for (int c = 0; c < kW; ++c) {
            r[c] = rsv[c];
            s[c] = r[c] * tot[c];
            a[c] = tot[kW + c];
        }
        r[kW] = fast_rsqrt(fmaf(tot[2 * kW + 2], p.inv_d, p.eps));
        s[kW] = r[kW] * tot[2 * kW];
        a[kW] = tot[2 * kW + 1];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < kW; ++c) mx = fmaxf(mx, s[c]);
        if (has_p) mx = fmaxf(mx, s[kW]);
        float al[kW + 1];
        float z = 0.f;
#pragma unroll
        for (int c = 0; c <= kW; ++c) {
            al[c] = (c < kW || has_p) ? fast_exp2((s[c] - mx) * kLog2e) : 0.f;
            z += al[c];
        }
        const float inv_z = 1.0f / z;
        float delta = 0.f;
#pragma unroll
        for (int c = 0; c <= kW; ++c) {
            al[c] *= inv_z;
            delta = fmaf(al[c], a[c], delta);
        }
        float c1[kW + 1], c2v[kW + 1];
#pragma unroll
        for (int c = 0; c <= kW; ++c) {
            const float ds = al[c] * (a[c] - delta);
            c1[c] = al[c];
            c2v[c] = ds * r[c];
            const float c3 = ds * r[c] * r[c] * s[c] * p.inv_d;
            if (c < kW) {
                if (ln == c) c3r[(int64_t)lq * nbp + c] = c3;  // frozen source c
            } else if (ln == 0) {
                p.ws_kappa[t * p.n_q + lq] = has_p ? c3 : 0.f;   // the partial sum, or none
            }
        }

        // coefficient rows of the read: the source holding each row i <= l
        float* A1 = p.ws_a1 + (t * (int64_t)p.n_q + lq) * p.nh8;
        float* A2 = p.ws_a2 + (t * (int64_t)p.n_q + lq) * p.nh8;
        float* A2T = p.ws_a2t + t * (int64_t)p.n_hist * p.nq8 + lq;
        for (int i = ln; i < p.nh8; i += 64) {
            float e1 = 0.f, e2 = 0.f;
            if (i <= l) {
                const int blk = i == 0 ? 0 : (i - 1) / S + 1;
                const int xs = blk <= G ? blk : kW;  // a frozen source, or the partial sum
#pragma unroll
                for (int c = 0; c <= kW; ++c)
                    if (xs == c) {
                        e1 = c1[c];
                        e2 = c2v[c];
                    }
            }
            A1[i] = e1;
            A2[i] = e2;
            if (i < p.n_hist) A2T[(int64_t)i * p.nq8] = e2;
        }
    }
}

template <typename TG, int NCH, int NBMAX, int G = 0>
__device__ __forceinline__ void bg_dispatch(int g, const BwdParams& p, const float* src, const float* rsv,
                                            float* c3r, int nbp, const bf16_t* hist_tok, const TG* dout_tok,
                                            int64_t t, int ln, const BgLane& q, int la, int lb) {
    if constexpr (G < NBMAX) {
        if (g == G)
            bg_group<TG, NCH, G>(p, src, rsv, c3r, nbp, hist_tok, dout_tok, t, ln, q, la, lb);
        else
            bg_dispatch<TG, NCH, NBMAX, G + 1>(g, p, src, rsv, c3r, nbp, hist_tok, dout_tok, t, ln, q,
                                               la, lb);
    }
}

template <typename TG, int NCH, int NBMAX>
__global__ __launch_bounds__(64 * kBgWaves) void bwd_scores_group_kernel(BwdParams p, int nb) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int nbp = bg_nbp(nb);
    float* const src = reinterpret_cast<float*>(lds_raw);
    float* const rsv = src + (int64_t)nb * NCH * 512;
    float* const c3r = rsv + nbp;  // [n_q][nbp]: slot c of read lq = its C3 term for source c
    int* const counter = reinterpret_cast<int*>(c3r + (int64_t)p.n_q * nbp);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = threadIdx.x & 63;
    const int64_t t = blockIdx.x;
    const int d = p.d, S = p.S;
    const int64_t row_elems = p.T * (int64_t)d;
    const bf16_t* hist_tok = static_cast<const bf16_t*>(p.hist) + t * d;
    const TG* dout_tok = static_cast<const TG*>(p.dout) + t * d;

    BgLane q;
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
        const int ch = c2 * 64 + ln;
        q.live[c2] = c2 < NCH && ch < p.nc;
        q.h_off[c2] = q.live[c2] ? (uint32_t)(ch * 16) : kOOB;
        q.g_off[c2] = q.live[c2] ? (uint32_t)(ch * 8 * sizeof(TG)) : kOOB;
        q.w_off[c2] = q.live[c2] ? (uint32_t)(ch * 32) : kOOB;
    }
    if (threadIdx.x == 0) *counter = 0;
    // per-read C3 slots start at zero (a read writes its frozen sources only)
    for (int i = threadIdx.x; i < p.n_q * nbp; i += blockDim.x) c3r[i] = 0.f;
    // the padding reads n_q .. nq8-1 of A2T are zero
    float* const A2T = p.ws_a2t + t * (int64_t)p.n_hist * p.nq8;
    if (p.nq8 > p.n_q)
        for (int k = threadIdx.x; k < p.n_hist * (p.nq8 - p.n_q); k += blockDim.x)
            A2T[(int64_t)(k / (p.nq8 - p.n_q)) * p.nq8 + p.n_q + k % (p.nq8 - p.n_q)] = 0.f;

    // ---- prologue: frozen sources v_0, b_1, ... in fp32, their RMS scales ------
    for (int c = wave; c < nb; c += kBgWaves) {
        const int i0 = c == 0 ? 0 : (c - 1) * S + 1;
        const int i1 = c == 0 ? 0 : c * S;  // inclusive; c * S <= last read < n_hist
        float acc[NCH][8];
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[c2][e] = 0.f;
        for (int ib = i0; ib <= i1; ib += 4) {
            Chunk<bf16_t> ch[4][NCH];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (ib + u <= i1) {
                    const rsrc_t rr = make_rsrc(hist_tok + (ib + u) * row_elems, (uint64_t)d * 2);
#pragma unroll
                    for (int c2 = 0; c2 < NCH; ++c2) ch[u][c2].load(rr, q.h_off[c2]);
                }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (ib + u <= i1) {
#pragma unroll
                    for (int c2 = 0; c2 < NCH; ++c2) {
                        float x[8];
                        ch[u][c2].to_float(x);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[c2][e] += x[e];
                    }
                }
        }
        float sq = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sq = fmaf(acc[c2][e], acc[c2][e], sq);
            if (q.live[c2]) {
                float* dst = src + c * NCH * 512 + (2 * c2) * 256 + 4 * ln;
                *reinterpret_cast<f32x4*>(dst) = f32x4{acc[c2][0], acc[c2][1], acc[c2][2], acc[c2][3]};
                *reinterpret_cast<f32x4*>(dst + 256) = f32x4{acc[c2][4], acc[c2][5], acc[c2][6], acc[c2][7]};
            }
        }
        sq = tg_sum<64>(sq);
        if (ln == 0) rsv[c] = fast_rsqrt(fmaf(sq, p.inv_d, p.eps));
    }
    __syncthreads();

    // ---- block groups, latest group first --------------------------------------
    const int l_last = p.q_begin + p.n_q - 1;
    const int g_last = l_last / S;
    for (;;) {
        int u = 0;
        if (ln == 0) u = atomicAdd(counter, 1);
        u = __builtin_amdgcn_readfirstlane(u);
        if (u > g_last) break;
        const int g = g_last - u;
        int la = g * S;
        int lb = g * S + S - 1;
        if (la < p.q_begin) la = p.q_begin;
        if (lb > l_last) lb = l_last;
        if (la > lb) continue;
        bg_dispatch<TG, NCH, NBMAX>(g, p, src, rsv, c3r, nbp, hist_tok, dout_tok, t, ln, q, la, lb);
    }
    __syncthreads();

    // C3 per source: the reads' contributions summed in read order
    for (int b = threadIdx.x; b < p.n_blk; b += blockDim.x) {
        float c3 = 0.f;
        if (b < nb)
            for (int lq = 0; lq < p.n_q; ++lq) c3 += c3r[(int64_t)lq * nbp + b];
        p.ws_c3[t * p.n_blk + b] = c3;
    }
}

template <typename TG, int NCH>
hipError_t launch_bg_nch(const BwdParams& p, int nb, size_t lds, hipStream_t stream) {
    auto go = [&](auto kern) {
        const hipError_t e = prepare_dynamic_lds((const void*)kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)p.T), dim3(64 * kBgWaves), lds, stream, p, nb);
        return hipGetLastError();
    };
    if (nb <= 9) return go(bwd_scores_group_kernel<TG, NCH, 9>);
    return go(bwd_scores_group_kernel<TG, NCH, kBgMaxSources>);
}

template <typename TG>
hipError_t launch_bg(const BwdParams& p, int nb, size_t lds, hipStream_t stream) {
    switch ((p.nc + 63) / 64) {
        case 1: return launch_bg_nch<TG, 1>(p, nb, lds, stream);
        case 2: return launch_bg_nch<TG, 2>(p, nb, lds, stream);
        default: return hipErrorInvalidValue;
    }
}

int bg_sources(const BwdParams& p, size_t* lds) {
    if (p.hist_dt != ATTNRES_BF16 || p.S < 2 || p.n_q < kBgMinReads || p.nc > 2 * 64) return 0;
    if (p.T * 64 * kBgWaves >= ((int64_t)1 << 32)) return 0;
    const int nb = 1 + (p.q_begin + p.n_q - 1) / p.S;
    if (nb > kBgMaxSources) return 0;
    const int max_lds = device_max_lds();
    const int64_t bytes = bg_lds_bytes(nb, p.nc, p.n_q);
    if (bytes > max_lds) return 0;
    *lds = (size_t)bytes;
    return nb;
}

}  // namespace

bool bwd_scores_group_applies(const BwdParams& p) {
    size_t lds = 0;
    return bg_sources(p, &lds) > 0;
}

hipError_t launch_bwd_scores_group(const BwdParams& p, hipStream_t stream) {
    size_t lds = 0;
    const int nb = bg_sources(p, &lds);
    if (nb == 0) return hipErrorInvalidValue;
    return p.dout_dt == ATTNRES_BF16 ? launch_bg<bf16_t>(p, nb, lds, stream)
                                     : launch_bg<float>(p, nb, lds, stream);
}

}  // namespace attnres
