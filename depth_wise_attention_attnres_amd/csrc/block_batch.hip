// block_batch.hip -- Block AttnRes forward for calls with many reads, one wave
// per group of reads, on gfx950.
//
// Block reading ("DepthBench reading notes" sec. 2.5; DataCamp, block
// section): read l with m = floor(l / S) attends over v_0, the completed block
// sums b_1..b_m and, when l mod S != 0, the partial sum p_l of rows mS+1..l.
//
// The two-phase kernel (block_fwd.hip) gives each of a token's waves a slice
// of d and runs every read in every wave, so the per-read work that does not
// scale with d -- the reductions of the dots, the softmax, the loop -- is paid
// once per wave.  Here one wave owns all of d for a group of reads:
//   prologue  the workgroup (one per token) forms the frozen sources v_0,
//             b_1, b_2, ... in fp32 from the raw rows, stores them in LDS and
//             forms their RMS scales;
//   groups    the waves take block groups g (reads gS .. gS+S-1) from a
//             workgroup counter, latest group first.  A group streams its rows
//             gS+1.. again (the prologue read them) to form each read's partial
//             sum in registers, and for every read: the dots of
//             its query with the frozen sources (from LDS) and with the partial
//             sum, one transposing wave reduction of all of them, the exact
//             softmax over [frozen sources, partial] (equal to the two-phase
//             merge), and the weighted sum, rounded once and stored.
// Lane `ln` owns the 16-byte chunks ln, ln + 64, ... of d.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

constexpr int kBbWaves = 8;
constexpr int kBbMinReads = 16;
constexpr int kBbMaxSources = 13;  // v_0 + completed blocks a read of the call sees

// LDS: the frozen sources in fp32, then their RMS scales [NBMAX] and the
// group counter.  Element e of 16-byte chunk ch = 64 c2 + ln of source c sits
// at float ((e / 4) NCH + c2) NBMAX + c) 256 + 4 ln + e % 4: every offset past
// the lane's base is a compile-time constant (an immediate of the LDS
// instruction, no address register per source), and a wave's 16-byte reads and
// writes cover 1 KB of consecutive bytes (no bank conflicts).
template <int NCH, int NBMAX>
struct BbLds {
    static constexpr int kSrcFloats = 2 * NCH * NBMAX * 256;
    static constexpr int kBytes = kSrcFloats * 4 + ((NBMAX + 3) & ~3) * 4 + 16;
    __device__ static constexpr int at(int plane, int c2, int c) {
        return ((plane * NCH + c2) * NBMAX + c) * 256;
    }
};

// 8 fp32 values of chunk c2 of source c (lane base `sl` = src + 4 ln)
template <int NCH, int NBMAX>
__device__ __forceinline__ void bb_lds_read(const float* sl, int c2, int c, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(sl + BbLds<NCH, NBMAX>::at(0, c2, c));
    const f32x4 b = *reinterpret_cast<const f32x4*>(sl + BbLds<NCH, NBMAX>::at(1, c2, c));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        x[q] = a[q];
        x[4 + q] = b[q];
    }
}

// The reads la..lb of block group G, all in block group G (la >= G S).
// Lane ln owns chunks ch = c2 * 64 + ln (c2 < NCH) of d; chunks past d are
// dead: their global loads return zeros and their stores are dropped (buffer
// range checks), and they skip LDS.
//
// Every read needs two passes over its frozen sources: the dots (for the
// softmax), then the weighted sum.  The sources do not change within a group,
// so the weighted sum of read l and the dots of read l + 1 share one pass:
// each source chunk is read from LDS once and feeds both (one LDS read per
// source, chunk and read instead of two).  Inside the pass, chunk c2 of the
// partial sum first serves read l's output, then takes row l + 1 and serves
// read l + 1's dots; the row and query of read l + 2 are requested when the
// pass ends, one pass ahead of their use.  (Requested chunk by chunk inside the
// pass, as soon as each register is free, they push the four-chunk variant
// past 128 VGPRs into spills.)
template <typename TO, int NCH, int NBMAX, int G>
__device__ __forceinline__ void bb_group(const FwdParams& p, const float* sl, const float* rsv,
                                        const bf16_t* hist_tok, int64_t t, int ln, int la, int lb) {
    constexpr int kV = G + 3;  // frozen-source dots, partial dot, partial sum of squares
    const int d = p.d;
    const int64_t row_elems = p.T * (int64_t)d;
    const uint64_t tok_bytes = (uint64_t)d * 2;
    const int g0 = G * p.S;  // the group's first read; its partial sums start at row g0 + 1
    const uint32_t in_off = (uint32_t)ln * 16;   // bf16 chunk c2: + 1024 c2
    const uint32_t w_off = (uint32_t)ln * 32;    // fp32 chunk c2: + 2048 c2
    const uint32_t out_off = (uint32_t)ln * 8 * sizeof(TO);

    float part[NCH][8];
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[c2][e] = 0.f;
    // row i (its loads read zeros without touching memory when !live)
    auto row_rsrc = [&](int i, bool live) {
        return make_rsrc(hist_tok + (live ? i : 0) * row_elems, live ? tok_bytes : 0);
    };
    // query of read l (one per read, or one per read and token)
    auto w_rsrc = [&](int l, bool live) {
        const int64_t jq = (live ? l : la) - p.q_begin;
        const float* wrow = p.qtok != nullptr ? p.qtok + (jq * p.T + t) * d : p.w + jq * d;
        return make_rsrc(wrow, live ? (uint64_t)d * 4 : 0);
    };
    // rows g0+1 .. la-1 (the part of the partial sum before the first read), four at a time
    for (int i0 = g0 + 1; i0 < la; i0 += 4) {
        Chunk<bf16_t> cb[4][NCH];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const rsrc_t rr = row_rsrc(i0 + u, i0 + u < la);
#pragma unroll
            for (int c2 = 0; c2 < NCH; ++c2) cb[u][c2].load(rr, in_off + 1024u * c2);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c2 = 0; c2 < NCH; ++c2) {
                float x[8];
                cb[u][c2].to_float(x);
#pragma unroll
                for (int e = 0; e < 8; ++e) part[c2][e] += x[e];
            }
    }
    // row and query of the next read to be scored, in flight
    Chunk<bf16_t> rl[NCH];
    Chunk<float> wq[NCH];
    {
        const rsrc_t rr = row_rsrc(la, la > g0);  // read g0 has no partial sum
        const rsrc_t wr = w_rsrc(la, true);
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
            rl[c2].load(rr, in_off + 1024u * c2);
            wq[c2].load(wr, w_off + 2048u * c2);
        }
    }

    float a[G + 1];  // weights of the frozen sources and of the partial sum
    float ap = 0.f;
    // One pass over the sources: read lo's weighted sum (OUT) and/or the dots of
    // read lo + 1 (DOT; for the first read, lo + 1 = la and there is no output).
    // Row lo + 1 joins the partial sum in a DOT pass; its registers and the
    // query's then take row and query lo + 2.
    auto pass = [&](auto out_tag, auto dot_tag, int lo, float (&v)[kV]) {
        constexpr bool OUT = decltype(out_tag)::value;
        constexpr bool DOT = decltype(dot_tag)::value;
        const int l2 = lo + 2;  // the read whose row and query are requested next
        const bool live2 = l2 <= lb;
        const rsrc_t rr2 = row_rsrc(l2, DOT && live2);
        const rsrc_t wr2 = w_rsrc(l2, DOT && live2);
        const int64_t jo = (OUT ? lo : la) - p.q_begin;  // output row of read lo
        const rsrc_t orr = make_rsrc(static_cast<TO*>(p.out) + jo * row_elems + t * d,
                                     OUT ? (uint64_t)d * sizeof(TO) : 0);
#pragma unroll
        for (int j = 0; j < kV; ++j) v[j] = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
            const int ch = c2 * 64 + ln;
            float o[8];
            if constexpr (OUT) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = ap * part[c2][e];
            }
            float wv[8];
            if constexpr (DOT) {
                float x[8];
                rl[c2].to_float(x);
#pragma unroll
                for (int e = 0; e < 8; ++e) part[c2][e] += x[e];
                wq[c2].to_float(wv);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[G + 1] = fmaf(wv[e], part[c2][e], v[G + 1]);
                    v[G + 2] = fmaf(part[c2][e], part[c2][e], v[G + 2]);
                }
            }
            if (ch < p.nc) {
#pragma unroll
                for (int c = 0; c <= G; ++c) {
                    float x[8];
                    bb_lds_read<NCH, NBMAX>(sl, c2, c, x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if constexpr (OUT) o[e] = fmaf(a[c], x[e], o[e]);
                        if constexpr (DOT) v[c] = fmaf(wv[e], x[e], v[c]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (OUT) store_chunk((TO*)nullptr, orr, out_off + 8u * sizeof(TO) * 64u * c2, o);
        }
        if constexpr (DOT) {
#pragma unroll
            for (int c2 = 0; c2 < NCH; ++c2) {
                rl[c2].load(rr2, in_off + 1024u * c2);
                wq[c2].load(wr2, w_off + 2048u * c2);
            }
        }
    };
    // the exact softmax over [v_0, b_1..b_G, partial] of read l from its dots
    auto coeffs = [&](int l, const float (&v)[kV]) {
        const bool has_p = l > g0;
        float tot[kV];
        wave_totals<0, kV>(v, tot, ln);
        float s[G + 1];
        float M = -INFINITY;
#pragma unroll
        for (int c = 0; c <= G; ++c) {
            s[c] = rsv[c] * kLog2e * tot[c];  // RMS scales from LDS, when the read is scored
            M = fmaxf(M, s[c]);
        }
        float sp = -INFINITY;
        if (has_p) {
            sp = fast_rsqrt(fmaf(tot[G + 2], p.inv_d, p.eps)) * tot[G + 1] * kLog2e;
            M = fmaxf(M, sp);
        }
        float Z = 0.f;
#pragma unroll
        for (int c = 0; c <= G; ++c) {
            a[c] = fast_exp2(s[c] - M);
            Z += a[c];
        }
        const float ep = has_p ? fast_exp2(sp - M) : 0.f;
        Z += ep;
        const float inv = 1.0f / Z;
#pragma unroll
        for (int c = 0; c <= G; ++c) a[c] *= inv;
        ap = ep * inv;
        const int64_t j = l - p.q_begin;
        if (p.lse != nullptr && ln == 0) p.lse[j * p.T + t] = (M + fast_log2(Z)) * kLn2;
        if (p.alpha != nullptr) {  // weight probe in source order, zeros past the sources
            const int ns = G + 1 + (has_p ? 1 : 0);
            for (int x = ln; x < p.n_hist; x += 64) {
                float ax = 0.f;
#pragma unroll
                for (int c = 0; c <= G; ++c)
                    if (x == c) ax = a[c];
                if (x == G + 1 && x < ns) ax = ap;
                p.alpha[(j * p.n_hist + x) * p.T + t] = ax;
            }
        }
    };
    using yes = std::true_type;
    using no = std::false_type;
    float v[kV];
    pass(no{}, yes{}, la - 1, v);  // dots of read la
    coeffs(la, v);
    for (int l = la; l < lb; ++l) {
        pass(yes{}, yes{}, l, v);  // output of read l, dots of read l + 1
        coeffs(l + 1, v);
    }
    pass(yes{}, no{}, lb, v);  // output of read lb
}

template <typename TO, int NCH, int NBMAX, int G = 0>
__device__ __forceinline__ void bb_dispatch(int g, const FwdParams& p, const float* sl, const float* rsv,
                                            const bf16_t* hist_tok, int64_t t, int ln, int la, int lb) {
    if constexpr (G < NBMAX) {
        if (g == G)
            bb_group<TO, NCH, NBMAX, G>(p, sl, rsv, hist_tok, t, ln, la, lb);
        else
            bb_dispatch<TO, NCH, NBMAX, G + 1>(g, p, sl, rsv, hist_tok, t, ln, la, lb);
    }
}

// Source c of a token (v_0 for c = 0, else the sum of block c's rows) in fp32
// into the LDS planes at `src`, and its RMS scale into rsv[c].  Rows are
// requested four at a time.
template <int NCH, int NBMAX>
__device__ __forceinline__ void bb_form_source(const FwdParams& p, float* src, float* rsv, const bf16_t* hist_tok,
                                               int c, int ln) {
    const int S = p.S;
    const int64_t row_elems = p.T * (int64_t)p.d;
    const uint64_t tok_bytes = (uint64_t)p.d * 2;
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
                const rsrc_t rr = make_rsrc(hist_tok + (ib + u) * row_elems, tok_bytes);
#pragma unroll
                for (int c2 = 0; c2 < NCH; ++c2) ch[u][c2].load(rr, (uint32_t)ln * 16 + 1024u * c2);
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
        if (c2 * 64 + ln < p.nc) {  // the two planes of the chunk (see BbLds)
            float* dst = src + 4 * ln;
            *reinterpret_cast<f32x4*>(dst + BbLds<NCH, NBMAX>::at(0, c2, c)) =
                f32x4{acc[c2][0], acc[c2][1], acc[c2][2], acc[c2][3]};
            *reinterpret_cast<f32x4*>(dst + BbLds<NCH, NBMAX>::at(1, c2, c)) =
                f32x4{acc[c2][4], acc[c2][5], acc[c2][6], acc[c2][7]};
        }
    }
    sq = tg_sum<64>(sq);
    if (ln == 0) rsv[c] = fast_rsqrt(fmaf(sq, p.inv_d, p.eps));
}

template <typename TO, int NCH, int NBMAX>
// Four waves per SIMD (at most 128 VGPRs): two workgroups (tokens) per CU, so
// one token's loads overlap the other's arithmetic.
__global__ __launch_bounds__(64 * kBbWaves) __attribute__((amdgpu_waves_per_eu(4)))
void block_batch_kernel(FwdParams p, int nb) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    float* const src = reinterpret_cast<float*>(lds_raw);
    float* const rsv = src + BbLds<NCH, NBMAX>::kSrcFloats;
    int* const counter = reinterpret_cast<int*>(rsv + ((NBMAX + 3) & ~3));

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = threadIdx.x & 63;
    const int64_t t = blockIdx.x;
    const int S = p.S;
    const bf16_t* hist_tok = static_cast<const bf16_t*>(p.hist) + t * p.d;

    if (threadIdx.x == 0) *counter = 0;

    // ---- prologue: frozen sources v_0, b_1, ... in fp32, their RMS scales ------
    for (int c = wave; c < nb; c += kBbWaves) bb_form_source<NCH, NBMAX>(p, src, rsv, hist_tok, c, ln);
    __syncthreads();

    // ---- block groups, latest group first ---------------------------------------
    // (Whole groups rather than halves: a second half would re-read the first
    // half's rows to catch up its partial sum, and the extra traffic cost more
    // than the finer balance gained: 20.6 against 19.3 ms at 128K / S=8.)
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
        bb_dispatch<TO, NCH, NBMAX>(g, p, src + 4 * ln, rsv, hist_tok, t, ln, la, lb);
    }
}

template <typename TO, int NCH>
hipError_t launch_bb_nch(const FwdParams& p, int nb, hipStream_t stream) {
    auto go = [&](auto kern, size_t lds) {
        const hipError_t e = prepare_dynamic_lds((const void*)kern, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)p.T), dim3(64 * kBbWaves), lds, stream, p, nb);
        return hipGetLastError();
    };
    // the group index dispatch is instantiated up to NBMAX - 1
    if (nb <= 9) return go(block_batch_kernel<TO, NCH, 9>, (size_t)BbLds<NCH, 9>::kBytes);
    return go(block_batch_kernel<TO, NCH, kBbMaxSources>, (size_t)BbLds<NCH, kBbMaxSources>::kBytes);
}

template <typename TO>
hipError_t launch_bb(const FwdParams& p, int nb, hipStream_t stream) {
    switch ((p.nc + 63) / 64) {
        case 1: return launch_bb_nch<TO, 1>(p, nb, stream);
        case 2: return launch_bb_nch<TO, 2>(p, nb, stream);
        case 3: return launch_bb_nch<TO, 3>(p, nb, stream);
        case 4: return launch_bb_nch<TO, 4>(p, nb, stream);
        default: return hipErrorInvalidValue;
    }
}

// LDS bytes of the instantiation that serves nb sources at nch chunks per lane
int64_t bb_lds_bytes(int nb, int nch) {
    const int nbmax = nb <= 9 ? 9 : kBbMaxSources;
    return (int64_t)2 * nch * nbmax * 1024 + ((nbmax + 3) & ~3) * 4 + 16;
}

// sources a read of the call can see (v_0 and the completed blocks), or 0 if
// the call does not qualify
int bb_sources(const FwdParams& p, attnres_dtype hist_dt) {
    if (hist_dt != ATTNRES_BF16 || p.S < 2 || p.n_q < kBbMinReads || p.nc > 4 * 64) return 0;
    if (p.T * 64 * kBbWaves >= ((int64_t)1 << 32)) return 0;
    const int nb = 1 + (p.q_begin + p.n_q - 1) / p.S;
    if (nb > kBbMaxSources) return 0;
    const int max_lds = device_max_lds();
    if (bb_lds_bytes(nb, (p.nc + 63) / 64) > max_lds) return 0;
    return nb;
}

}  // namespace

bool block_batch_applies(const FwdParams& p, attnres_dtype hist_dt) {
    return bb_sources(p, hist_dt) > 0;
}

hipError_t launch_block_batch(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                              hipStream_t stream) {
    const int nb = bb_sources(p, hist_dt);
    if (nb == 0) return hipErrorInvalidValue;
    return out_dt == ATTNRES_BF16 ? launch_bb<bf16_t>(p, nb, stream)
                                  : launch_bb<float>(p, nb, stream);
}

}  // namespace attnres
