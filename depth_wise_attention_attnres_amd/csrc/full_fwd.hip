// full_fwd.hip -- Full AttnRes forward on gfx950.
//
// One read l of one token ("DepthBench reading notes" sec. 2.3): scores
// s_i = r(v_i) (w_l . v_i) over rows i = 0..l, softmax over depth, and
// h_l = sum_i softmax_i v_i.  The kernel streams the rows of each token once
// per read, in depth order, with an online softmax (running max m, running
// sum Z, fp32 accumulator), so every row is read from HBM once per read and
// nothing but the output is written.  The RMS scale r(v_i) comes from the
// caller's cache when valid, else from the sum of squares of the row already
// in registers (and is then written back to the cache).
//
// The same kernel serves Block reads with many blocks (BLOCK = true): the
// sources of read l are then v_0, the block sums and the partial sum, each
// formed on the fly in fp32 from the raw rows it covers and scored when its
// last row has been added ("DepthBench reading notes" sec. 2.5; DataCamp,
// block section).
//
// Thread mapping: a token group (TG) of LPT lanes per token, NCH 16-byte
// chunks per lane (see device_common.hpp); 256-thread blocks hold 256/LPT
// consecutive tokens.  Row accesses are buffer loads from a wave-uniform row
// base; loads of the next PF rows are in flight while a row is consumed.  The
// max is rescaled lazily: only when a new score exceeds it.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

// Workgroup size of the streaming kernel (tokens per workgroup = threads / LPT).
constexpr int kStreamThreads = 256;
// Cache policy of the history loads: a single-read call touches each row
// once (non-temporal); with several reads the wave re-reads the token's rows
// for every read, so they are loaded with the default policy.
constexpr int kHistAuxOnce = 2;

template <typename TI, typename TO, int LPT, int NCH, int PF, bool BLOCK>
__global__ __launch_bounds__(kStreamThreads) void full_fwd_stream_kernel(FwdParams p) {
    constexpr int TPB = kStreamThreads / LPT;  // tokens per block
    const int ln = threadIdx.x % LPT;
    const int64_t tok0 = (int64_t)blockIdx.x * TPB;
    // token within the block; with one token per wave it is wave-uniform, and
    // saying so keeps every per-token address (query row, probe) scalar
    const int tl = LPT == 64 ? __builtin_amdgcn_readfirstlane(threadIdx.x / LPT) : threadIdx.x / LPT;
    const int64_t t = tok0 + tl;
    if (t >= p.T) return;  // whole token groups leave together

    const int64_t row_elems = p.T * (int64_t)p.d;            // elements between rows
    const int64_t blk_tok = p.T - tok0 < TPB ? p.T - tok0 : TPB;  // tokens of this block
    const uint64_t blk_elems = (uint64_t)blk_tok * p.d;
    const TI* hist_blk = static_cast<const TI*>(p.hist) + tok0 * p.d;
    TO* out_blk = static_cast<TO*>(p.out) + tok0 * p.d;

    // byte offsets of this lane's chunks inside the block's slice of a row;
    // chunks past d get kOOB (loads read zeros, stores are dropped)
    uint32_t in_off[NCH], out_off[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = c * LPT + ln;
        const uint32_t e = (uint32_t)(tl * p.d + ch * 8);
        in_off[c] = ch < p.nc ? e * (uint32_t)sizeof(TI) : kOOB;
        out_off[c] = ch < p.nc ? e * (uint32_t)sizeof(TO) : kOOB;
    }
    const uint32_t tok_f32_off = (uint32_t)tl * 4u;

    for (int j = 0; j < p.n_q; ++j) {
        const int l = p.q_begin + j;
        float wv[NCH][8];
        {
            // the read's query: one per read, or one per (read, token)
            const float* wrow = p.qtok != nullptr ? p.qtok + ((int64_t)j * p.T + t) * p.d
                                                  : p.w + (int64_t)j * p.d;
            const rsrc_t wr = make_rsrc(wrow, (uint64_t)p.d * 4);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const uint32_t off = in_off[c] == kOOB ? kOOB : (uint32_t)((c * LPT + ln) * 32);
                Chunk<float> ch;
                ch.load(wr, off);
                ch.to_float(wv[c]);
            }
        }

        float acc[NCH][8];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
        float m2 = -INFINITY;  // running max of scores, log2 domain
        float Z = 0.f;         // running sum of exp2(s2 - m2)
        int ns = 0;            // sources scored so far
        // weight probe: lane 0 keeps each source's score in alpha and turns
        // the scores into weights once the read's log-sum-exp is known
        float* const al = p.alpha != nullptr ? p.alpha + (int64_t)j * p.n_hist * p.T + t : nullptr;
        float run[BLOCK ? NCH : 1][8];  // Block: the fp32 sum being formed
#pragma unroll
        for (int c = 0; c < (BLOCK ? NCH : 1); ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) run[c][e] = 0.f;

        // ring of PF prefetched rows (and their cached scales)
        Chunk<TI> buf[PF][NCH];
        float rbuf[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            rbuf[u] = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) buf[u][c].zero();
        }
        auto issue = [&](int u, int i) {
            const rsrc_t rr = make_rsrc(hist_blk + i * row_elems, blk_elems * sizeof(TI));
            if (p.n_q == 1) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) buf[u][c].template load<kHistAuxOnce>(rr, in_off[c]);
            } else {
#pragma unroll
                for (int c = 0; c < NCH; ++c) buf[u][c].load(rr, in_off[c]);
            }
            if (i < p.rinv_valid) {
                if constexpr (LPT == 64) {  // one token per wave: a scalar load
                    rbuf[u] = const_view(p.rinv)[(int64_t)i * p.T + t];
                } else {
                    const rsrc_t cr = make_rsrc(p.rinv + (int64_t)i * p.T + tok0, (uint64_t)blk_tok * 4);
                    rbuf[u] = load_f32(cr, tok_f32_off);
                }
            }
        };
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (u <= l) issue(u, u);

        for (int i0 = 0; i0 <= l; i0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int i = i0 + u;
                if (i > l) break;
                float xf[NCH][8];
#pragma unroll
                for (int c = 0; c < NCH; ++c) buf[u][c].to_float(xf[c]);
                const float rc = rbuf[u];
                if (i + PF <= l) issue(u, i + PF);

                if constexpr (BLOCK) {
                    // v_0 is a source of its own; other rows join the running
                    // sum, which becomes a source when its block closes or at
                    // the read's own row (the partial sum)
                    if (i > 0) {
#pragma unroll
                        for (int c = 0; c < NCH; ++c)
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                run[c][e] += xf[c][e];
                                xf[c][e] = run[c][e];
                            }
                        if (i % p.S != 0 && i != l) continue;
#pragma unroll
                        for (int c = 0; c < NCH; ++c)
#pragma unroll
                            for (int e = 0; e < 8; ++e) run[c][e] = 0.f;
                    }
                }

                const bool need_sq = BLOCK || i >= p.rinv_valid;  // uniform over the grid
                float dp = 0.f, sq = 0.f;
                if (need_sq) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            dp = fmaf(wv[c][e], xf[c][e], dp);
                            sq = fmaf(xf[c][e], xf[c][e], sq);
                        }
                    dp = tg_sum<LPT>(dp);
                    sq = tg_sum<LPT>(sq);
                } else {
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e) dp = fmaf(wv[c][e], xf[c][e], dp);
                    dp = tg_sum<LPT>(dp);
                }
                float r = rc;
                if (need_sq) {
                    r = fast_rsqrt(fmaf(sq, p.inv_d, p.eps));
                    // cache row i is written once per call, by the first read of
                    // the call that sees it
                    const int owner = i - p.q_begin > 0 ? i - p.q_begin : 0;
                    if (!BLOCK && p.rinv != nullptr && j == owner && ln == 0)
                        p.rinv[(int64_t)i * p.T + t] = r;
                }
                const float s2 = r * dp * kLog2e;
                if (al != nullptr && ln == 0) al[(int64_t)ns * p.T] = s2;
                ++ns;
                if (s2 > m2) {  // new running max: rescale what is accumulated
                    const float cs = fast_exp2(m2 - s2);
                    Z *= cs;
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[c][e] *= cs;
                    m2 = s2;
                }
                const float pw = fast_exp2(s2 - m2);
                Z += pw;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[c][e] = fmaf(pw, xf[c][e], acc[c][e]);
            }
        }

        const float inv_z = 1.0f / Z;
        const rsrc_t orr = make_rsrc(out_blk + (int64_t)j * row_elems, blk_elems * sizeof(TO));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[c][e] *= inv_z;
            store_chunk((TO*)nullptr, orr, out_off[c], acc[c]);
        }
        if (p.normed != nullptr) {  // fused pre-norm of the output (uniform branch)
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(acc[c][e], acc[c][e], ss);
            ss = tg_sum<LPT>(ss);
            const float rn = fast_rsqrt(fmaf(ss, p.inv_d, p.eps));
            const rsrc_t nrr = make_rsrc(static_cast<TO*>(p.normed) + tok0 * p.d + (int64_t)j * row_elems,
                                         blk_elems * sizeof(TO));
            const rsrc_t grr = make_rsrc(p.norm_gain + (int64_t)j * p.d, (uint64_t)p.d * 4);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float g[8];
                if (p.norm_gain != nullptr) {
                    Chunk<float> gc;
                    gc.load(grr, in_off[c] == kOOB ? kOOB : (uint32_t)((c * LPT + ln) * 32));
                    gc.to_float(g);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) g[e] = 1.f;
                }
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = g[e] * (acc[c][e] * rn);
                store_chunk((TO*)nullptr, nrr, out_off[c], y);
            }
        }
        if (p.lse != nullptr && ln == 0) p.lse[(int64_t)j * p.T + t] = (m2 + fast_log2(Z)) * kLn2;
        if (al != nullptr && ln == 0) {  // the same lane reads back what it wrote
            const float lse2 = m2 + fast_log2(Z);
            for (int x = 0; x < ns; ++x) al[(int64_t)x * p.T] = fast_exp2(al[(int64_t)x * p.T] - lse2);
            for (int x = ns; x < p.n_hist; ++x) al[(int64_t)x * p.T] = 0.f;
        }
    }
}

// ---------------------------------------------------------------------------
// launch selection

namespace {

template <typename TI, typename TO, int LPT, int NCH, int PF, bool BLOCK>
hipError_t launch_stream(const FwdParams& p, hipStream_t stream) {
    constexpr int TPB = kStreamThreads / LPT;
    const int64_t blocks = (p.T + TPB - 1) / TPB;
    hipLaunchKernelGGL((full_fwd_stream_kernel<TI, TO, LPT, NCH, PF, BLOCK>),
                       dim3((unsigned)blocks), dim3(kStreamThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename TI, typename TO, bool BLOCK>
hipError_t dispatch_stream(const FwdParams& p, hipStream_t stream) {
    // Full reads of bf16 rows with d <= 896: 16 lanes per token (four tokens
    // per wave), ceil(d / 128) chunks per lane.  At d = 896 or 640 every lane
    // is busy (64 lanes per token leave 12.5% / 37.5% of the lanes idle), each
    // wave reads four tokens' rows contiguously, and a wave sum takes four DPP
    // steps instead of six.  One row in flight per token: the registers of the
    // wider tiles leave room for no more at two waves per SIMD.  Measured on
    // the read-by-read sweeps: L=32 / d=896 11.54 -> 10.80 ms, L=70 / d=640
    // 37.2 -> 34.1 ms (a second row in flight: 11.45 and 34.6 ms).
    if constexpr (!BLOCK && sizeof(TI) == 2) {
        switch (p.nc <= 112 ? (p.nc + 15) / 16 : 0) {
            case 1: return launch_stream<TI, TO, 16, 1, 4, BLOCK>(p, stream);
            case 2: return launch_stream<TI, TO, 16, 2, 4, BLOCK>(p, stream);
            case 3: return launch_stream<TI, TO, 16, 3, 2, BLOCK>(p, stream);
            case 4: return launch_stream<TI, TO, 16, 4, 2, BLOCK>(p, stream);
            case 5: return launch_stream<TI, TO, 16, 5, 1, BLOCK>(p, stream);
            case 6: return launch_stream<TI, TO, 16, 6, 1, BLOCK>(p, stream);
            case 7: return launch_stream<TI, TO, 16, 7, 1, BLOCK>(p, stream);
            default: break;
        }
    }
    // LPT = 64 lanes per token, NCH chunks per lane: one token per wave
    const int nch = (p.nc + 63) / 64;
    switch (nch) {
        case 1: return launch_stream<TI, TO, 64, 1, 4, BLOCK>(p, stream);
        case 2: return launch_stream<TI, TO, 64, 2, 4, BLOCK>(p, stream);
        case 3: return launch_stream<TI, TO, 64, 3, 3, BLOCK>(p, stream);
        case 4: return launch_stream<TI, TO, 64, 4, 2, BLOCK>(p, stream);
        case 5: return launch_stream<TI, TO, 64, 5, 2, BLOCK>(p, stream);
        case 6: return launch_stream<TI, TO, 64, 6, 2, BLOCK>(p, stream);
        case 7: return launch_stream<TI, TO, 64, 7, 2, BLOCK>(p, stream);
        case 8: return launch_stream<TI, TO, 64, 8, 1, BLOCK>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_full_fwd(const FullFwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                           hipStream_t stream) {
    if (full_batch_mfma_applies(p, hist_dt, out_dt)) return launch_full_batch_mfma(p, stream);
    if (full_batch_applies(p, hist_dt)) return launch_full_batch(p, hist_dt, out_dt, stream);
    if (hist_dt == ATTNRES_BF16 && out_dt == ATTNRES_BF16)
        return dispatch_stream<bf16_t, bf16_t, false>(p, stream);
    if (hist_dt == ATTNRES_BF16 && out_dt == ATTNRES_F32)
        return dispatch_stream<bf16_t, float, false>(p, stream);
    if (hist_dt == ATTNRES_F32 && out_dt == ATTNRES_F32)
        return dispatch_stream<float, float, false>(p, stream);
    return dispatch_stream<float, bf16_t, false>(p, stream);
}

hipError_t launch_block_stream(const BlockFwdParams& p, hipStream_t stream) {
    if (p.hist_dt == ATTNRES_BF16 && p.out_dt == ATTNRES_BF16)
        return dispatch_stream<bf16_t, bf16_t, true>(p, stream);
    if (p.hist_dt == ATTNRES_BF16 && p.out_dt == ATTNRES_F32)
        return dispatch_stream<bf16_t, float, true>(p, stream);
    if (p.hist_dt == ATTNRES_F32 && p.out_dt == ATTNRES_F32)
        return dispatch_stream<float, float, true>(p, stream);
    return dispatch_stream<float, bf16_t, true>(p, stream);
}

}  // namespace attnres
