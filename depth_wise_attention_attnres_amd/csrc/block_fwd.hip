// block_fwd.hip -- Block AttnRes forward, two-phase, on gfx950.
//
// Block reading ("DepthBench reading notes" sec. 2.5; "LLMRes", Block
// paragraph; DataCamp, block section): block c sums sublayer outputs
// (c-1)S+1 .. cS; read l with m = floor(l/S) attends over v_0, b_1..b_m and,
// when l mod S != 0, the running partial sum p_l = v_{mS+1} + ... + v_l.
// Two-phase computation (DataCamp, "two-phase computation"): the reads of a
// block group share the frozen sources [v_0, b_1..b_m], so their scores
// against those sources are computed as one batch (phase 1: max M1, sum Z1,
// weights); the partial sum is then scored per read and merged by the
// log-sum-exp rule (phase 2):
//   M = max(M1, s_p), A = Z1 e^(M1 - M), B = e^(s_p - M),
//   h = (sum_c e^(s_c - M) x_c + B p) / (A + B),  lse = M + log(A + B).
//
// Mapping: one workgroup of NW waves per token; lane `ln` owns the 16-byte
// chunk ln of d (8 elements), so the whole raw history of the token is read
// exactly once, in depth order, and the fp32 sources live in registers
// (NSRC x 8 VGPRs per lane).  Reads are processed in chunks of at most CR
// consecutive reads inside one block group:
//   A1  partial sums of the chunk's reads (fp32), the next chunk's rows are
//       then requested (the rows of this chunk are dead);
//   A2  per-lane partial dots (queries double-buffered from L2), summed over
//       each 16-lane row with DPP butterflies; each row's sums go to LDS;
//   A3  one lane per value adds the row sums (fixed order);
//   A4  one lane per read forms scores, the phase-1 softmax and the phase-2
//       merge, and publishes the coefficients;
//   B   every lane forms its chunk of the outputs from register sources.
// The chunk body is instantiated per block group G, so every loop over
// sources has a compile-time bound.  Three workgroup barriers per chunk.
// Block sums are fp32 and never rounded.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

template <int NSRC, int CR>
struct BlockLds {
    static constexpr int kStride = NSRC + 2;     // values per read: NSRC dots, p dot, p sumsq
    static constexpr int kVals = CR * kStride + 1;  // + sum of squares of a new source
};

// Per-token state of the two-phase kernel, held in registers.
template <typename TI, int NSRC, int CR>
struct BlockState {
    float src[NSRC][8];   // v_0, b_1, b_2, ... (fp32)
    float part_sum[8];    // running partial sum of the current block
    Chunk<TI> rows[CR];   // raw rows of the chunk (then of the next chunk)
    Chunk<float> wbuf[2]; // pseudo-queries, double-buffered
};

// Shared-memory layout of one workgroup.
template <int NW, int NSRC, int CR>
struct BlockShared {
    static constexpr int kRowSlots = 4 * NW;  // 16-lane rows in the workgroup
    float* part;  // [kVals][kRowSlots] row sums
    float* fin;   // [kVals] totals
    float* coef;  // [CR][kStride] output coefficients (slot NSRC: the partial)
    float* rs;    // [NSRC] RMS scale of each source
};

// Everything one chunk does, for a chunk of block group G (sources 0..G).
// l0: first read of the chunk, n: reads in the chunk, nl0/nl1: next chunk.
template <typename TI, typename TO, int NW, int NSRC, int CR, int G>
__device__ __forceinline__ void block_chunk(const BlockFwdParams& p, BlockState<TI, NSRC, CR>& st,
                                            const BlockShared<NW, NSRC, CR>& sh, int64_t t,
                                            int l0, int n, int nl0, int nl1,
                                            const TI* hist_tok, TO* out_tok, uint32_t in_off,
                                            uint32_t out_off, uint32_t w_off) {
    constexpr int kStride = BlockLds<NSRC, CR>::kStride;
    constexpr int kVals = BlockLds<NSRC, CR>::kVals;
    constexpr int kSq = CR * kStride;
    constexpr int kRowSlots = 4 * NW;
    const int tid = threadIdx.x;
    const int row_slot = tid >> 4;
    const int64_t row_elems = p.T * (int64_t)p.d;
    const uint64_t tok_in_bytes = (uint64_t)p.d * sizeof(TI);
    const uint64_t tok_out_bytes = (uint64_t)p.d * sizeof(TO);
    const int S = p.S;
    const bool new_src = (l0 == G * S);   // row l0 closes block G (or is v_0)

    auto issue_w = [&](int slot, int l) {
        const rsrc_t wr = make_rsrc(p.w + (int64_t)(l - p.q_begin) * p.d, (uint64_t)p.d * 4);
        st.wbuf[slot].load(wr, w_off);
    };
    const int k_first = p.q_begin > l0 ? p.q_begin - l0 : 0;  // first read with an output
    if (k_first < n) {  // slot chosen by branch so the buffer index stays compile-time
        if (k_first & 1)
            issue_w(1, l0 + k_first);
        else
            issue_w(0, l0 + k_first);
    }

    // ---- A1: the new source and the partial sums -------------------------
    float pk[CR][8];
    {
        float xf[8];
        st.rows[0].to_float(xf);
        if (new_src) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                st.src[G][e] = G == 0 ? xf[e] : st.part_sum[e] + xf[e];
                st.part_sum[e] = 0.f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) st.part_sum[e] += xf[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[0][e] = st.part_sum[e];
#pragma unroll
        for (int k = 1; k < CR; ++k) {
            if (k < n) {
                st.rows[k].to_float(xf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    st.part_sum[e] += xf[e];
                    pk[k][e] = st.part_sum[e];
                }
            }
        }
    }
    // rows of this chunk are consumed: request the next chunk's rows now
    if (nl0 < p.q_begin + p.n_q) {
#pragma unroll
        for (int k = 0; k < CR; ++k)
            if (k < nl1 - nl0) {
                const rsrc_t rr = make_rsrc(hist_tok + (int64_t)(nl0 + k) * row_elems, tok_in_bytes);
                st.rows[k].load(rr, in_off);
            }
    }

    // ---- A2: partial dots, summed over 16-lane rows, into LDS --------------
    // After the row butterfly all 16 lanes of a row hold the row's sum and all
    // of them store it to the same LDS word.
    if (new_src) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq = fmaf(st.src[G][e], st.src[G][e], sq);
        sq = tg_sum<16>(sq);
        sh.part[kSq * kRowSlots + row_slot] = sq;
    }
#pragma unroll
    for (int k = 0; k < CR; ++k) {
        const int l = l0 + k;
        if (k < n && l >= p.q_begin) {
            float wv[8];
            st.wbuf[k & 1].to_float(wv);
            if (k + 1 < n) issue_w((k + 1) & 1, l + 1);
            constexpr int kV = G + 3;  // G+1 frozen-source dots, partial dot, partial sumsq
            float v[kV];
#pragma unroll
            for (int c = 0; c <= G; ++c) {          // phase 1: the frozen sources
                float dp = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) dp = fmaf(wv[e], st.src[c][e], dp);
                v[c] = dp;
            }
            {                                       // phase 2: the partial sum
                float dp = 0.f, sq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    dp = fmaf(wv[e], pk[k][e], dp);
                    sq = fmaf(pk[k][e], pk[k][e], sq);
                }
                v[G + 1] = dp;
                v[G + 2] = sq;
            }
#pragma unroll
            for (int c = 0; c < kV; ++c) v[c] += dpp<kDppXor1>(v[c]);
#pragma unroll
            for (int c = 0; c < kV; ++c) v[c] += dpp<kDppXor2>(v[c]);
#pragma unroll
            for (int c = 0; c < kV; ++c) v[c] += dpp<kDppHalfMirror>(v[c]);
#pragma unroll
            for (int c = 0; c < kV; ++c) v[c] += dpp<kDppMirror>(v[c]);
            float* pp = sh.part + k * kStride * kRowSlots + row_slot;
#pragma unroll
            for (int c = 0; c <= G; ++c) pp[c * kRowSlots] = v[c];
            pp[NSRC * kRowSlots] = v[G + 1];
            pp[(NSRC + 1) * kRowSlots] = v[G + 2];
        }
    }
    __syncthreads();

    // ---- A3: totals over the row sums (fixed order) -----------------------
    for (int u = tid; u < kVals; u += 64 * NW) {
        const f32x4* q = reinterpret_cast<const f32x4*>(sh.part + u * kRowSlots);
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < kRowSlots / 4; ++r) {
            const f32x4 a = q[r];
            s += a[0];
            s += a[1];
            s += a[2];
            s += a[3];
        }
        sh.fin[u] = s;
    }
    __syncthreads();

    // ---- A4: scores, phase-1 softmax, phase-2 merge (one lane per read) ---
    if (tid < n && l0 + tid >= p.q_begin) {
        const int k = tid;
        const int l = l0 + k;
        const float* f = sh.fin + k * kStride;
        float s2[G + 1];
        float M1 = -INFINITY;
#pragma unroll
        for (int c = 0; c <= G; ++c) {
            const float r = (new_src && c == G) ? fast_rsqrt(fmaf(sh.fin[kSq], p.inv_d, p.eps))
                                                : sh.rs[c];
            s2[c] = r * f[c] * kLog2e;
            M1 = fmaxf(M1, s2[c]);
        }
        float Z1 = 0.f;
#pragma unroll
        for (int c = 0; c <= G; ++c) {
            s2[c] = fast_exp2(s2[c] - M1);
            Z1 += s2[c];
        }
        float M = M1, A = Z1, B = 0.f;
        if (l != G * S) {
            const float rp = fast_rsqrt(fmaf(f[NSRC + 1], p.inv_d, p.eps));
            const float sp = rp * f[NSRC] * kLog2e;
            M = fmaxf(M1, sp);
            A = Z1 * fast_exp2(M1 - M);
            B = fast_exp2(sp - M);
        }
        const float inv = 1.0f / (A + B);
        const float scale1 = fast_exp2(M1 - M) * inv;  // e^(s_c - M1) -> e^(s_c - M) / (A + B)
        float* cf = sh.coef + k * kStride;
#pragma unroll
        for (int c = 0; c <= G; ++c) cf[c] = s2[c] * scale1;
        cf[NSRC] = B * inv;
        if (p.lse != nullptr)
            p.lse[(int64_t)(l - p.q_begin) * p.T + t] = (M + fast_log2(A + B)) * kLn2;
    }
    if (new_src && tid == 0) sh.rs[G] = fast_rsqrt(fmaf(sh.fin[kSq], p.inv_d, p.eps));
    __syncthreads();

    // ---- B: outputs ------------------------------------------------------
#pragma unroll
    for (int k = 0; k < CR; ++k) {
        const int l = l0 + k;
        if (k < n && l >= p.q_begin) {
            const float* cf = sh.coef + k * kStride;
            float o[8];
            const float cp = l != G * S ? cf[NSRC] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = cp * pk[k][e];
#pragma unroll
            for (int c = 0; c <= G; ++c) {
                const float a = cf[c];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(a, st.src[c][e], o[e]);
            }
            const rsrc_t orr = make_rsrc(out_tok + (int64_t)(l - p.q_begin) * row_elems, tok_out_bytes);
            store_chunk((TO*)nullptr, orr, out_off, o);
        }
    }
}

template <typename TI, typename TO, int NW, int NSRC, int CR, int G = 0>
__device__ __forceinline__ void block_chunk_dispatch(int g, const BlockFwdParams& p,
                                                     BlockState<TI, NSRC, CR>& st,
                                                     const BlockShared<NW, NSRC, CR>& sh, int64_t t,
                                                     int l0, int n, int nl0, int nl1,
                                                     const TI* hist_tok, TO* out_tok,
                                                     uint32_t in_off, uint32_t out_off,
                                                     uint32_t w_off) {
    if constexpr (G < NSRC) {
        if (g == G)
            block_chunk<TI, TO, NW, NSRC, CR, G>(p, st, sh, t, l0, n, nl0, nl1, hist_tok, out_tok,
                                                 in_off, out_off, w_off);
        else
            block_chunk_dispatch<TI, TO, NW, NSRC, CR, G + 1>(g, p, st, sh, t, l0, n, nl0, nl1,
                                                              hist_tok, out_tok, in_off, out_off,
                                                              w_off);
    }
}

// Two workgroups per CU (two waves per SIMD) keep one token's barrier phases
// overlapped with another's loads and arithmetic: cap registers at 256.
template <typename TI, typename TO, int NW, int NSRC, int CR>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void block_fwd_twophase_kernel(BlockFwdParams p) {
    constexpr int kStride = BlockLds<NSRC, CR>::kStride;
    constexpr int kVals = BlockLds<NSRC, CR>::kVals;
    constexpr int kRowSlots = 4 * NW;

    extern __shared__ float lds[];
    BlockShared<NW, NSRC, CR> sh;
    sh.part = lds;
    sh.fin = sh.part + kVals * kRowSlots;
    sh.coef = sh.fin + kVals;
    sh.rs = sh.coef + CR * kStride;

    const int ln = threadIdx.x;                   // chunk index of d owned by this lane
    const int64_t t = blockIdx.x;                 // token
    const TI* hist_tok = static_cast<const TI*>(p.hist) + t * p.d;
    TO* out_tok = static_cast<TO*>(p.out) + t * p.d;
    const uint32_t in_off = ln < p.nc ? (uint32_t)(ln * 8 * sizeof(TI)) : kOOB;
    const uint32_t out_off = ln < p.nc ? (uint32_t)(ln * 8 * sizeof(TO)) : kOOB;
    const uint32_t w_off = ln < p.nc ? (uint32_t)(ln * 32) : kOOB;
    const int q_end = p.q_begin + p.n_q;
    const int S = p.S;
    const int64_t row_elems = p.T * (int64_t)p.d;

    BlockState<TI, NSRC, CR> st;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.part_sum[e] = 0.f;
#pragma unroll
    for (int c = 0; c < NSRC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) st.src[c][e] = 0.f;

    auto chunk_end = [&](int l0) {
        const int g = l0 / S;
        int l1 = (g + 1) * S;
        if (l1 > l0 + CR) l1 = l0 + CR;
        if (l1 > q_end) l1 = q_end;
        return l1;
    };

    int l0 = 0;
    int l1 = chunk_end(0);
#pragma unroll
    for (int k = 0; k < CR; ++k)
        if (k < l1) {
            const rsrc_t rr = make_rsrc(hist_tok + (int64_t)k * row_elems, (uint64_t)p.d * sizeof(TI));
            st.rows[k].load(rr, in_off);
        }
    while (l0 < q_end) {
        const int nl0 = l1;
        const int nl1 = nl0 < q_end ? chunk_end(nl0) : nl0;
        block_chunk_dispatch<TI, TO, NW, NSRC, CR>(l0 / S, p, st, sh, t, l0, l1 - l0, nl0, nl1,
                                                   hist_tok, out_tok, in_off, out_off, w_off);
        l0 = nl0;
        l1 = nl1;
    }
}

// ---------------------------------------------------------------------------
// launch selection

namespace {

template <typename TI, typename TO, int NW, int NSRC, int CR>
hipError_t launch_twophase(const BlockFwdParams& p, hipStream_t stream) {
    constexpr int kStride = BlockLds<NSRC, CR>::kStride;
    constexpr int kVals = BlockLds<NSRC, CR>::kVals;
    const size_t lds = sizeof(float) * (kVals * 4 * NW + kVals + CR * kStride + NSRC);
    hipLaunchKernelGGL((block_fwd_twophase_kernel<TI, TO, NW, NSRC, CR>), dim3((unsigned)p.T),
                       dim3(64 * NW), lds, stream, p);
    return hipGetLastError();
}

template <typename TI, typename TO, int NW>
hipError_t dispatch_nsrc(const BlockFwdParams& p, int nsrc, hipStream_t stream) {
    // reads per chunk: as many as the registers allow without spilling
    // (sources, partial sums and the chunk's rows all live in VGPRs)
    if (nsrc <= 5)
        return p.S >= 8 ? launch_twophase<TI, TO, NW, 5, 8>(p, stream)
                        : launch_twophase<TI, TO, NW, 5, 4>(p, stream);
    if (nsrc <= 9) return launch_twophase<TI, TO, NW, 9, 4>(p, stream);
    return launch_twophase<TI, TO, NW, 13, 4>(p, stream);
}

template <typename TI, typename TO>
hipError_t dispatch_block(const BlockFwdParams& p, hipStream_t stream) {
    // sources a read of this call can see: v_0 plus the completed blocks
    const int last = p.q_begin + p.n_q - 1;
    const int nsrc = 1 + last / p.S;
    if (nsrc <= kBlockMaxRegSources) {
        if (p.nc <= 64) return dispatch_nsrc<TI, TO, 1>(p, nsrc, stream);
        if (p.nc <= 128) return dispatch_nsrc<TI, TO, 2>(p, nsrc, stream);
        if (p.nc <= 256) return dispatch_nsrc<TI, TO, 4>(p, nsrc, stream);
        return dispatch_nsrc<TI, TO, 8>(p, nsrc, stream);
    }
    // many blocks: stream the raw rows per read and form the sums on the fly
    return launch_block_stream(p, stream);
}

}  // namespace

hipError_t launch_block_fwd(const BlockFwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                            hipStream_t stream) {
    if (hist_dt == ATTNRES_BF16 && out_dt == ATTNRES_BF16)
        return dispatch_block<bf16_t, bf16_t>(p, stream);
    if (hist_dt == ATTNRES_BF16 && out_dt == ATTNRES_F32)
        return dispatch_block<bf16_t, float>(p, stream);
    if (hist_dt == ATTNRES_F32 && out_dt == ATTNRES_F32)
        return dispatch_block<float, float>(p, stream);
    return dispatch_block<float, bf16_t>(p, stream);
}

}  // namespace attnres
