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
// (NSRC x 8 VGPRs per lane).  Reads are processed in chunks of at most 8
// consecutive reads inside one block group:
//   A1  partial sums of the chunk's reads (fp32), the next chunk's rows are
//       then requested (the rows of this chunk are dead);
//   A2  per-lane partial dots, reduced across each 16-lane row with DPP and
//       written to LDS (one float per row and value);
//   A3  one lane per value sums the row partials (fixed order);
//   A4  one lane per read forms scores, the phase-1 softmax and the phase-2
//       merge, and publishes the coefficients;
//   B   every lane forms its chunk of the outputs from register sources.
// Block sums are fp32 and never rounded.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

constexpr int kChunkReads = 8;  // reads processed per chunk

template <int NSRC>
struct BlockLds {
    static constexpr int kStride = NSRC + 2;              // values per read: NSRC dots, p dot, p sumsq
    static constexpr int kVals = kChunkReads * kStride + 1;  // + sum of squares of a new source
};

// sum over a 16-lane row; every lane of the row gets the sum
__device__ __forceinline__ float row_sum(float v) { return tg_sum<16>(v); }

}  // namespace

template <typename TI, typename TO, int NW, int NSRC>
__global__ __launch_bounds__(64 * NW) void block_fwd_twophase_kernel(BlockFwdParams p) {
    constexpr int kThreads = 64 * NW;
    constexpr int kRows = 4 * NW;                 // 16-lane rows in the workgroup
    constexpr int kStride = BlockLds<NSRC>::kStride;
    constexpr int kVals = BlockLds<NSRC>::kVals;
    constexpr int kSq = kChunkReads * kStride;    // index of the new source's sum of squares

    extern __shared__ float lds[];
    float* part = lds;                            // [kVals][kRows]
    float* fin = part + kVals * kRows;            // [kVals]
    float* coef = fin + kVals;                    // [kChunkReads][kStride]  (slot NSRC = partial)
    float* rs = coef + kChunkReads * kStride;     // [NSRC] RMS scale of each source

    const int tid = threadIdx.x;
    const int ln = tid;                           // chunk index of d owned by this lane
    const int row_id = tid >> 4;
    const int64_t t = blockIdx.x;                 // token

    const int64_t row_elems = p.T * (int64_t)p.d;
    const TI* hist_tok = static_cast<const TI*>(p.hist) + t * p.d;
    TO* out_tok = static_cast<TO*>(p.out) + t * p.d;
    const uint32_t in_off = ln < p.nc ? (uint32_t)(ln * 8 * sizeof(TI)) : kOOB;
    const uint32_t out_off = ln < p.nc ? (uint32_t)(ln * 8 * sizeof(TO)) : kOOB;
    const uint32_t w_off = ln < p.nc ? (uint32_t)(ln * 32) : kOOB;
    const uint64_t tok_in_bytes = (uint64_t)p.d * sizeof(TI);
    const uint64_t tok_out_bytes = (uint64_t)p.d * sizeof(TO);
    const int q_end = p.q_begin + p.n_q;
    const int S = p.S;

    float src[NSRC][8];   // v_0, b_1, b_2, ... (fp32)
    float part_sum[8];    // running partial sum of the current block
#pragma unroll
    for (int e = 0; e < 8; ++e) part_sum[e] = 0.f;
#pragma unroll
    for (int c = 0; c < NSRC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) src[c][e] = 0.f;

    Chunk<TI> rows[kChunkReads];
    auto issue_rows = [&](int l0, int n) {
#pragma unroll
        for (int k = 0; k < kChunkReads; ++k)
            if (k < n) {
                const rsrc_t rr = make_rsrc(hist_tok + (int64_t)(l0 + k) * row_elems, tok_in_bytes);
                rows[k].load(rr, in_off);
            }
    };
    auto chunk_end = [&](int l0) {
        const int g = l0 / S;
        int l1 = (g + 1) * S;
        if (l1 > l0 + kChunkReads) l1 = l0 + kChunkReads;
        if (l1 > q_end) l1 = q_end;
        return l1;
    };

    int l0 = 0;
    int l1 = chunk_end(0);
    issue_rows(0, l1);

    while (l0 < q_end) {
        const int n = l1 - l0;
        const int g = l0 / S;                      // block group of the chunk (sources 0..g)
        const bool new_src = (l0 == g * S);        // row l0 closes block g (or is v_0)

        // ---- A1: sources and partial sums ------------------------------------
        float pk[kChunkReads][8];
        {
            float xf[8];
            rows[0].to_float(xf);
            if (new_src) {
#pragma unroll
                for (int c = 0; c < NSRC; ++c)
                    if (c == g) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            src[c][e] = g == 0 ? xf[e] : part_sum[e] + xf[e];
                            part_sum[e] = 0.f;
                        }
                    }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) part_sum[e] += xf[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[0][e] = part_sum[e];
#pragma unroll
            for (int k = 1; k < kChunkReads; ++k) {
                if (k < n) {
                    rows[k].to_float(xf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        part_sum[e] += xf[e];
                        pk[k][e] = part_sum[e];
                    }
                }
            }
        }
        // rows of this chunk are consumed: request the next chunk's rows now
        const int nl0 = l1;
        const int nl1 = nl0 < q_end ? chunk_end(nl0) : nl0;
        if (nl0 < q_end) issue_rows(nl0, nl1 - nl0);

        // ---- A2: partial dots, row-reduced, into LDS --------------------------
        auto put = [&](int idx, float v) {
            v = row_sum(v);
            if ((tid & 15) == 0) part[idx * kRows + row_id] = v;
        };
        if (new_src) {
            float sq = 0.f;
#pragma unroll
            for (int c = 0; c < NSRC; ++c)
                if (c == g) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) sq = fmaf(src[c][e], src[c][e], sq);
                }
            put(kSq, sq);
        }
#pragma unroll
        for (int k = 0; k < kChunkReads; ++k) {
            const int l = l0 + k;
            if (k < n && l >= p.q_begin) {
                float wv[8];
                {
                    const rsrc_t wr = make_rsrc(p.w + (int64_t)(l - p.q_begin) * p.d, (uint64_t)p.d * 4);
                    Chunk<float> wc;
                    wc.load(wr, w_off);
                    wc.to_float(wv);
                }
                // phase 1: the frozen sources
#pragma unroll
                for (int c = 0; c < NSRC; ++c) {
                    if (c <= g) {
                        float dp = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) dp = fmaf(wv[e], src[c][e], dp);
                        put(k * kStride + c, dp);
                    }
                }
                // phase 2: the partial sum, when non-empty
                if (l != g * S) {
                    float dp = 0.f, sq = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        dp = fmaf(wv[e], pk[k][e], dp);
                        sq = fmaf(pk[k][e], pk[k][e], sq);
                    }
                    put(k * kStride + NSRC, dp);
                    put(k * kStride + NSRC + 1, sq);
                }
            }
        }
        __syncthreads();

        // ---- A3: finish the sums (fixed order over rows) ----------------------
        for (int v = tid; v < kVals; v += kThreads) {
            float s = 0.f;
#pragma unroll
            for (int r = 0; r < kRows; ++r) s += part[v * kRows + r];
            fin[v] = s;
        }
        __syncthreads();

        // ---- A4: scores, phase-1 softmax, phase-2 merge (one lane per read) ---
        if (tid < n && l0 + tid >= p.q_begin) {
            const int k = tid;
            const int l = l0 + k;
            float r_new = 0.f;
            if (new_src) r_new = fast_rsqrt(fmaf(fin[kSq], p.inv_d, p.eps));
            float s2[NSRC];
            float M1 = -INFINITY;
#pragma unroll
            for (int c = 0; c < NSRC; ++c) {
                if (c <= g) {
                    const float r = (new_src && c == g) ? r_new : rs[c];
                    s2[c] = r * fin[k * kStride + c] * kLog2e;
                    M1 = fmaxf(M1, s2[c]);
                }
            }
            float Z1 = 0.f;
#pragma unroll
            for (int c = 0; c < NSRC; ++c) {
                if (c <= g) {
                    s2[c] = fast_exp2(s2[c] - M1);
                    Z1 += s2[c];
                }
            }
            float M = M1, A = Z1, B = 0.f;
            if (l != g * S) {
                const float rp = fast_rsqrt(fmaf(fin[k * kStride + NSRC + 1], p.inv_d, p.eps));
                const float sp = rp * fin[k * kStride + NSRC] * kLog2e;
                M = fmaxf(M1, sp);
                A = Z1 * fast_exp2(M1 - M);
                B = fast_exp2(sp - M);
            }
            const float inv = 1.0f / (A + B);
            const float scale1 = fast_exp2(M1 - M) * inv;  // e^(s_c - M1) -> e^(s_c - M) / (A + B)
#pragma unroll
            for (int c = 0; c < NSRC; ++c)
                if (c <= g) coef[k * kStride + c] = s2[c] * scale1;
            coef[k * kStride + NSRC] = B * inv;
            if (p.lse != nullptr)
                p.lse[(int64_t)(l - p.q_begin) * p.T + t] = (M + fast_log2(A + B)) * kLn2;
        }
        if (new_src && tid == 0) rs[g] = fast_rsqrt(fmaf(fin[kSq], p.inv_d, p.eps));
        __syncthreads();

        // ---- B: outputs ------------------------------------------------------
#pragma unroll
        for (int k = 0; k < kChunkReads; ++k) {
            const int l = l0 + k;
            if (k < n && l >= p.q_begin) {
                float o[8];
                const float cp = l != g * S ? coef[k * kStride + NSRC] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = cp * pk[k][e];
#pragma unroll
                for (int c = 0; c < NSRC; ++c) {
                    if (c <= g) {
                        const float a = coef[k * kStride + c];
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[e] = fmaf(a, src[c][e], o[e]);
                    }
                }
                const rsrc_t orr =
                    make_rsrc(out_tok + (int64_t)(l - p.q_begin) * row_elems, tok_out_bytes);
                store_chunk((TO*)nullptr, orr, out_off, o);
            }
        }
        l0 = nl0;
        l1 = nl1;
    }
}

// ---------------------------------------------------------------------------
// launch selection

namespace {

template <typename TI, typename TO, int NW, int NSRC>
hipError_t launch_twophase(const BlockFwdParams& p, hipStream_t stream) {
    constexpr int kRows = 4 * NW;
    constexpr int kStride = BlockLds<NSRC>::kStride;
    constexpr int kVals = BlockLds<NSRC>::kVals;
    const size_t lds = sizeof(float) * (kVals * kRows + kVals + kChunkReads * kStride + NSRC);
    hipLaunchKernelGGL((block_fwd_twophase_kernel<TI, TO, NW, NSRC>), dim3((unsigned)p.T),
                       dim3(64 * NW), lds, stream, p);
    return hipGetLastError();
}

template <typename TI, typename TO, int NW>
hipError_t dispatch_nsrc(const BlockFwdParams& p, int nsrc, hipStream_t stream) {
    if (nsrc <= 5) return launch_twophase<TI, TO, NW, 5>(p, stream);
    if (nsrc <= 9) return launch_twophase<TI, TO, NW, 9>(p, stream);
    return launch_twophase<TI, TO, NW, 13>(p, stream);
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
