// full_batch.hip -- Full AttnRes forward for calls with many reads, on gfx950.
//
// Read l of a token sees its rows 0..l ("DepthBench reading notes" sec. 2.3),
// so the reads of one call share most of their rows.  Streaming each token's
// rows once per read (full_fwd.hip) moves about n_q / 2 times the token's
// history, and that working set -- rows x d per token, for the thousands of
// tokens in flight -- does not stay in L2.  This kernel brings every row of
// a token from HBM once, into LDS, and serves all of the token's reads from
// there.  When a token's rows exceed the LDS a workgroup may hold, the first
// n_lds rows are staged and the rest (needed only by the last groups of
// reads) are read from global memory in both passes.
//
// Mapping: one workgroup of kBatchWaves waves per token.
//   prologue  the waves copy rows 0..n_lds-1 into LDS (input type, row-major,
//             16-byte chunks along d) and form the RMS scale r_i of every row
//             the call sees: from the caller's cache when the row is valid
//             there, else from the row's sum of squares (then written to the
//             cache);
//   groups    the reads are cut into groups of R consecutive reads, which the
//             waves take from a workgroup counter, the group with the most
//             rows first.  A group is two passes over its rows:
//     A  the R dots w_l . v_i of each row, reduced over the wave; the scores
//        s = r_i (w_l . v_i) (log2 units) go to a per-wave LDS table; then,
//        per read, the exact softmax over its rows i <= l: max, sum, weights
//        written back in place (zero for i > l), log-sum-exp;
//     B  h_l = sum_i alpha_{l,i} v_i in fp32 registers, one rounding, stored
//        (and the optional pre-norm of the output, as in the streaming kernel).
// Lane `ln` owns the 16-byte chunks ln, ln + 64, ... of d, so every LDS row
// read is 64 consecutive chunks (no bank conflicts) and every output store
// is contiguous.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

constexpr int kBatchWaves = 8;
// Reads per group.  Groups of 8 halve the row visits but leave too few groups
// to balance the waves (49 reads: 7 groups for 8 waves, the longest on the
// critical path) and measured slower; 4 it is, one f32x4 per row of the
// score table.
constexpr int kBatchR = 4;
// Fewer reads than this share too few rows to pay for the staging and would
// leave most of the workgroup's waves without a group.
constexpr int kBatchMinReads = 16;

// 64-lane sums of R values, one DPP level at a time over all values so that
// independent operations sit between the dependent ones
template <int R>
__device__ __forceinline__ void wave_sum_multi(float (&v)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] += dpp<kDppXor1>(v[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] += dpp<kDppXor2>(v[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] += dpp<kDppHalfMirror>(v[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] += dpp<kDppMirror>(v[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = swap16_sum(v[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = swap32_sum(v[r]);
}

// raw 16-byte (bf16) or 32-byte (fp32) chunk of a row in LDS
template <typename TI> struct LdsChunk;
template <> struct LdsChunk<bf16_t> {
    u32x4 v;
    __device__ __forceinline__ void load(const bf16_t* row, int ch) {
        v = *reinterpret_cast<const u32x4*>(row + 8 * ch);
    }
    __device__ __forceinline__ void load_global(rsrc_t r, uint32_t off) {
        v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
    __device__ __forceinline__ void to_float(float (&f)[8]) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
        }
    }
};
template <> struct LdsChunk<float> {
    u32x4 a, b;
    __device__ __forceinline__ void load(const float* row, int ch) {
        a = *reinterpret_cast<const u32x4*>(row + 8 * ch);
        b = *reinterpret_cast<const u32x4*>(row + 8 * ch + 4);
    }
    __device__ __forceinline__ void load_global(rsrc_t r, uint32_t off) {
        a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
    }
    __device__ __forceinline__ void to_float(float (&f)[8]) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[q] = __uint_as_float(a[q]);
            f[4 + q] = __uint_as_float(b[q]);
        }
    }
};

__device__ __forceinline__ void store_raw(bf16_t* row, int ch, const Chunk<bf16_t>& c) {
    *reinterpret_cast<u32x4*>(row + 8 * ch) = c.v;
}
__device__ __forceinline__ void store_raw(float* row, int ch, const Chunk<float>& c) {
    *reinterpret_cast<u32x4*>(row + 8 * ch) = c.a;
    *reinterpret_cast<u32x4*>(row + 8 * ch + 4) = c.b;
}

// LDS layout of one workgroup: rows [n_lds][d] (input type), the RMS scales
// [n_pad], kBatchWaves score tables [n_pad][R], the group counter.
struct BatchLayout {
    int64_t rows_bytes, rs_off, tab_off, counter_off, bytes;
};
__host__ __device__ inline BatchLayout batch_layout(int n_lds, int n_pad, int d, int elem) {
    BatchLayout L;
    L.rows_bytes = (int64_t)n_lds * d * elem;  // d % 8 == 0: a multiple of 16
    L.rs_off = L.rows_bytes;
    L.tab_off = L.rs_off + (int64_t)n_pad * 4;  // n_pad % 4 == 0: 16-byte aligned
    L.counter_off = L.tab_off + (int64_t)kBatchWaves * n_pad * kBatchR * 4;
    L.bytes = L.counter_off + 16;
    return L;
}

template <typename TI, typename TO, int NCH>
__global__ __launch_bounds__(64 * kBatchWaves) void full_batch_kernel(FwdParams p, int n_rows, int n_lds,
                                                                      int n_pad) {
    constexpr int R = kBatchR;
    constexpr int RV = R / 4;  // f32x4 per row of the score table
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const BatchLayout L = batch_layout(n_lds, n_pad, p.d, (int)sizeof(TI));
    TI* const rows = reinterpret_cast<TI*>(lds_raw);
    float* const rs = reinterpret_cast<float*>(lds_raw + L.rs_off);
    int* const counter = reinterpret_cast<int*>(lds_raw + L.counter_off);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = threadIdx.x & 63;
    const int64_t t = blockIdx.x;
    const int d = p.d;
    const int64_t row_elems = p.T * (int64_t)d;
    const TI* hist_tok = static_cast<const TI*>(p.hist) + t * d;
    const uint64_t tok_bytes = (uint64_t)d * sizeof(TI);

    bool live[NCH];
    uint32_t in_off[NCH], out_off[NCH], w_off[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = c * 64 + ln;
        live[c] = ch < p.nc;
        in_off[c] = live[c] ? (uint32_t)(ch * 8 * sizeof(TI)) : kOOB;
        out_off[c] = live[c] ? (uint32_t)(ch * 8 * sizeof(TO)) : kOOB;
        w_off[c] = live[c] ? (uint32_t)(ch * 32) : kOOB;
    }
    if (threadIdx.x == 0) *counter = 0;

    // ---- prologue: the token's rows into LDS, their RMS scales ------------
    {
        constexpr int U = 4;  // rows in flight per wave
        const cf32_ptr cache = const_view(p.rinv);
        for (int ib = wave; ib < n_rows; ib += kBatchWaves * U) {
            Chunk<TI> ch[U][NCH];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = ib + u * kBatchWaves;
                if (i < n_rows) {
                    // staged rows are read from HBM once (non-temporal); rows past
                    // the LDS are read again by the passes and keep the default policy
                    const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, tok_bytes);
                    if (i < n_lds) {
#pragma unroll
                        for (int c = 0; c < NCH; ++c) ch[u][c].template load<kAuxNT>(rr, in_off[c]);
                    } else {
#pragma unroll
                        for (int c = 0; c < NCH; ++c) ch[u][c].load(rr, in_off[c]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = ib + u * kBatchWaves;
                if (i < n_rows) {
                    if (i < n_lds) {
                        TI* const row = rows + (int64_t)i * d;
#pragma unroll
                        for (int c = 0; c < NCH; ++c)
                            if (live[c]) store_raw(row, c * 64 + ln, ch[u][c]);
                    }
                    float r;
                    if (i < p.rinv_valid) {
                        r = cache[(int64_t)i * p.T + t];
                    } else {
                        float sq = 0.f;
#pragma unroll
                        for (int c = 0; c < NCH; ++c) {
                            float x[8];
                            ch[u][c].to_float(x);
#pragma unroll
                            for (int e = 0; e < 8; ++e) sq = fmaf(x[e], x[e], sq);
                        }
                        sq = tg_sum<64>(sq);
                        r = fast_rsqrt(fmaf(sq, p.inv_d, p.eps));
                        if (p.rinv != nullptr && ln == 0) p.rinv[(int64_t)i * p.T + t] = r;
                    }
                    if (ln == 0) rs[i] = r;
                }
            }
        }
    }
    __syncthreads();

    // Rows 0..l_max in order, one row ahead in flight: first the rows staged in
    // LDS, then (past n_lds) rows from global memory, in two loops so that each
    // loop's registers are filled by one kind of load only.
    auto walk_rows = [&](int l_max, auto&& body) {
        const int i_lds = l_max < n_lds - 1 ? l_max : n_lds - 1;  // last row in LDS
        {
            LdsChunk<TI> cur[NCH], nxt[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                if (live[c]) cur[c].load(rows, c * 64 + ln);
            for (int i = 0; i <= i_lds; ++i) {
                if (i < i_lds) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        if (live[c]) nxt[c].load(rows + (int64_t)(i + 1) * d, c * 64 + ln);
                }
                body(cur, i);
#pragma unroll
                for (int c = 0; c < NCH; ++c) cur[c] = nxt[c];
            }
        }
        if (i_lds < l_max) {
            auto issue = [&](LdsChunk<TI> (&dst)[NCH], int i) {
                const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, tok_bytes);
#pragma unroll
                for (int c = 0; c < NCH; ++c) dst[c].load_global(rr, in_off[c]);
            };
            LdsChunk<TI> cur[NCH], nxt[NCH];
            issue(cur, i_lds + 1);
            for (int i = i_lds + 1; i <= l_max; ++i) {
                if (i < l_max) issue(nxt, i + 1);
                body(cur, i);
#pragma unroll
                for (int c = 0; c < NCH; ++c) cur[c] = nxt[c];
            }
        }
    };

    // ---- groups of R reads ---------------------------------------------------
    f32x4* const tab = reinterpret_cast<f32x4*>(lds_raw + L.tab_off) + (int64_t)wave * n_pad * RV;
    float* const tabf = reinterpret_cast<float*>(tab);
    const int n_groups = (p.n_q + R - 1) / R;
    for (;;) {
        int idx = 0;
        if (ln == 0) idx = atomicAdd(counter, 1);
        idx = __builtin_amdgcn_readfirstlane(idx);
        if (idx >= n_groups) break;
        const int g = n_groups - 1 - idx;  // the group with the most rows first
        const int j0 = g * R;
        const int nr = p.n_q - j0 < R ? p.n_q - j0 : R;  // reads in this group
        const int l0 = p.q_begin + j0;                    // read of the group's first query
        const int l_max = l0 + nr - 1;                    // rows 0..l_max

        float wv[R][NCH][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const rsrc_t wr = make_rsrc(p.w + (int64_t)(j0 + r) * d, r < nr ? (uint64_t)d * 4 : 0);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                Chunk<float> q;
                q.load(wr, w_off[c]);
                q.to_float(wv[r][c]);
            }
        }

        // pass A: scores
        walk_rows(l_max, [&](const LdsChunk<TI> (&cur)[NCH], int i) {
                float dot[R];
#pragma unroll
                for (int r = 0; r < R; ++r) dot[r] = 0.f;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    if (!live[c]) continue;
                    float x[8];
                    cur[c].to_float(x);
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e) dot[r] = fmaf(wv[r][c][e], x[e], dot[r]);
                }
                const float tot = wave_sum_transposed<4>(dot, ln);
                if (wave_sum_holder<4>(ln)) {
                    const int r = ln & 3;
                    tabf[i * R + r] = (r < nr && i <= l0 + r) ? rs[i] * kLog2e * tot : -INFINITY;
                }
        });
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // exact softmax of each read over its rows; weights written in place
        float M[R], Z[R];
#pragma unroll
        for (int r = 0; r < R; ++r) M[r] = -INFINITY;
        for (int i = ln; i <= l_max; i += 64) {
#pragma unroll
            for (int q = 0; q < RV; ++q) {
                const f32x4 s = tab[i * RV + q];
#pragma unroll
                for (int r = 0; r < 4; ++r) M[4 * q + r] = fmaxf(M[4 * q + r], s[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            M[r] = tg_max<64>(M[r]);
            if (r >= nr) M[r] = 0.f;  // no such read: keep exp2 finite, weights zero
            Z[r] = 0.f;
        }
        for (int i = ln; i <= l_max; i += 64) {
#pragma unroll
            for (int q = 0; q < RV; ++q) {
                const f32x4 s = tab[i * RV + q];
#pragma unroll
                for (int r = 0; r < 4; ++r) Z[4 * q + r] += fast_exp2(s[r] - M[4 * q + r]);
            }
        }
        wave_sum_multi<R>(Z);
        float inv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) inv[r] = r < nr ? 1.0f / Z[r] : 0.f;
        for (int i = ln; i <= l_max; i += 64) {
#pragma unroll
            for (int q = 0; q < RV; ++q) {
                const f32x4 s = tab[i * RV + q];
                f32x4 a;
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = fast_exp2(s[r] - M[4 * q + r]) * inv[4 * q + r];
                tab[i * RV + q] = a;
                if (p.alpha != nullptr) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * q + r < nr)
                            p.alpha[((int64_t)(j0 + 4 * q + r) * p.n_hist + i) * p.T + t] = a[r];
                }
            }
        }
        if (p.alpha != nullptr) {  // sources a read does not see
            for (int i = l_max + 1 + ln; i < p.n_hist; i += 64)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (r < nr) p.alpha[((int64_t)(j0 + r) * p.n_hist + i) * p.T + t] = 0.f;
        }
        if (p.lse != nullptr && ln == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (r < nr) p.lse[(int64_t)(j0 + r) * p.T + t] = (M[r] + fast_log2(Z[r])) * kLn2;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // pass B: the weighted sums
        float acc[R][NCH][8];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][c][e] = 0.f;
        walk_rows(l_max, [&](const LdsChunk<TI> (&cur)[NCH], int i) {
                float a[R];
#pragma unroll
                for (int q = 0; q < RV; ++q) {
                    const f32x4 a4 = tab[i * RV + q];
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[4 * q + r] = a4[r];
                }
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    if (!live[c]) continue;
                    float x[8];
                    cur[c].to_float(x);
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[r][c][e] = fmaf(a[r], x[e], acc[r][c][e]);
                }
        });
        // the next group rewrites this wave's table only after these reads
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();

#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r >= nr) continue;
            const int j = j0 + r;
            const rsrc_t orr = make_rsrc(static_cast<TO*>(p.out) + (int64_t)j * row_elems + t * d,
                                         (uint64_t)d * sizeof(TO));
#pragma unroll
            for (int c = 0; c < NCH; ++c) store_chunk((TO*)nullptr, orr, out_off[c], acc[r][c]);
            if (p.normed != nullptr) {  // fused pre-norm of the output (uniform branch)
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss = fmaf(acc[r][c][e], acc[r][c][e], ss);
                ss = tg_sum<64>(ss);
                const float rn = fast_rsqrt(fmaf(ss, p.inv_d, p.eps));
                const rsrc_t nrr = make_rsrc(static_cast<TO*>(p.normed) + (int64_t)j * row_elems + t * d,
                                             (uint64_t)d * sizeof(TO));
                const rsrc_t grr = make_rsrc(p.norm_gain + (int64_t)j * d,
                                             p.norm_gain != nullptr ? (uint64_t)d * 4 : 0);
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    float gn[8];
                    if (p.norm_gain != nullptr) {
                        Chunk<float> gc;
                        gc.load(grr, w_off[c]);
                        gc.to_float(gn);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) gn[e] = 1.f;
                    }
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = gn[e] * (acc[r][c][e] * rn);
                    store_chunk((TO*)nullptr, nrr, out_off[c], y);
                }
            }
        }
    }
}

template <typename TI, typename TO, int NCH>
hipError_t launch_batch(const FwdParams& p, int n_rows, int n_lds, int n_pad, size_t lds,
                        hipStream_t stream) {
    const hipError_t e = prepare_dynamic_lds((const void*)full_batch_kernel<TI, TO, NCH>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((full_batch_kernel<TI, TO, NCH>), dim3((unsigned)p.T), dim3(64 * kBatchWaves), lds,
                       stream, p, n_rows, n_lds, n_pad);
    return hipGetLastError();
}

template <typename TI, typename TO>
hipError_t dispatch_batch(const FwdParams& p, int n_rows, int n_lds, int n_pad, size_t lds,
                          hipStream_t stream) {
    switch ((p.nc + 63) / 64) {
        case 1: return launch_batch<TI, TO, 1>(p, n_rows, n_lds, n_pad, lds, stream);
        case 2: return launch_batch<TI, TO, 2>(p, n_rows, n_lds, n_pad, lds, stream);
        case 3: return launch_batch<TI, TO, 3>(p, n_rows, n_lds, n_pad, lds, stream);
        case 4:
            if constexpr (sizeof(TI) == 2) return launch_batch<TI, TO, 4>(p, n_rows, n_lds, n_pad, lds, stream);
            return hipErrorInvalidValue;  // fp32 rows: batch_plan stops at 3
        default: return hipErrorInvalidValue;
    }
}

// Whether a call qualifies, and how many of its rows go to LDS.
struct BatchPlan {
    bool ok;
    int n_rows, n_lds, n_pad;
    size_t lds;
};

BatchPlan batch_plan(const FwdParams& p, attnres_dtype hist_dt) {
    BatchPlan b{false, 0, 0, 0, 0};
    if (p.qtok != nullptr || p.n_q < kBatchMinReads) return b;
    // chunks per lane: up to 4 (bf16) or 3 (fp32 rows need twice the registers)
    if (p.nc > (hist_dt == ATTNRES_BF16 ? 4 : 3) * 64) return b;
    // one workgroup of 64 * kBatchWaves work-items per token, in a 32-bit grid
    if (p.T * 64 * kBatchWaves >= ((int64_t)1 << 32)) return b;
    const int max_lds = device_max_lds();
    if (max_lds <= 0) return b;
    const int elem = hist_dt == ATTNRES_BF16 ? 2 : 4;
    b.n_rows = p.q_begin + p.n_q;
    b.n_pad = (b.n_rows + 3) & ~3;
    const int64_t room = (int64_t)max_lds - batch_layout(0, b.n_pad, p.d, elem).bytes;
    const int64_t fit = room > 0 ? room / ((int64_t)p.d * elem) : 0;
    b.n_lds = fit < b.n_rows ? (int)fit : b.n_rows;
    // rows past n_lds are read from global memory in both passes of every group
    // that sees them: worth it while at least two thirds of the rows are staged
    if (3 * (int64_t)b.n_lds < 2 * (int64_t)b.n_rows) return b;
    b.lds = (size_t)batch_layout(b.n_lds, b.n_pad, p.d, elem).bytes;
    b.ok = true;
    return b;
}

}  // namespace

bool full_batch_applies(const FwdParams& p, attnres_dtype hist_dt) { return batch_plan(p, hist_dt).ok; }

hipError_t launch_full_batch(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt,
                             hipStream_t stream) {
    const BatchPlan b = batch_plan(p, hist_dt);
    if (!b.ok) return hipErrorInvalidValue;
    if (hist_dt == ATTNRES_BF16 && out_dt == ATTNRES_BF16)
        return dispatch_batch<bf16_t, bf16_t>(p, b.n_rows, b.n_lds, b.n_pad, b.lds, stream);
    if (hist_dt == ATTNRES_BF16 && out_dt == ATTNRES_F32)
        return dispatch_batch<bf16_t, float>(p, b.n_rows, b.n_lds, b.n_pad, b.lds, stream);
    if (hist_dt == ATTNRES_F32 && out_dt == ATTNRES_F32)
        return dispatch_batch<float, float>(p, b.n_rows, b.n_lds, b.n_pad, b.lds, stream);
    return dispatch_batch<float, bf16_t>(p, b.n_rows, b.n_lds, b.n_pad, b.lds, stream);
}

}  // namespace attnres
