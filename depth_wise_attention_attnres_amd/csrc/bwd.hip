// bwd.hip -- AttnRes backward on gfx950 (Full = Block with S = 1).
//
// The pages state no gradient; this is the derivative of the forward read
// ("DepthBench reading notes" sec. 2.3; block reading of sec. 2.5 and of the
// DataCamp block section).  For one token and read l with upstream gradient
// g = dL/dh_l, over the read's sources x (v_0, block sums, partial sum):
//   s_x = r_x (w_l . x),  alpha = softmax_x(s),  a_x = g . x,
//   delta = sum_x alpha_x a_x,  ds_x = alpha_x (a_x - delta),
//   dL/dx  = alpha_x g + ds_x r_x w_l - (ds_x r_x^2 s_x / d) x,
//   dL/dw_l = sum_x ds_x r_x x.
// A source that is a sum of history rows passes dL/dx to every row in it.
//
// Per token this becomes: row coefficients A1[l][i] = alpha of the source of
// read l that contains row i, A2[l][i] = ds r of that source, and the "-k x"
// terms, which couple the rows of one source:
//   dv_i = sum_l (A1[l][i] g_l + A2[l][i] w_l)
//          - C3[src] x_src                       (v_0 or a block sum, summed over reads)
//          - sum over reads whose partial holds row i of kappa_l p_l
//   dw_l = sum_t sum_i A2[t][l][i] v_{t,i}.
// Kernels:
//   bwd_scores  one wave per token: streams the token's rows once per pass of
//               R reads (block sums formed on the fly in fp32), reduces the
//               score and gradient dots of every source for the pass's reads
//               across the wave, renormalises each read's softmax over its own
//               scores (a single source gets alpha = 1 exactly), forms ds, and
//               writes A1, A2 (row-major and transposed), C3 and kappa.
//   bwd_dhist   one wave per (token, 128-column slice of d): accumulates
//               dv for 64-row tiles in registers (coefficients are uniform
//               across the wave, so they come through the scalar cache),
//               then adds the source-coupling terms with a forward (prefix)
//               and a backward (suffix) pass over each block, and stores dhist.
//   bwd_dw_part one wave per (128-column slice, chunk of 32 tokens):
//               per-chunk partial dw for 64-read tiles.
//   bwd_dw_sum  fixed-order sum of the partials (bitwise reproducible).
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

constexpr int kSlice = 128;   // columns of d per wave in bwd_dhist / bwd_dw_part
constexpr int kRowTile = 64;  // rows (or reads) accumulated in registers at once
constexpr int kChunkTokens = 32;

// two consecutive elements of a row
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
    __device__ __forceinline__ static void load(rsrc_t r, uint32_t off, float& a, float& b) {
        const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        a = __uint_as_float(u << 16);
        b = __uint_as_float(u & 0xffff0000u);
    }
    __device__ __forceinline__ static void store(rsrc_t r, uint32_t off, float a, float b) {
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(a, b), r, off, 0, 0);
    }
};
template <> struct Pair<float> {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __device__ __forceinline__ static void load(rsrc_t r, uint32_t off, float& a, float& b) {
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        a = __uint_as_float(u[0]);
        b = __uint_as_float(u[1]);
    }
    __device__ __forceinline__ static void store(rsrc_t r, uint32_t off, float a, float b) {
        const u32x2 u = {__float_as_uint(a), __float_as_uint(b)};
        __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
    }
};

// index of the source of read l that contains row i (i <= l)
__device__ __forceinline__ int src_of(int l, int i, int S) {
    if (i == 0) return 0;
    const int c = (i - 1) / S + 1;  // block of row i
    const int m = l / S;            // completed blocks seen by read l
    return c <= m ? c : m + 1;      // the block, or the partial sum
}

}  // namespace

// ---------------------------------------------------------------------------
// bwd_scores: one wave (= one workgroup) per token.  Reads are processed R
// at a time: one pass over the token's rows 0..l_max forms every source once
// (v_0, block sums, the partial sums of the pass's reads) and scores it
// against all reads of the pass that see it, so the rows are streamed
// n_q / R times instead of n_q times.

template <typename TI, typename TG, int NCH, int PF, int R>
__global__ __launch_bounds__(64) void bwd_scores_kernel(BwdParams p) {
    const int ln = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int S = p.S;

    extern __shared__ float lds[];
    // per read of the pass and source: a = g.x, r, s (score); then alpha, c1, c2
    float* v_a = lds;                      // [R][nx]
    float* v_r = v_a + R * p.nx;
    float* v_s = v_r + R * p.nx;
    float* v_alpha = v_s + R * p.nx;
    float* c1s = v_alpha + R * p.nx;
    float* c2s = c1s + R * p.nx;
    float* c3acc = c2s + R * p.nx;         // [n_blk] summed over reads

    for (int i = ln; i < p.n_blk; i += 64) c3acc[i] = 0.f;

    const int64_t row_elems = p.T * (int64_t)p.d;
    const TI* hist_tok = static_cast<const TI*>(p.hist) + t * p.d;
    const TG* dout_tok = static_cast<const TG*>(p.dout) + t * p.d;
    uint32_t h_off[NCH], g_off[NCH], w_off[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = c * 64 + ln;
        h_off[c] = ch < p.nc ? (uint32_t)(ch * 8 * sizeof(TI)) : kOOB;
        g_off[c] = ch < p.nc ? (uint32_t)(ch * 8 * sizeof(TG)) : kOOB;
        w_off[c] = ch < p.nc ? (uint32_t)(ch * 32) : kOOB;
    }
    const uint64_t h_bytes = (uint64_t)p.d * sizeof(TI);

    float* A1 = p.ws_a1 + t * (int64_t)p.n_q * p.nh8;
    float* A2 = p.ws_a2 + t * (int64_t)p.n_q * p.nh8;
    float* A2T = p.ws_a2t + t * (int64_t)p.n_hist * p.n_q;

    for (int lq0 = 0; lq0 < p.n_q; lq0 += R) {
        const int nr = p.n_q - lq0 < R ? p.n_q - lq0 : R;  // reads in this pass
        const int l_lo = p.q_begin + lq0;                 // first read of the pass
        const int l_hi = l_lo + nr - 1;                   // last read of the pass
        float wv[R][NCH][8], gv[R][NCH][8];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int lq = q < nr ? lq0 + q : lq0;  // a valid row; unused when q >= nr
            const rsrc_t wr = make_rsrc(p.w + (int64_t)lq * p.d, (uint64_t)p.d * 4);
            const rsrc_t gr = make_rsrc(dout_tok + (int64_t)lq * row_elems, (uint64_t)p.d * sizeof(TG));
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                Chunk<float> wc;
                wc.load(wr, w_off[c]);
                wc.to_float(wv[q][c]);
                Chunk<TG> gc;
                gc.load(gr, g_off[c]);
                gc.to_float(gv[q][c]);
            }
        }
        int nsrc[R];
#pragma unroll
        for (int q = 0; q < R; ++q) nsrc[q] = 0;
        float run[NCH][8];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) run[c][e] = 0.f;

        Chunk<TI> buf[PF][NCH];
#pragma unroll
        for (int u = 0; u < PF; ++u)
#pragma unroll
            for (int c = 0; c < NCH; ++c) buf[u][c].zero();
        auto issue = [&](int u, int i) {
            const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, h_bytes);
#pragma unroll
            for (int c = 0; c < NCH; ++c) buf[u][c].load(rr, h_off[c]);
        };
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (u <= l_hi) issue(u, u);

        for (int i0 = 0; i0 <= l_hi; i0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int i = i0 + u;
                if (i > l_hi) break;
                float xf[NCH][8];
#pragma unroll
                for (int c = 0; c < NCH; ++c) buf[u][c].to_float(xf[c]);
                if (i + PF <= l_hi) issue(u, i + PF);
                // which reads of the pass see the source emitted at row i:
                // v_0 or a block closing at i -> every read l >= i; otherwise
                // the partial sum of read l = i (if that read is in the pass)
                bool block_src = true;
                if (i > 0) {
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            run[c][e] += xf[c][e];
                            xf[c][e] = run[c][e];
                        }
                    block_src = (i % S == 0);
                    if (!block_src && (i < l_lo || i > l_hi)) continue;
                    if (block_src) {
#pragma unroll
                        for (int c = 0; c < NCH; ++c)
#pragma unroll
                            for (int e = 0; e < 8; ++e) run[c][e] = 0.f;
                    }
                }
                float sq = 0.f;
                float wx[R], gx[R];
#pragma unroll
                for (int q = 0; q < R; ++q) wx[q] = gx[q] = 0.f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sq = fmaf(xf[c][e], xf[c][e], sq);
#pragma unroll
                        for (int q = 0; q < R; ++q) {
                            wx[q] = fmaf(wv[q][c][e], xf[c][e], wx[q]);
                            gx[q] = fmaf(gv[q][c][e], xf[c][e], gx[q]);
                        }
                    }
                sq = tg_sum<64>(sq);
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    wx[q] = tg_sum<64>(wx[q]);
                    gx[q] = tg_sum<64>(gx[q]);
                }
                const float r = fast_rsqrt(fmaf(sq, p.inv_d, p.eps));
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    const int l = l_lo + q;
                    const bool sees = q < nr && (block_src ? l >= i : l == i);
                    if (sees) {
                        if (ln == 0) {
                            v_a[q * p.nx + nsrc[q]] = gx[q];
                            v_r[q * p.nx + nsrc[q]] = r;
                            v_s[q * p.nx + nsrc[q]] = r * wx[q];
                        }
                        ++nsrc[q];
                    }
                }
            }
        }
        __syncthreads();

        for (int q = 0; q < nr; ++q) {
            const int lq = lq0 + q;
            const int l = l_lo + q;
            const int ns = nsrc[q];
            float* va = v_a + q * p.nx;
            float* vr = v_r + q * p.nx;
            float* vs = v_s + q * p.nx;
            float* val = v_alpha + q * p.nx;
            float* cc1 = c1s + q * p.nx;
            float* cc2 = c2s + q * p.nx;
            // softmax over the read's sources (lanes hold sources ln, ln + 64, ...)
            float mx = -INFINITY;
            for (int xs = ln; xs < ns; xs += 64) mx = fmaxf(mx, vs[xs]);
            mx = tg_max<64>(mx);
            float z = 0.f;
            for (int xs = ln; xs < ns; xs += 64) {
                const float e = fast_exp2((vs[xs] - mx) * kLog2e);
                val[xs] = e;
                z += e;
            }
            z = tg_sum<64>(z);
            const float inv_z = 1.0f / z;
            float delta = 0.f;
            for (int xs = ln; xs < ns; xs += 64) {
                const float alpha = val[xs] * inv_z;
                val[xs] = alpha;
                delta = fmaf(alpha, va[xs], delta);
            }
            delta = tg_sum<64>(delta);

            const int m = l / S;
            for (int xs = ln; xs < ns; xs += 64) {
                const float alpha = val[xs], r = vr[xs];
                const float ds = alpha * (va[xs] - delta);
                cc1[xs] = alpha;
                cc2[xs] = ds * r;
                const float c3 = ds * r * r * vs[xs] * p.inv_d;
                if (xs <= m)
                    c3acc[xs] += c3;  // v_0 or a block sum: same lane for a slot on every read
                else
                    p.ws_kappa[t * p.n_q + lq] = c3;  // the partial sum of this read
            }
            if (ln == 0 && l % S == 0) p.ws_kappa[t * p.n_q + lq] = 0.f;  // no partial
        }
        __syncthreads();

        for (int q = 0; q < nr; ++q) {
            const int lq = lq0 + q;
            const int l = l_lo + q;
            for (int i = ln; i < p.nh8; i += 64) {
                float c1 = 0.f, c2 = 0.f;
                if (i <= l) {
                    const int xs = src_of(l, i, S);
                    c1 = c1s[q * p.nx + xs];
                    c2 = c2s[q * p.nx + xs];
                }
                A1[(int64_t)lq * p.nh8 + i] = c1;
                A2[(int64_t)lq * p.nh8 + i] = c2;
                if (i < p.n_hist) A2T[(int64_t)i * p.n_q + lq] = c2;
            }
        }
        __syncthreads();
    }
    for (int i = ln; i < p.n_blk; i += 64) p.ws_c3[t * p.n_blk + i] = c3acc[i];
}

// ---------------------------------------------------------------------------
// bwd_dhist: one wave per (128-column slice, token).

template <typename TI, typename TG, typename TO>
__global__ __launch_bounds__(64) void bwd_dhist_kernel(BwdParams p) {
    const int ln = threadIdx.x;
    const int e0 = blockIdx.y * kSlice + 2 * ln;  // this lane's two columns
    const int64_t t = blockIdx.x;
    const bool valid = e0 < p.d;
    const int S = p.S;
    const int q_end = p.q_begin + p.n_q;

    const int64_t row_elems = p.T * (int64_t)p.d;
    const TI* hist_tok = static_cast<const TI*>(p.hist) + t * p.d;
    const TG* dout_tok = static_cast<const TG*>(p.dout) + t * p.d;
    TO* dh_tok = static_cast<TO*>(p.dhist) + t * p.d;
    const uint32_t h_off = valid ? (uint32_t)(e0 * sizeof(TI)) : kOOB;
    const uint32_t g_off = valid ? (uint32_t)(e0 * sizeof(TG)) : kOOB;
    const uint32_t o_off = valid ? (uint32_t)(e0 * sizeof(TO)) : kOOB;
    const uint32_t w_off = valid ? (uint32_t)(e0 * 4) : kOOB;

    const float* __restrict__ A1 = p.ws_a1 + t * (int64_t)p.n_q * p.nh8;
    const float* __restrict__ A2 = p.ws_a2 + t * (int64_t)p.n_q * p.nh8;
    const float* __restrict__ C3 = p.ws_c3 + t * p.n_blk;
    const float* __restrict__ kap = p.ws_kappa + t * p.n_q;

    auto load_row = [&](int i, float& a, float& b) {
        const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, (uint64_t)p.d * sizeof(TI));
        Pair<TI>::load(rr, h_off, a, b);
    };
    // kappa of read l (0 for reads outside the call)
    auto kappa = [&](int l) { return (l >= p.q_begin && l < q_end) ? kap[l - p.q_begin] : 0.f; };

    for (int rt0 = 0; rt0 < p.n_hist; rt0 += kRowTile) {
        float dv[kRowTile][2];
#pragma unroll
        for (int i = 0; i < kRowTile; ++i) dv[i][0] = dv[i][1] = 0.f;

        // value path and query path: sum over the reads that see a row of the tile
        const int lq0 = rt0 > p.q_begin ? rt0 - p.q_begin : 0;
        for (int lq = lq0; lq < p.n_q; ++lq) {
            const int l = p.q_begin + lq;
            float g0, g1, w0, w1;
            {
                const rsrc_t gr = make_rsrc(dout_tok + (int64_t)lq * row_elems, (uint64_t)p.d * sizeof(TG));
                Pair<TG>::load(gr, g_off, g0, g1);
                const rsrc_t wr = make_rsrc(p.w + (int64_t)lq * p.d, (uint64_t)p.d * 4);
                Pair<float>::load(wr, w_off, w0, w1);
            }
            const float* a1 = A1 + (int64_t)lq * p.nh8 + rt0;
            const float* a2 = A2 + (int64_t)lq * p.nh8 + rt0;
#pragma unroll
            for (int q8 = 0; q8 < kRowTile / 8; ++q8) {
                if (rt0 + 8 * q8 <= l) {  // rows past l have zero coefficients
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int i = 8 * q8 + q;
                        const float c1 = a1[i], c2 = a2[i];
                        dv[i][0] = fmaf(c1, g0, fmaf(c2, w0, dv[i][0]));
                        dv[i][1] = fmaf(c1, g1, fmaf(c2, w1, dv[i][1]));
                    }
                }
            }
        }

        // source-coupling terms.  Row j of block c (rows j0..j1; v_0 is a block
        // of its own) gets  sum over rows m of the block of coef(j, m) v_m  with
        //   coef(j, m) = C3[c] + K(max(j, m)),  K(m) = sum of kappa_l, l = m..Lc,
        // Lc the last read whose partial sum holds row m (K = 0 past Lc).  Split
        // into a forward pass (m <= j: (C3[c] + K(j)) times the prefix sum) and
        // a backward pass (m > j: suffix of (C3[c] + K(m)) v_m).
        const int rt1 = rt0 + kRowTile < p.n_hist ? rt0 + kRowTile : p.n_hist;  // tile end
        auto block_of = [&](int j) { return j == 0 ? 0 : (j - 1) / S + 1; };
        auto block_first = [&](int c) { return c == 0 ? 0 : (c - 1) * S + 1; };
        auto block_last = [&](int c) {
            if (c == 0) return 0;
            return c * S < p.n_hist - 1 ? c * S : p.n_hist - 1;
        };
        auto coef_of = [&](int j) {  // C3[c] + K(j) for row j
            const int c = block_of(j);
            float K = 0.f;
            if (c > 0) {
                const int Lc = c * S - 1 < q_end - 1 ? c * S - 1 : q_end - 1;
                for (int l = j; l <= Lc; ++l) K += kappa(l);
            }
            return C3[c] + K;
        };
        __shared__ float coef_t[kRowTile];
        if (rt0 + ln < rt1) coef_t[ln] = coef_of(rt0 + ln);
        __syncthreads();

        // forward pass: prefix sums within blocks
        float pf0 = 0.f, pf1 = 0.f;
        {
            const int c = block_of(rt0);
            for (int m = block_first(c); m < rt0; ++m) {  // rows of the block in earlier tiles
                float u0, u1;
                load_row(m, u0, u1);
                pf0 += u0;
                pf1 += u1;
            }
        }
#pragma unroll
        for (int ii = 0; ii < kRowTile; ++ii) {
            const int j = rt0 + ii;
            if (j < rt1) {
                if (ii > 0 && j == block_first(block_of(j))) pf0 = pf1 = 0.f;
                float v0, v1;
                load_row(j, v0, v1);
                pf0 += v0;
                pf1 += v1;
                const float k = coef_t[ii];
                dv[ii][0] = fmaf(-k, pf0, dv[ii][0]);
                dv[ii][1] = fmaf(-k, pf1, dv[ii][1]);
            }
        }
        // backward pass: suffix sums within blocks
        float bs0 = 0.f, bs1 = 0.f;
        {
            const int c = block_of(rt1 - 1);
            for (int m = block_last(c); m >= rt1; --m) {  // rows of the block in later tiles
                float u0, u1;
                load_row(m, u0, u1);
                const float k = coef_of(m);
                bs0 = fmaf(k, u0, bs0);
                bs1 = fmaf(k, u1, bs1);
            }
        }
#pragma unroll
        for (int ii = kRowTile - 1; ii >= 0; --ii) {
            const int j = rt0 + ii;
            if (j < rt1) {
                dv[ii][0] -= bs0;
                dv[ii][1] -= bs1;
                if (j == block_first(block_of(j))) {
                    bs0 = bs1 = 0.f;
                } else {
                    float v0, v1;
                    load_row(j, v0, v1);
                    const float k = coef_t[ii];
                    bs0 = fmaf(k, v0, bs0);
                    bs1 = fmaf(k, v1, bs1);
                }
            }
        }
        __syncthreads();  // coef_t is rewritten by the next tile

#pragma unroll
        for (int ii = 0; ii < kRowTile; ++ii) {
            const int j = rt0 + ii;
            if (j < rt1) {
                const rsrc_t orr = make_rsrc(dh_tok + j * row_elems, (uint64_t)p.d * sizeof(TO));
                Pair<TO>::store(orr, o_off, dv[ii][0], dv[ii][1]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_dw_part: one wave per (128-column slice, chunk of tokens).

template <typename TI>
__global__ __launch_bounds__(64) void bwd_dw_part_kernel(BwdParams p) {
    const int ln = threadIdx.x;
    const int e0 = blockIdx.x * kSlice + 2 * ln;
    const int chunk = blockIdx.y;
    const bool valid = e0 < p.d;
    const uint32_t h_off = valid ? (uint32_t)(e0 * sizeof(TI)) : kOOB;
    const int64_t row_elems = p.T * (int64_t)p.d;
    const int64_t t_lo = (int64_t)chunk * kChunkTokens;
    const int64_t t_hi = t_lo + kChunkTokens < p.T ? t_lo + kChunkTokens : p.T;

    for (int qt0 = 0; qt0 < p.n_q; qt0 += kRowTile) {
        float acc[kRowTile][2];
#pragma unroll
        for (int q = 0; q < kRowTile; ++q) acc[q][0] = acc[q][1] = 0.f;
        const int l_max = p.q_begin + (qt0 + kRowTile < p.n_q ? qt0 + kRowTile : p.n_q) - 1;
        for (int64_t t = t_lo; t < t_hi; ++t) {
            const TI* hist_tok = static_cast<const TI*>(p.hist) + t * p.d;
            const float* __restrict__ a2t = p.ws_a2t + t * (int64_t)p.n_hist * p.n_q + qt0;
            for (int i = 0; i <= l_max; ++i) {
                float v0, v1;
                const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, (uint64_t)p.d * sizeof(TI));
                Pair<TI>::load(rr, h_off, v0, v1);
                const float* a = a2t + (int64_t)i * p.n_q;
#pragma unroll
                for (int q8 = 0; q8 < kRowTile / 8; ++q8) {
                    if (qt0 + 8 * q8 < p.n_q) {
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int qq = 8 * q8 + q;
                            const float c = qt0 + qq < p.n_q ? a[qq] : 0.f;
                            acc[qq][0] = fmaf(c, v0, acc[qq][0]);
                            acc[qq][1] = fmaf(c, v1, acc[qq][1]);
                        }
                    }
                }
            }
        }
        if (valid) {
            float* part = p.ws_dwpart + (int64_t)chunk * p.n_q * p.d;
#pragma unroll
            for (int q = 0; q < kRowTile; ++q) {
                if (qt0 + q < p.n_q) {
                    part[(int64_t)(qt0 + q) * p.d + e0] = acc[q][0];
                    part[(int64_t)(qt0 + q) * p.d + e0 + 1] = acc[q][1];
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void bwd_dw_sum_kernel(BwdParams p, int n_chunks) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.n_q * p.d;
    if (idx >= total) return;
    float s = 0.f;
    for (int c = 0; c < n_chunks; ++c) s += p.ws_dwpart[(int64_t)c * total + idx];
    p.dw[idx] = s;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* dst, int64_t n_words) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_words; i += stride) dst[i] = 0u;
}

hipError_t launch_fill_zero(void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t words = bytes / 4;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<uint32_t*>(dst), words);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// workspace and launch

BwdLayout bwd_layout(int64_t S, int64_t n_hist, int64_t T, int64_t d, int64_t n_q) {
    BwdLayout L;
    auto up = [](int64_t x, int64_t a) { return (x + a - 1) / a * a; };
    L.nh8 = up(n_hist, 8);
    L.n_blk = 1 + (n_hist - 1 + S - 1) / S;
    L.nx = 1 + (n_hist - 1) / S + 1;
    L.n_chunks = (T + kChunkTokens - 1) / kChunkTokens;
    int64_t off = 0;
    auto take = [&](int64_t floats) {
        const int64_t o = off;
        off += up(floats * 4, 256);
        return o;
    };
    L.off_a1 = take(T * n_q * L.nh8);
    L.off_a2 = take(T * n_q * L.nh8);
    L.off_a2t = take(T * n_hist * n_q);
    L.off_c3 = take(T * L.n_blk);
    L.off_kappa = take(T * n_q);
    L.off_dwpart = take(L.n_chunks * n_q * d);
    L.bytes = off;
    return L;
}

namespace {

template <typename TI, typename TG>
hipError_t launch_scores(const BwdParams& p, hipStream_t stream) {
    const int nch = (p.nc + 63) / 64;
    switch (nch) {
#define ATTNRES_SCORES(N, PF, R)                                                          \
    case N:                                                                               \
        hipLaunchKernelGGL((bwd_scores_kernel<TI, TG, N, PF, R>), dim3((unsigned)p.T),   \
                           dim3(64), sizeof(float) * (6 * (size_t)R * p.nx + p.n_blk),    \
                           stream, p);                                                    \
        break;
        ATTNRES_SCORES(1, 4, 4)
        ATTNRES_SCORES(2, 2, 4)
        ATTNRES_SCORES(3, 2, 2)
        ATTNRES_SCORES(4, 2, 2)
        ATTNRES_SCORES(5, 1, 1)
        ATTNRES_SCORES(6, 1, 1)
        ATTNRES_SCORES(7, 1, 1)
        ATTNRES_SCORES(8, 1, 1)
#undef ATTNRES_SCORES
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TI, typename TG, typename TO>
hipError_t launch_rest(const BwdParams& p, int n_chunks, hipStream_t stream) {
    const unsigned slices = (unsigned)((p.d + kSlice - 1) / kSlice);
    hipLaunchKernelGGL((bwd_dhist_kernel<TI, TG, TO>), dim3((unsigned)p.T, slices), dim3(64), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dw_part_kernel<TI>), dim3(slices, (unsigned)n_chunks), dim3(64), 0,
                       stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)p.n_q * p.d;
    hipLaunchKernelGGL(bwd_dw_sum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, p, n_chunks);
    return hipGetLastError();
}

template <typename TI, typename TG>
hipError_t dispatch_out(const BwdParams& p, int n_chunks, hipStream_t stream) {
    return p.dhist_dt == ATTNRES_BF16 ? launch_rest<TI, TG, bf16_t>(p, n_chunks, stream)
                                      : launch_rest<TI, TG, float>(p, n_chunks, stream);
}

template <typename TI, typename TG>
hipError_t run_bwd(const BwdParams& p, int n_chunks, hipStream_t stream) {
    hipError_t e = launch_scores<TI, TG>(p, stream);
    if (e != hipSuccess) return e;
    return dispatch_out<TI, TG>(p, n_chunks, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int n_chunks, hipStream_t stream) {
    if (p.hist_dt == ATTNRES_BF16)
        return p.dout_dt == ATTNRES_BF16 ? run_bwd<bf16_t, bf16_t>(p, n_chunks, stream)
                                         : run_bwd<bf16_t, float>(p, n_chunks, stream);
    return p.dout_dt == ATTNRES_BF16 ? run_bwd<float, bf16_t>(p, n_chunks, stream)
                                     : run_bwd<float, float>(p, n_chunks, stream);
}

}  // namespace attnres
