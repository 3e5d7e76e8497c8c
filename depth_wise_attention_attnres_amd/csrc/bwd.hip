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
//   bwd_dhist   fp32 history gradients (and calls the matrix-core kernel of
//               bwd_dhist_mfma.hip does not take): one wave per (token,
//               256-column slice of d): accumulates dv for row tiles in
//               registers while the reads' dout and w rows stream through a
//               prefetch ring (coefficients are uniform across the wave, so
//               they come through the scalar cache), then adds the
//               source-coupling terms with a forward (prefix) and a backward
//               (suffix) pass over each block, and stores dhist.  bf16
//               gradients go to bwd_dhist_mfma.hip, which forms the same sums
//               as one small matrix product per token.
//   bwd_dw_part one wave per (128-column slice, chunk of 32 tokens):
//               per-chunk partial dw for tiles of 32 reads on the matrix cores
//               (fp32 MFMA), the chunk's (token, row) pairs streamed through a
//               prefetch ring.
//   bwd_dw_sum  fixed-order sum of the partials in two stages, groups of
//               chunks then the groups (bitwise reproducible).
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

constexpr int kSlice = 256;  // columns of d per wave in bwd_dhist / bwd_dw_part (4 per lane)
constexpr int kDwSlice = 128;  // columns of d per wave in bwd_dw_part (32 lanes x 4 per pair)
constexpr int kChunkTokens = 32;

// four consecutive elements of a row
template <typename T> struct Quad;
template <> struct Quad<bf16_t> {
    typedef uint32_t raw_t __attribute__((ext_vector_type(2)));
    raw_t raw;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        raw = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
    __device__ __forceinline__ void load(const bf16_t* ptr) { raw = *reinterpret_cast<const raw_t*>(ptr); }
    __device__ __forceinline__ void to_float(float* f) const {
        f[0] = __uint_as_float(raw[0] << 16);
        f[1] = __uint_as_float(raw[0] & 0xffff0000u);
        f[2] = __uint_as_float(raw[1] << 16);
        f[3] = __uint_as_float(raw[1] & 0xffff0000u);
    }
    __device__ __forceinline__ static void store(rsrc_t r, uint32_t off, const float* f) {
        const raw_t u = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
        __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
    }
};
template <> struct Quad<float> {
    u32x4 raw;
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        raw = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
    __device__ __forceinline__ void load(const float* ptr) { raw = *reinterpret_cast<const u32x4*>(ptr); }
    __device__ __forceinline__ void to_float(float* f) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(raw[e]);
    }
    __device__ __forceinline__ static void store(rsrc_t r, uint32_t off, const float* f) {
        const u32x4 u = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                         __float_as_uint(f[3])};
        __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, 0);
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
    float* A2T = p.ws_a2t + t * (int64_t)p.n_hist * p.nq8;
    // the padding reads n_q .. nq8-1 of A2T are zero
    for (int k = ln; k < p.n_hist * (p.nq8 - p.n_q); k += 64) {
        const int i = k / (p.nq8 - p.n_q);
        A2T[(int64_t)i * p.nq8 + p.n_q + k % (p.nq8 - p.n_q)] = 0.f;
    }

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
                if (i < p.n_hist) A2T[(int64_t)i * p.nq8 + lq] = c2;
            }
        }
        __syncthreads();
    }
    for (int i = ln; i < p.n_blk; i += 64) p.ws_c3[t * p.n_blk + i] = c3acc[i];
}

// ---------------------------------------------------------------------------
// Matrix-core coefficients of Full reads (bf16 history and dout).  Per token
// the dots the backward needs are  P = W X^T  and  Q = G X^T  (reads x rows),
// contractions over d with d contiguous in memory -- the operand layout of
// v_mfma_f32_32x32x16_bf16, where lane j supplies 8 consecutive elements
// k = 8 (j / 32) .. + 7 of row j % 32 of both A and B.  bf16 x bf16 products
// are exact in fp32; the fp32 queries are split once per call into three bf16
// parts whose sum is w, so P keeps fp32 accuracy.  A Full read's sources are
// single rows, so the RMS scales need only |x_i|^2, which the waves form on
// the vector ALUs from the row fragments they already hold.  Then, per read,
// the softmax over its rows, delta, ds, and the coefficient rows written
// straight to the workspace.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void split_w_kernel(const float* w, int64_t n, uint16_t* hi,
                                                       uint16_t* mid, uint16_t* lo) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float x = w[i];
    const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;  // round to nearest even
    const float r1 = x - __uint_as_float(h << 16);      // exact
    const uint32_t m = pack_bf16x2(r1, 0.f) & 0xffffu;
    const float r2 = r1 - __uint_as_float(m << 16);     // exact
    const uint32_t l = pack_bf16x2(r2, 0.f) & 0xffffu;
    hi[i] = (uint16_t)h;
    mid[i] = (uint16_t)m;
    lo[i] = (uint16_t)l;
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* ptr, bool ok) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(ptr);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Eight waves per workgroup, TT tokens per workgroup (the three query parts
// are the same for every token, so two tokens share their slices).  Wave
// w < TT * npairs takes token w / npairs and the (w % npairs)-th (row tile b,
// read tile a) pair whose reads see rows of the tile: row tile b is rows
// 32 b .. 32 b + 31, read tile a reads 32 a .. ; the first pair of each row
// tile also forms the tile's |x_i|^2.  All waves load the operand slices and
// then take (token, read) jobs wave, wave + 8, ... for the softmax.  n_q <= 64
// (at most two read tiles), q_begin + n_q <= 128 (at most four row tiles).
constexpr int kScStage = 128;                 // K elements per stage
constexpr int kScChunks = kScStage / 8;       // 16-byte chunks per slice row and stage
constexpr int kScRowLds = kScStage + 8;       // bf16 per LDS slice row (padded)
constexpr int kScMaxPer = 12;                 // 16-byte chunks per thread and stage
constexpr int kScMaxSlices = kScMaxPer * 512 / (kScStage / 8);  // 384

// LDS floats before the slices (P, Q, |x|^2, per-wave C3), rounded up to 16 bytes
__host__ __device__ inline int sc_lds_floats(int tt, int n_q, int nr) {
    return (2 * tt * n_q * nr + tt * nr + 8 * tt * nr + 3) & ~3;
}

template <int TT>
__global__ __launch_bounds__(512) void bwd_scores_full_kernel(BwdParams p, int nb, int npairs) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, ln = tid & 63;
    const int h = ln >> 5, m = ln & 31;
    constexpr int nwaves = 8;
    const int64_t t0 = (int64_t)blockIdx.x * TT;
    const int ntok = p.T - t0 < TT ? (int)(p.T - t0) : TT;
    const int nr = p.q_begin + p.n_q;  // rows any read of the call sees
    const int na = (p.n_q + 31) / 32;  // read tiles
    const int64_t row_elems = p.T * (int64_t)p.d;

    extern __shared__ float lds[];
    float* P = lds;                          // [TT][n_q][nr] w_l . x_i
    float* Q = P + TT * p.n_q * nr;          // [TT][n_q][nr] g_l . x_i
    float* pn = Q + TT * p.n_q * nr;         // [TT][nr] |x_i|^2
    float* c3w = pn + TT * nr;               // [nwaves][TT][nr] C3 summed over each wave's reads
    for (int i = tid; i < nwaves * TT * nr; i += blockDim.x) c3w[i] = 0.f;

    // ---- dots on the matrix cores -------------------------------------------
    // this wave's pair: walk the row tiles, each with read tiles amin(b) .. na-1
    // (read l sees rows 0..l, so a read tile sees row tile b when its last
    // read reaches 32 b)
    const int u = wave / npairs;  // this wave's token in the workgroup
    int b = -1, a = 0, first_a = 0;
    if (u < ntok) {
        int k = wave - u * npairs;
        for (int bb = 0; bb < nb && b < 0; ++bb) {
            const int amin = 32 * bb - p.q_begin - 31 > 0 ? (32 * bb - p.q_begin) / 32 : 0;
            const int cnt = na - amin;
            if (k < cnt) {
                b = bb;
                a = amin + k;
                first_a = amin;
            } else {
                k -= cnt;
            }
        }
    }
    // K goes in stages of kScStage elements.  The stage's slices of each
    // token's rows (X) and upstream gradients (G), and of the three query
    // parts (W) -- TT (nr + n_q) + 3 n_q slices of kScStage bf16 each -- are
    // brought into LDS with coalesced 16-byte loads (sixteen lanes per
    // 256-byte slice), staged in registers while the previous stage
    // multiplies, then every wave reads its matrix operands from LDS.  A load
    // instruction spans two history rows (each row in its own page; a load
    // spanning many pages stalls the address unit).  (Loaded straight from
    // memory, each operand load touched 32 rows' cache lines for 32 bytes.)
    const int per_tok = nr + p.n_q;
    const int n_sl = TT * per_tok + 3 * p.n_q;
    bf16_t* sl = reinterpret_cast<bf16_t*>(lds + sc_lds_floats(TT, p.n_q, nr));  // [n_sl][kScRowLds]
    const int64_t wsz = (int64_t)p.n_q * p.d;
    // Loads walk the token slices interleaved (load slice rr * TT + tu is
    // row rr of token tu), so one load instruction spans two rows; LDS keeps
    // them token-major (slice tu * per_tok + rr), where the operand reads are
    // free of bank conflicts.
    auto lds_slice = [&](int r) {  // LDS slice of load slice r
        if (r >= TT * per_tok) return r;
        const int rr = r / TT;
        return (r - rr * TT) * per_tok + rr;
    };
    auto slice_src = [&](int r) -> const bf16_t* {  // start of load slice r's row, or null (zeros)
        if (r < TT * per_tok) {
            const int rr = r / TT, tu = r - rr * TT;
            if (tu >= ntok) return nullptr;
            const int64_t t = t0 + tu;
            if (rr < nr) return static_cast<const bf16_t*>(p.hist) + rr * row_elems + t * p.d;
            return static_cast<const bf16_t*>(p.dout) + (rr - nr) * row_elems + t * p.d;
        }
        r -= TT * per_tok;
        return reinterpret_cast<const bf16_t*>(p.ws_wsplit) + (int64_t)(r / p.n_q) * wsz +
               (int64_t)(r % p.n_q) * p.d;
    };
    const int n_chunks = n_sl * kScChunks;  // 16-byte chunks per stage (<= kScMaxPer * 512)
    u32x4 stg[kScMaxPer];
    auto gload = [&](int k0) {
#pragma unroll
        for (int c = 0; c < kScMaxPer; ++c) {
            u32x4 v = {0u, 0u, 0u, 0u};
            const int idx = tid + 512 * c;
            if (idx < n_chunks) {
                const int r = idx / kScChunks, k = k0 + 8 * (idx % kScChunks);
                const bf16_t* src = slice_src(r);
                if (src != nullptr && k < p.d) v = *reinterpret_cast<const u32x4*>(src + k);
            }
            stg[c] = v;
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int c = 0; c < kScMaxPer; ++c) {
            const int idx = tid + 512 * c;
            if (idx < n_chunks)
                *reinterpret_cast<u32x4*>(sl + lds_slice(idx / kScChunks) * kScRowLds + 8 * (idx % kScChunks)) =
                    stg[c];
        }
    };
    auto frag = [&](int r, int k) {  // 8 bf16 of LDS slice r at element k
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(sl + r * kScRowLds + k));
    };

    const bool norms = b >= 0 && a == first_a;
    const int row = 32 * (b < 0 ? 0 : b) + m;
    const bool row_ok = b >= 0 && row < nr;
    const int lq_w = 32 * a + m;
    const bool rd_ok = b >= 0 && lq_w < p.n_q;
    const int uu = u < TT ? u : 0;
    const int xs = uu * per_tok + (row_ok ? row : 0);             // X slice of this lane's row
    const int gs = uu * per_tok + nr + (rd_ok ? lq_w : 0);        // G slice of this lane's read
    const int ws0 = TT * per_tok + (rd_ok ? lq_w : 0);            // W0 slice; W1, W2 follow by n_q
    // The matrix accumulators are folded into fp32 totals every kFold
    // K-steps, so no sum runs longer than d / (16 kFold) + kFold terms (the
    // scores feed exponentials, whose relative error is the absolute error
    // of the score).
    constexpr int kFold = 16;
    f32x16 accP, accQ, totP, totQ;
#pragma unroll
    for (int r = 0; r < 16; ++r) accP[r] = accQ[r] = totP[r] = totQ[r] = 0.f;
    float sq = 0.f;  // this lane's part of |x_row|^2
    const int n_stages = (p.d + kScStage - 1) / kScStage;
    gload(0);
    lstore();
    __syncthreads();
    int st = 0;  // K-steps of 16 done
    for (int sg = 0; sg < n_stages; ++sg) {
        if (sg + 1 < n_stages) gload((sg + 1) * kScStage);
        if (b >= 0) {
#pragma unroll
            for (int sub = 0; sub < kScStage / 16; ++sub) {
                const int k = 16 * sub + 8 * h;
                if (16 * (sg * (kScStage / 16) + sub) >= p.d) break;
                const bf16x8_t x = frag(xs, k);
                const bf16x8_t g = frag(gs, k);
                const bf16x8_t w0 = frag(ws0, k);
                const bf16x8_t w1 = frag(ws0 + p.n_q, k);
                const bf16x8_t w2 = frag(ws0 + 2 * p.n_q, k);
                if (norms) {
                    const u32x4 xv = __builtin_bit_cast(u32x4, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = __uint_as_float(xv[e] << 16);
                        const float hi = __uint_as_float(xv[e] & 0xffff0000u);
                        sq = fmaf(lo, lo, sq);
                        sq = fmaf(hi, hi, sq);
                    }
                }
                accP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2, x, accP, 0, 0, 0);
                accP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w1, x, accP, 0, 0, 0);
                accP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w0, x, accP, 0, 0, 0);
                accQ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g, x, accQ, 0, 0, 0);
                ++st;
                if (st % kFold == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        totP[r] += accP[r];
                        totQ[r] += accQ[r];
                        accP[r] = accQ[r] = 0.f;
                    }
                }
            }
        }
        if (sg + 1 < n_stages) {
            __syncthreads();  // every wave is done with this stage's slices
            lstore();
            __syncthreads();
        }
    }
    if (b >= 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            totP[r] += accP[r];
            totQ[r] += accQ[r];
        }
        if (norms) {  // lanes m and m + 32 hold the two halves of each step's k
            sq = swap32_sum(sq);
            if (h == 0 && row_ok) pn[u * nr + row] = sq;
        }
        // lane j, register r holds D[i][n = m], i = 8 (r / 4) + 4 h + r % 4
        float* Pu = P + u * p.n_q * nr;
        float* Qu = Q + u * p.n_q * nr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * h + r % 4;
            const int lqo = 32 * a + i;
            if (row_ok && lqo < p.n_q) {
                Pu[lqo * nr + row] = totP[r];
                Qu[lqo * nr + row] = totQ[r];
            }
        }
    }
    __syncthreads();

    // ---- per (token, read): softmax over the read's rows, ds, coefficients --
    for (int job = wave; job < ntok * p.n_q; job += nwaves) {
        const int tu = job / p.n_q, lq = job - tu * p.n_q;
        const int64_t t = t0 + tu;
        float* A1 = p.ws_a1 + t * (int64_t)p.n_q * p.nh8;
        float* A2 = p.ws_a2 + t * (int64_t)p.n_q * p.nh8;
        float* A2T = p.ws_a2t + t * (int64_t)p.n_hist * p.nq8;
        const float* pnu = pn + tu * nr;
        float* c3s = c3w + (wave * TT + tu) * nr;
        const int l = p.q_begin + lq;
        const int ns = l + 1;  // rows 0..l, one source each
        const float* Pl = P + (tu * p.n_q + lq) * nr;
        const float* Ql = Q + (tu * p.n_q + lq) * nr;
        // lanes hold rows ln, ln + 64, ...; later rows (more than 64) are
        // recomputed in each pass
        float mx = -INFINITY;
        for (int i = ln; i < ns; i += 64)
            mx = fmaxf(mx, fast_rsqrt(fmaf(pnu[i], p.inv_d, p.eps)) * Pl[i]);
        mx = tg_max<64>(mx);
        float z = 0.f, zd = 0.f;  // sum of e and of e * a
        for (int i = ln; i < ns; i += 64) {
            const float e = fast_exp2((fast_rsqrt(fmaf(pnu[i], p.inv_d, p.eps)) * Pl[i] - mx) * kLog2e);
            z += e;
            zd = fmaf(e, Ql[i], zd);
        }
        z = tg_sum<64>(z);
        zd = tg_sum<64>(zd);
        const float inv_z = 1.0f / z;
        const float delta = zd * inv_z;
        for (int i = ln; i < p.nh8; i += 64) {  // row-major A1 / A2: contiguous in i
            float c1 = 0.f, c2 = 0.f;
            if (i < ns) {
                const float r = fast_rsqrt(fmaf(pnu[i], p.inv_d, p.eps));
                const float s2 = r * Pl[i];
                const float alpha = fast_exp2((s2 - mx) * kLog2e) * inv_z;
                const float ds = alpha * (Ql[i] - delta);
                c1 = alpha;
                c2 = ds * r;
                c3s[i] += ds * r * r * s2 * p.inv_d;  // same lane for a row on every job of this wave
            }
            A1[(int64_t)lq * p.nh8 + i] = c1;
            A2[(int64_t)lq * p.nh8 + i] = c2;
            if (i < p.n_hist) A2T[(int64_t)i * p.nq8 + lq] = c2;
        }
        if (ln == 0) p.ws_kappa[t * p.n_q + lq] = 0.f;  // Full: no partial sums
    }
    // the padding reads n_q .. nq8 - 1 of A2T are zero
    const int npad = p.nq8 - p.n_q;
    for (int k = tid; k < ntok * p.n_hist * npad; k += blockDim.x) {
        const int tu = k / (p.n_hist * npad), rem = k - tu * p.n_hist * npad;
        const int i = rem / npad;
        p.ws_a2t[(t0 + tu) * (int64_t)p.n_hist * p.nq8 + (int64_t)i * p.nq8 + p.n_q + rem % npad] = 0.f;
    }
    __syncthreads();
    // C3 summed over the waves in a fixed order; rows no read sees get 0
    for (int k = tid; k < ntok * p.n_blk; k += blockDim.x) {
        const int tu = k / p.n_blk, i = k - tu * p.n_blk;
        float c3 = 0.f;
        if (i < nr)
            for (int w = 0; w < nwaves; ++w) c3 += c3w[(w * TT + tu) * nr + i];
        p.ws_c3[(t0 + tu) * p.n_blk + i] = c3;
    }
}

// ---------------------------------------------------------------------------
// bwd_dhist: one wave per (token, 256-column slice); lane owns 4 columns.
// Rows are handled in tiles of RT accumulated in registers; the reads' dout
// and w rows stream through a ring of PF prefetched loads.

template <typename TI, typename TG, typename TO, int RT, int PF>
__global__ __launch_bounds__(64) void bwd_dhist_kernel(BwdParams p) {
    const int ln = threadIdx.x;
    // slices of one token are neighbours in dispatch order, so the token's
    // coefficients are fetched from HBM once and then served by L2
    // the slices of one token share an XCD (and its L2): the token's
    // coefficients are fetched from HBM once, then served by that L2
    const int slices = (p.d + kSlice - 1) / kSlice;
    int64_t t;
    int slice;
    xcd_group(blockIdx.x, slices, t, slice);
    if (t >= p.T) return;  // whole workgroups of one wave
    const int e0 = slice * kSlice + 4 * ln;  // this lane's four columns
    const bool valid = e0 < p.d;                   // d % 8 == 0: all four or none
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

    const cf32_ptr A1 = const_view(p.ws_a1 + t * (int64_t)p.n_q * p.nh8);
    const cf32_ptr A2 = const_view(p.ws_a2 + t * (int64_t)p.n_q * p.nh8);
    const cf32_ptr C3 = const_view(p.ws_c3 + t * p.n_blk);
    const cf32_ptr kap = const_view(p.ws_kappa + t * p.n_q);

    auto load_row = [&](int i, float* v) {
        const rsrc_t rr = make_rsrc(hist_tok + i * row_elems, (uint64_t)p.d * sizeof(TI));
        Quad<TI> q;
        q.load(rr, h_off);
        q.to_float(v);
    };
    // kappa of read l (0 for reads outside the call)
    auto kappa = [&](int l) { return (l >= p.q_begin && l < q_end) ? kap[l - p.q_begin] : 0.f; };

    __shared__ float coef_t[RT];
    for (int rt0 = 0; rt0 < p.n_hist; rt0 += RT) {
        float dv[RT][4];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) dv[i][e] = 0.f;

        // value path and query path: sum over the reads that see a row of the tile
        const int lq0 = rt0 > p.q_begin ? rt0 - p.q_begin : 0;
        const int n_l = p.n_q - lq0;
        Quad<TG> gq[PF];
        Quad<float> wq[PF];
        auto issue = [&](int u, int lq) {
            const rsrc_t gr = make_rsrc(dout_tok + (int64_t)lq * row_elems, (uint64_t)p.d * sizeof(TG));
            gq[u].load(gr, g_off);
            const rsrc_t wr = make_rsrc(p.w + (int64_t)lq * p.d, (uint64_t)p.d * 4);
            wq[u].load(wr, w_off);
        };
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (u < n_l) issue(u, lq0 + u);
        for (int j0 = 0; j0 < n_l; j0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int j = j0 + u;
                if (j >= n_l) break;
                const int lq = lq0 + j;
                const int l = p.q_begin + lq;
                float g[4], w[4];
                gq[u].to_float(g);
                wq[u].to_float(w);
                if (j + PF < n_l) issue(u, lq + PF);
                const cf32_ptr a1 = A1 + (int64_t)lq * p.nh8 + rt0;
                const cf32_ptr a2 = A2 + (int64_t)lq * p.nh8 + rt0;
#pragma unroll
                for (int q8 = 0; q8 < RT / 8; ++q8) {
                    if (rt0 + 8 * q8 <= l) {  // rows past l have zero coefficients
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int i = 8 * q8 + q;
                            const float c1 = a1[i], c2 = a2[i];
#pragma unroll
                            for (int e = 0; e < 4; ++e) dv[i][e] = fmaf(c1, g[e], fmaf(c2, w[e], dv[i][e]));
                        }
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
        const int rt1 = rt0 + RT < p.n_hist ? rt0 + RT : p.n_hist;  // tile end
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
        for (int k = ln; k < RT; k += 64)
            if (rt0 + k < rt1) coef_t[k] = coef_of(rt0 + k);
        __syncthreads();

        // the tile's rows, eight at a time (rows past the tile read zeros)
        auto load_group = [&](int g0, Quad<TI>* xr) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = rt0 + g0 + q;
                const int jr = j < rt1 ? j : rt1 - 1;
                const rsrc_t rr = make_rsrc(hist_tok + jr * row_elems, (uint64_t)p.d * sizeof(TI));
                xr[q].load(rr, j < rt1 ? h_off : kOOB);
            }
        };

        // forward pass: prefix sums within blocks
        float pf[4] = {0.f, 0.f, 0.f, 0.f};
        {
            const int c = block_of(rt0);
            for (int m = block_first(c); m < rt0; ++m) {  // rows of the block in earlier tiles
                float u[4];
                load_row(m, u);
#pragma unroll
                for (int e = 0; e < 4; ++e) pf[e] += u[e];
            }
        }
#pragma unroll
        for (int g0 = 0; g0 < RT; g0 += 8) {
            if (rt0 + g0 < rt1) {
                Quad<TI> xr[8];
                load_group(g0, xr);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int ii = g0 + q;
                    const int j = rt0 + ii;
                    if (j < rt1) {
                        if (ii > 0 && j == block_first(block_of(j)))
#pragma unroll
                            for (int e = 0; e < 4; ++e) pf[e] = 0.f;
                        float v[4];
                        xr[q].to_float(v);
                        const float k = coef_t[ii];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pf[e] += v[e];
                            dv[ii][e] = fmaf(-k, pf[e], dv[ii][e]);
                        }
                    }
                }
            }
        }
        // backward pass: suffix sums within blocks
        float bs[4] = {0.f, 0.f, 0.f, 0.f};
        {
            const int c = block_of(rt1 - 1);
            for (int m = block_last(c); m >= rt1; --m) {  // rows of the block in later tiles
                float u[4];
                load_row(m, u);
                const float k = coef_of(m);
#pragma unroll
                for (int e = 0; e < 4; ++e) bs[e] = fmaf(k, u[e], bs[e]);
            }
        }
#pragma unroll
        for (int g0 = RT - 8; g0 >= 0; g0 -= 8) {
            if (rt0 + g0 < rt1) {
                Quad<TI> xr[8];
                load_group(g0, xr);
#pragma unroll
                for (int q = 7; q >= 0; --q) {
                    const int ii = g0 + q;
                    const int j = rt0 + ii;
                    if (j < rt1) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) dv[ii][e] -= bs[e];
                        if (j == block_first(block_of(j))) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) bs[e] = 0.f;
                        } else {
                            float v[4];
                            xr[q].to_float(v);
                            const float k = coef_t[ii];
#pragma unroll
                            for (int e = 0; e < 4; ++e) bs[e] = fmaf(k, v[e], bs[e]);
                        }
                    }
                }
            }
        }
        __syncthreads();  // coef_t is rewritten by the next tile

#pragma unroll
        for (int ii = 0; ii < RT; ++ii) {
            const int j = rt0 + ii;
            if (j < rt1) {
                const rsrc_t orr = make_rsrc(dh_tok + j * row_elems, (uint64_t)p.d * sizeof(TO));
                if (p.accumulate) {  // uniform branch; the host allows it for fp32 dhist only
                    Quad<TO> old;
                    old.load(orr, o_off);
                    float f[4];
                    old.to_float(f);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dv[ii][e] += f[e];
                }
                Quad<TO>::store(orr, o_off, dv[ii]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_dw_part: per chunk of tokens, the partial  dw[l][k] = sum over the
// chunk's (token, row) pairs of A2T[pair][l] x[pair][k]  -- a dense
// contraction over pairs, done on the matrix cores in fp32
// (v_mfma_f32_32x32x2f32: D[32x32] += A[32x2] B[2x32]).
// One wave per (128-column slice, chunk); it accumulates a tile of 32 reads.
// A step takes one history row i and two neighbouring tokens 2u, 2u + 1 of
// the chunk; lane j (half h = j / 32, m = j % 32) supplies
//   A[i' = m][k = h] = x[i][token 2u + h][column c0 + 4m + e]  (MFMA e = 0..3)
//   B[k = h][n = m]  = A2T[token 2u + h][i][read qt0 + m]
// so a half-wave reads 128 contiguous columns of one row and 32 contiguous
// coefficients, and the two halves differ by one token: the buffer
// descriptors stay wave-uniform and every lane offset is fixed.  Lane j,
// accumulator register r then holds D[i'][n = m] with
// i' = 8 (r / 4) + 4 h + r % 4: the partial of read qt0 + m at columns
// c0 + 4 i' + e.

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename TI, int PF>
__global__ __launch_bounds__(64) void bwd_dw_part_kernel(BwdParams p) {
    constexpr int QT = 32;
    const int ln = threadIdx.x;
    const int h = ln >> 5, m = ln & 31;
    // the column slices of one chunk share an XCD, so the chunk's coefficients
    // come from HBM once and are then served by that L2
    const int slices = (p.d + kDwSlice - 1) / kDwSlice;
    int64_t chunk64;
    int slice;
    xcd_group(blockIdx.x, slices, chunk64, slice);
    const int n_chunks_all = (int)((p.T + kChunkTokens - 1) / kChunkTokens);
    if (chunk64 >= n_chunks_all) return;  // whole workgroups of one wave
    const int chunk = (int)chunk64;
    const int c0 = slice * kDwSlice;
    const bool valid = c0 + 4 * m < p.d;  // d % 8 == 0: all four columns or none
    const int64_t row_elems = p.T * (int64_t)p.d;
    const int64_t t_lo = (int64_t)chunk * kChunkTokens;
    const int n_tok = (int)(p.T - t_lo < kChunkTokens ? p.T - t_lo : kChunkTokens);
    const int n_pairs = (n_tok + 1) / 2;  // token pairs of the chunk
    const TI* hist_chunk = static_cast<const TI*>(p.hist) + t_lo * p.d;
    const float* a2t_chunk = p.ws_a2t + t_lo * (int64_t)p.n_hist * p.nq8;
    const int64_t a2t_tok = (int64_t)p.n_hist * p.nq8;  // floats per token of A2T
    // fixed lane offsets inside a step's two-token window
    const uint32_t x_off = (uint32_t)((h * p.d + c0 + 4 * m) * sizeof(TI));

    // The chunk's (token pair, row) steps go in one pass for two tiles of 32
    // reads at once (tile 0 stops at the last row its reads see), so the rows
    // are read once per 64 reads.  One buffer descriptor spans the chunk's 32
    // tokens of a row and one the chunk's coefficients; a step only moves the
    // lane offsets.
    const rsrc_t rc = make_rsrc(a2t_chunk, (uint64_t)n_tok * a2t_tok * 4);
    for (int qt0 = 0; qt0 < p.n_q; qt0 += 2 * QT) {
        const int nq0 = p.n_q - qt0 < QT ? p.n_q - qt0 : QT;      // reads of tile 0
        const int nq1 = p.n_q - qt0 - QT < QT ? p.n_q - qt0 - QT : QT;  // of tile 1 (may be <= 0)
        const int n_rows0 = p.q_begin + qt0 + nq0;                // rows tile 0 sees
        const int n_rows = nq1 > 0 ? n_rows0 + nq1 : n_rows0;    // rows either tile sees
        const int n_steps = n_rows * n_pairs;
        // coefficients of reads qt0 + m and qt0 + 32 + m (zero in A2T past n_q;
        // columns past nq8 would belong to the next row)
        const bool ok0 = qt0 + m < p.nq8, ok1 = nq1 > 0 && qt0 + QT + m < p.nq8;
        f32x16 acc0[4], acc1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc0[e][r] = acc1[e][r] = 0.f;

        Quad<TI> xr[PF];
        float cr0[PF], cr1[PF];
        int ir = 0, iu = 0;  // (row, token pair) of the next step to issue
        rsrc_t rx = make_rsrc(hist_chunk, (uint64_t)n_tok * p.d * sizeof(TI));
        auto issue = [&](int u) {
            const int tk = 2 * iu + h;  // this lane's token in the chunk
            const bool live = tk < n_tok;
            xr[u].load(rx, live && valid ? x_off + (uint32_t)(2 * iu * p.d * sizeof(TI)) : kOOB);
            const uint32_t cb = (uint32_t)(((int64_t)tk * a2t_tok + (int64_t)ir * p.nq8 + qt0 + m) * 4);
            cr0[u] = load_f32(rc, live && ok0 ? cb : kOOB);
            cr1[u] = load_f32(rc, live && ok1 ? cb + 4 * QT : kOOB);
            if (++iu == n_pairs) {
                iu = 0;
                ++ir;
                rx = make_rsrc(hist_chunk + (int64_t)ir * row_elems, (uint64_t)n_tok * p.d * sizeof(TI));
            }
        };
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (u < n_steps) issue(u);
        for (int s0 = 0; s0 < n_steps; s0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int st = s0 + u;
                if (st >= n_steps) break;
                float v[4];
                xr[u].to_float(v);
                const float c0v = cr0[u], c1v = cr1[u];
                if (st + PF < n_steps) issue(u);
                if (st < n_rows0 * n_pairs) {  // wave-uniform: rows tile 0 sees
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc0[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[e], c0v, acc0[e], 0, 0, 0);
                }
                if (nq1 > 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc1[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[e], c1v, acc1[e], 0, 0, 0);
                }
            }
        }
        auto store_tile = [&](const f32x16 (&acc)[4], int q0, int nq) {
            if (m < nq) {
                float* part = p.ws_dwpart + ((int64_t)chunk * p.n_q + q0 + m) * p.d;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 8 * (r / 4) + 4 * h + r % 4;
                    const int col = c0 + 4 * i;
                    if (col < p.d) *reinterpret_cast<f32x4*>(part + col) = {acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
                }
            }
        };
        store_tile(acc0, qt0, nq0);
        if (nq1 > 0) store_tile(acc1, qt0 + QT, nq1);
    }
}

// dw = sum of the per-chunk partials, in two fixed-order stages (bitwise
// reproducible): groups of consecutive chunks in parallel, then the groups.
__global__ __launch_bounds__(256) void bwd_dw_sum_kernel(BwdParams p, int n_chunks, int groups) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.n_q * p.d;
    if (idx >= total) return;
    const int per = (n_chunks + groups - 1) / groups;
    const int c0 = blockIdx.y * per;
    const int c1 = c0 + per < n_chunks ? c0 + per : n_chunks;
    float s = 0.f;
    for (int c = c0; c < c1; ++c) s += p.ws_dwpart[(int64_t)c * total + idx];
    p.ws_dwstage[(int64_t)blockIdx.y * total + idx] = s;
}

__global__ __launch_bounds__(256) void bwd_dw_final_kernel(BwdParams p, int groups) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.n_q * p.d;
    if (idx >= total) return;
    float s = 0.f;
    for (int g = 0; g < groups; ++g) s += p.ws_dwstage[(int64_t)g * total + idx];
    p.dw[idx] = p.accumulate ? p.dw[idx] + s : s;
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
    L.nq8 = up(n_q, 8);
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
    L.off_a2t = take(T * n_hist * L.nq8);
    L.off_c3 = take(T * L.n_blk);
    L.off_kappa = take(T * n_q);
    L.off_dwpart = take(L.n_chunks * n_q * d);
    L.off_wsplit = take((3 * n_q * d + 1) / 2);  // bf16
    L.n_dw_groups = L.n_chunks < 16 ? L.n_chunks : 16;
    L.off_dwstage = take(L.n_dw_groups * n_q * d);
    L.off_wsplit2 = take((bwd_wsplit2_elems(n_q, d) + 1) / 2);  // bf16
    L.bytes = off;
    return L;
}

namespace {


// Row tiles of the matrix-core coefficients (Full reads, bf16 history and
// upstream gradient, at most 64 reads and 128 rows): the number of 32-row
// tiles, or 0 when another kernel forms the coefficients.  Block keeps the
// other kernels: its sources are fewer than its rows, and the 32-row operand
// loads cost more there than the dots they feed (measured at 49 rows,
// d = 1024, S = 4: 3.6 against 2.5 ms).
int scores_mfma_tiles(const BwdParams& p) {
    if (p.hist_dt != ATTNRES_BF16 || p.dout_dt != ATTNRES_BF16) return 0;
    if (p.S != 1 || p.n_q > 64) return 0;
    const int nr = p.q_begin + p.n_q;
    const int nb = (nr + 31) / 32;
    return nb <= 4 ? nb : 0;
}

// streaming kernel: template arguments by chunks per lane
constexpr int kStreamPF[9] = {0, 4, 2, 2, 2, 1, 1, 1, 1};
constexpr int kStreamR[9] = {0, 4, 4, 2, 2, 1, 1, 1, 1};

// Which kernel forms the per-read coefficients of a call, and its dynamic LDS.
struct ScoresPlan {
    enum Kind { NONE, MFMA, GROUP, STREAM } kind;
    int nb, nwaves, tt;   // MFMA: row tiles, (row, read) tile pairs, tokens per workgroup
    size_t lds;           // MFMA, STREAM
};

ScoresPlan plan_scores(const BwdParams& p) {
    ScoresPlan s{ScoresPlan::NONE, 0, 0, 0, 0};
    const int max_lds = device_max_lds();
    const int nb = scores_mfma_tiles(p);
    if (nb > 0) {
        const int nr = p.q_begin + p.n_q;
        // one wave per (row tile, read tile) pair whose reads see the tile
        const int na = (p.n_q + 31) / 32;
        int npairs = 0;
        for (int b = 0; b < nb; ++b) {
            const int amin = 32 * b - p.q_begin - 31 > 0 ? (32 * b - p.q_begin) / 32 : 0;
            npairs += na - amin;
        }
        auto lds_for = [&](int tt) {
            return sizeof(float) * (size_t)sc_lds_floats(tt, p.n_q, nr) +
                   2 * (size_t)(tt * (nr + p.n_q) + 3 * p.n_q) * kScRowLds;
        };
        // two tokens per workgroup when their pairs fit the eight waves and
        // their slices the staging registers
        int tt = 2 * npairs <= 8 && 2 * (nr + p.n_q) + 3 * p.n_q <= kScMaxSlices && p.T >= 2 &&
                         lds_for(2) <= (size_t)max_lds ? 2 : 1;
        if (tt == 1 && (nr + 4 * p.n_q > kScMaxSlices || lds_for(1) > (size_t)max_lds)) tt = 0;
        if (tt > 0) {  // else one of the kernels below
            s.kind = ScoresPlan::MFMA;
            s.nb = nb;
            s.nwaves = npairs;
            s.tt = tt;
            s.lds = lds_for(tt);
            return s;
        }
    }
    if (bwd_scores_group_applies(p)) {
        s.kind = ScoresPlan::GROUP;
        return s;
    }
    const int nch = (p.nc + 63) / 64;
    if (nch < 1 || nch > 8) return s;
    const size_t lds = sizeof(float) * (6 * (size_t)kStreamR[nch] * p.nx + p.n_blk);
    if (lds > (size_t)max_lds) return s;  // too many sources for one token's LDS
    s.kind = ScoresPlan::STREAM;
    s.lds = lds;
    return s;
}

template <typename TI, typename TG>
hipError_t launch_scores(const BwdParams& p, const ScoresPlan& s, hipStream_t stream) {
    if (s.kind == ScoresPlan::MFMA) {
        const int64_t nw = (int64_t)p.n_q * p.d;
        uint16_t* hi = p.ws_wsplit;
        hipLaunchKernelGGL(split_w_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream,
                           p.w, nw, hi, hi + nw, hi + 2 * nw);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        auto go = [&](auto kern, int tt) {
            hipError_t e2 = prepare_dynamic_lds((const void*)kern, s.lds);
            if (e2 != hipSuccess) return e2;
            hipLaunchKernelGGL(kern, dim3((unsigned)((p.T + tt - 1) / tt)), dim3(512), s.lds, stream,
                               p, s.nb, s.nwaves);
            return hipGetLastError();
        };
        return s.tt == 2 ? go(bwd_scores_full_kernel<2>, 2) : go(bwd_scores_full_kernel<1>, 1);
    }
    if (s.kind == ScoresPlan::GROUP) return launch_bwd_scores_group(p, stream);
    if (s.kind != ScoresPlan::STREAM) return hipErrorInvalidValue;
    const int nch = (p.nc + 63) / 64;
    auto go = [&](auto kern) {
        const hipError_t e = prepare_dynamic_lds((const void*)kern, s.lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)p.T), dim3(64), s.lds, stream, p);
        return hipGetLastError();
    };
    switch (nch) {
#define ATTNRES_SCORES(N)                                                                   \
    case N:                                                                                 \
        return go(bwd_scores_kernel<TI, TG, N, kStreamPF[N], kStreamR[N]>);
        ATTNRES_SCORES(1)
        ATTNRES_SCORES(2)
        ATTNRES_SCORES(3)
        ATTNRES_SCORES(4)
        ATTNRES_SCORES(5)
        ATTNRES_SCORES(6)
        ATTNRES_SCORES(7)
        ATTNRES_SCORES(8)
#undef ATTNRES_SCORES
        default: return hipErrorInvalidValue;
    }
}

template <typename TI, typename TG, typename TO>
hipError_t launch_rest(const BwdParams& p, int n_chunks, int groups, hipStream_t stream) {
    // XCD-aware numbering (xcd_group): 8 slices ceil(T / 8) workgroups
    const unsigned slices = (unsigned)((p.d + kSlice - 1) / kSlice);
    const unsigned dh_blocks = (unsigned)((p.T + kNumXcd - 1) / kNumXcd) * kNumXcd * slices;
    hipError_t e = hipSuccess;
    if (std::is_same<TO, bf16_t>::value && bwd_dhist_mfma_applies(p))  // bf16 gradients
        e = launch_bwd_dhist_mfma(p, stream);
    else if (p.n_hist <= 8)
        hipLaunchKernelGGL((bwd_dhist_kernel<TI, TG, TO, 8, 4>), dim3(dh_blocks), dim3(64),
                           0, stream, p);
    else  // 16-row tiles: 125 VGPRs, four waves per SIMD (32-row tiles: 192, two
          // waves, 1 ms slower at 49 rows / d = 1024 although they stream fewer reads)
        hipLaunchKernelGGL((bwd_dhist_kernel<TI, TG, TO, 16, 4>), dim3(dh_blocks),
                           dim3(64), 0, stream, p);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bwd_dw_mfma_applies(p)) {  // bf16 history, at most 64 reads
        e = launch_bwd_dw_mfma(p, kChunkTokens, stream);
    } else {
        const unsigned dw_slices = (unsigned)((p.d + kDwSlice - 1) / kDwSlice);
        const unsigned dw_blocks = (unsigned)((n_chunks + kNumXcd - 1) / kNumXcd) * kNumXcd * dw_slices;
        hipLaunchKernelGGL((bwd_dw_part_kernel<TI, 8>), dim3(dw_blocks), dim3(64), 0,
                           stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)p.n_q * p.d;
    hipLaunchKernelGGL(bwd_dw_sum_kernel, dim3((unsigned)((total + 255) / 256), (unsigned)groups),
                       dim3(256), 0, stream, p, n_chunks, groups);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dw_final_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, p, groups);
    return hipGetLastError();
}

template <typename TI, typename TG>
hipError_t dispatch_out(const BwdParams& p, int n_chunks, int groups, hipStream_t stream) {
    return p.dhist_dt == ATTNRES_BF16 ? launch_rest<TI, TG, bf16_t>(p, n_chunks, groups, stream)
                                      : launch_rest<TI, TG, float>(p, n_chunks, groups, stream);
}

template <typename TI, typename TG>
hipError_t run_bwd(const BwdParams& p, int n_chunks, int groups, hipStream_t stream) {
    const ScoresPlan s = plan_scores(p);
    hipError_t e = launch_scores<TI, TG>(p, s, stream);
    if (e != hipSuccess) return e;
    return dispatch_out<TI, TG>(p, n_chunks, groups, stream);
}

}  // namespace

bool bwd_fits(const BwdParams& p) {
    // bwd_dw_part addresses a chunk's coefficients (32 tokens of A2T) from one
    // buffer descriptor, whose range is kOOB bytes
    if ((int64_t)kChunkTokens * p.n_hist * p.nq8 * 4 >= (int64_t)kOOB) return false;
    return plan_scores(p).kind != ScoresPlan::NONE;
}

hipError_t launch_bwd(const BwdParams& p, int n_chunks, int groups, hipStream_t stream) {
    if (p.hist_dt == ATTNRES_BF16)
        return p.dout_dt == ATTNRES_BF16 ? run_bwd<bf16_t, bf16_t>(p, n_chunks, groups, stream)
                                         : run_bwd<bf16_t, float>(p, n_chunks, groups, stream);
    return p.dout_dt == ATTNRES_BF16 ? run_bwd<float, bf16_t>(p, n_chunks, groups, stream)
                                     : run_bwd<float, float>(p, n_chunks, groups, stream);
}

}  // namespace attnres
