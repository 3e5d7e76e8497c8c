// full_batch_mfma.hip -- Full AttnRes forward for calls with many reads over a
// bf16 history with bf16 outputs, on the matrix cores of gfx950.
//
// Read l of a token sees its rows 0..l ("DepthBench reading notes" sec. 2.3).
// As in full_batch.hip, one workgroup per token stages the token's rows in LDS
// once and serves every read of the call from there; here both contractions
// of the reads run on v_mfma_f32_16x16x32_bf16, D[16 x 16] += A[16 x 32] B[32 x 16]
// (lane L supplies 8 consecutive k = 8 (L / 16) .. + 7 of row L % 16 of A and
// of column L % 16 of B; it receives D[4 (L / 16) + r][L % 16], r = 0..3):
//   scores   P[j][i] = w_{l_j} . v_i, m = read j, n = row i, k along d.  The
//            queries are shared by every token; each lane splits its 8 fp32
//            query values into three bf16 parts hi + mid + lo (each rounded to
//            nearest; their sum is the fp32 value), the rows are bf16 already,
//            so the scores carry fp32 products.  Jobs of one read tile (16
//            reads) and up to three row tiles (16 rows each) share the split.
//   softmax  s = r_i P[j][i] log2(e) where the read sees the row (else -inf);
//            max and sum per read over the row tiles through two small LDS
//            tables (fixed order), then the weights alpha, split into two
//            bf16 parts and stored as the B operand of:
//   outputs  h_j[e] = sum_i alpha[j][i] v_i[e], m = column e, n = read j, k
//            over rows in steps of 32.  A column of rows comes from two
//            transposing LDS reads (ds_read_b64_tr_b16: within 16 lanes, lane c
//            receives element c mod 4 of the 8-byte chunks that lanes 4 e + c / 4,
//            e = 0..3, fetch), so lane 4 e + q fetches columns 4 q .. 4 q + 3 of
//            row 8 g + 2 e + s for read s = 0, 1 (g = lane group); within a step,
//            k = 8 g + 4 s + e stands for that row, which puts the four rows a
//            16-lane group reads 8 banks apart.  The weights are stored in the
//            same order.
// bf16 x bf16 products are exact in fp32.  The weights' two-part bf16 split
// keeps 16 significant bits (error below 2^-17 of the weight), far below the
// rounding of the bf16 output; the scores, which also give the fp32
// log-sum-exp, keep all 24.  Outputs leave as 4 consecutive bf16 per lane.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kBmWaves = 8;
constexpr int kBmMinReads = 16;
constexpr int kBmMaxTiles = 6;       // reads and rows: at most 96 each (tiles of 16)
constexpr int kBmJobTiles = 3;       // row tiles per score job
constexpr int kBmJobsPerWave = 2;    // score jobs a wave holds through the softmax
// Rows per wave a token's prefetch holds (kBmWaves times as many per token;
// calls with more rows go to the vector kernel): 96 rows with one chunk per
// lane, 80 with two (the registers of the prefetch come on top of the output
// contraction's), 48 with three and 40 with four (the LDS holds 47 rows at
// d = 1536 and 36 at d = 2048)
template <int NCH>
constexpr int bm_rows_in_flight() { return NCH == 1 ? 12 : (NCH == 2 ? 10 : (NCH == 3 ? 6 : 5)); }
constexpr int kBmWRing = 4;          // K-steps of query fragments in flight
constexpr int kBmMaxKs = (16 * kBmMaxTiles + 31) / 32;  // row steps of 32 in the output contraction

// LDS layout of one workgroup (byte offsets).  Rows [n_rows][dst] bf16 (dst =
// d + 8: rows 16 bytes apart in bank order, so both the 16-byte operand reads
// and the column gathers are free of bank conflicts); the weights' two bf16
// parts [2][n_q][ast] (ast = 32 nks + 8); the per-read maxima and sums per row
// tile [n_q][nrb]; the RMS scales [n_rows].
struct BmLayout {
    int dst, ast, nrb, nrt, nks;
    int64_t ap_off, pm_off, ps_off, rs_off, bytes;
};
__host__ __device__ inline BmLayout bm_layout(int n_rows, int n_q, int d) {
    BmLayout L;
    L.dst = d + 8;
    L.nrb = (n_rows + 15) / 16;
    L.nrt = (n_q + 15) / 16;
    L.nks = (n_rows + 31) / 32;
    L.ast = 32 * L.nks + 8;
    L.ap_off = (int64_t)n_rows * L.dst * 2;  // d % 32 == 0: a multiple of 16
    L.pm_off = L.ap_off + (int64_t)2 * n_q * L.ast * 2;
    L.ps_off = L.pm_off + (int64_t)n_q * L.nrb * 4;
    L.rs_off = L.ps_off + (int64_t)n_q * L.nrb * 4;
    L.bytes = L.rs_off + (int64_t)((n_rows + 3) & ~3) * 4;
    return L;
}

// A score job: read tile a (reads 16 a .. 16 a + 15), row tiles b0 .. b0 + nb - 1.
struct BmJob {
    int a, b0, nb;
};
// last read of read tile a, and how many row tiles its reads see
__host__ __device__ inline int bm_tile_rows(const FwdParams& p, int a) {
    const int jl = 16 * a + 15 < p.n_q - 1 ? 16 * a + 15 : p.n_q - 1;
    return (p.q_begin + jl) / 16 + 1;
}
// the k-th job: the row tiles of each read tile cut into near-equal groups of
// at most kBmJobTiles; false past the last job
__host__ __device__ inline bool bm_job(const FwdParams& p, int nrt, int k, BmJob& J) {
    int idx = 0;
    for (int a = 0; a < nrt; ++a) {
        const int nb_a = bm_tile_rows(p, a);
        const int ng = (nb_a + kBmJobTiles - 1) / kBmJobTiles;
        if (k < idx + ng) {
            const int q = k - idx;
            J.a = a;
            J.b0 = q * nb_a / ng;
            J.nb = (q + 1) * nb_a / ng - J.b0;
            return true;
        }
        idx += ng;
    }
    return false;
}
__host__ __device__ inline int bm_num_jobs(const FwdParams& p, int nrt) {
    int n = 0;
    for (int a = 0; a < nrt; ++a) n += (bm_tile_rows(p, a) + kBmJobTiles - 1) / kBmJobTiles;
    return n;
}

// three bf16 parts of 8 fp32 values, each rounded to nearest even; every
// remainder is exact in fp32, so hi + mid + lo is the value
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8_t& hi, bf16x8_t& mid, bf16x8_t& lo) {
    u32x4 h, m, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t hp = pack_bf16x2(x[2 * q], x[2 * q + 1]);
        const float a0 = x[2 * q] - __uint_as_float(hp << 16);
        const float a1 = x[2 * q + 1] - __uint_as_float(hp & 0xffff0000u);
        const uint32_t mp = pack_bf16x2(a0, a1);
        const float b0 = a0 - __uint_as_float(mp << 16);
        const float b1 = a1 - __uint_as_float(mp & 0xffff0000u);
        h[q] = hp;
        m[q] = mp;
        l[q] = pack_bf16x2(b0, b1);
    }
    hi = __builtin_bit_cast(bf16x8_t, h);
    mid = __builtin_bit_cast(bf16x8_t, m);
    lo = __builtin_bit_cast(bf16x8_t, l);
}

// k index, within a step of 32 rows, of row u (0..31) of the step: row
// 8 g + 2 e + s is k = 8 g + 4 s + e
__device__ __forceinline__ int bm_kidx(int u) { return 8 * (u >> 3) + 4 * (u & 1) + ((u & 7) >> 1); }

typedef short bm_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bm_v4s bm_lds_v4s;

// The dots of one score job with NB row tiles: acc[u] += W (16 reads x d) times
// row tile u (d x 16 rows), in K-steps of 32.  The query fragments of the next
// kBmWRing K-steps are in flight (L2 latency is several K-steps of matrix
// work): whole rounds of kBmWRing steps refill each slot once it is consumed
// (past d the refill loads zeros and is never used), then the last d / 32 mod
// kBmWRing steps consume what is left.  No row is read past d.
template <int NB>
__device__ __forceinline__ void bm_scores(rsrc_t wr, uint32_t woff, const bf16_t* rows,
                                          const int (&roff)[kBmJobTiles], int d, f32x4 (&acc)[kBmJobTiles]) {
    Chunk<float> wring[kBmWRing];
    auto wload = [&](Chunk<float>& dst, int k) {
        dst.load(wr, woff == kOOB || k >= d ? kOOB : woff + (uint32_t)k * 4u);
    };
    auto step = [&](const Chunk<float>& wc, int k) {
        float wf[8];
        wc.to_float(wf);
        bf16x8_t whi, wmid, wlo;
        split3(wf, whi, wmid, wlo);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(rows + roff[u] + k));
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wlo, xb, acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wmid, xb, acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(whi, xb, acc[u], 0, 0, 0);
        }
    };
    // issued in slot order (as the loop refills them), so that the oldest load
    // in flight is always the next slot's
#pragma unroll
    for (int s = 0; s < kBmWRing; ++s) {
        wload(wring[s], 32 * s);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int nk = d / 32, kr = nk / kBmWRing * kBmWRing;
    for (int k0 = 0; k0 < 32 * kr; k0 += 32 * kBmWRing) {
#pragma unroll
        for (int s = 0; s < kBmWRing; ++s) {
            const int k = k0 + 32 * s;
            step(wring[s], k);
            // refill the slot once its values are consumed, into the same
            // registers (no copies of the ring at the loop's back edge)
            wload(wring[s], k + 32 * kBmWRing);
        }
    }
#pragma unroll
    for (int s = 0; s < kBmWRing - 1; ++s)
        if (kr + s < nk) step(wring[s], 32 * (kr + s));
}

// One workgroup per CU slot, looping over tokens t = blockIdx.x, + gridDim.x, ...
// A token's rows come from registers loaded during the previous token's
// output contraction (the first token's before the loop): the row loads of
// token t + gridDim.x are issued once token t's score contraction is done, so
// that no wait of that contraction (vector memory counts complete in issue
// order) includes them, and they arrive while the outputs are formed.
template <int NCH>
__global__ __launch_bounds__(64 * kBmWaves) void full_batch_mfma_kernel(FwdParams p, int n_rows) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const BmLayout L = bm_layout(n_rows, p.n_q, p.d);
    bf16_t* const rows = reinterpret_cast<bf16_t*>(lds_raw);
    const uint16_t* const rows16 = reinterpret_cast<const uint16_t*>(lds_raw);
    uint16_t* const ap = reinterpret_cast<uint16_t*>(lds_raw + L.ap_off);
    float* const pm = reinterpret_cast<float*>(lds_raw + L.pm_off);
    float* const ps = reinterpret_cast<float*>(lds_raw + L.ps_off);
    float* const rs = reinterpret_cast<float*>(lds_raw + L.rs_off);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = threadIdx.x & 63;
    const int g = ln >> 4, c16 = ln & 15;
    const int d = p.d, dst = L.dst, n_q = p.n_q;
    const int64_t row_elems = p.T * (int64_t)d;
    const uint64_t tok_bytes = (uint64_t)d * 2;
    const cf32_ptr cache = const_view(p.rinv);

    // rows wave + kBmWaves u (u < U) of a token: this lane's 16-byte chunks
    constexpr int U = bm_rows_in_flight<NCH>();
    bool live[NCH];
    uint32_t in_off[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = c * 64 + ln;
        live[c] = ch < p.nc;
        in_off[c] = live[c] ? (uint32_t)(ch * 16) : kOOB;
    }
    Chunk<bf16_t> pf[U][NCH];
    auto prefetch = [&](int64_t tt) {
        const bf16_t* htok = static_cast<const bf16_t*>(p.hist) + tt * d;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = wave + u * kBmWaves;
            // rows past n_rows: a zero-length range (loads return zeros)
            const rsrc_t rr = make_rsrc(htok + (i < n_rows ? i : 0) * row_elems, i < n_rows ? tok_bytes : 0);
#pragma unroll
            for (int c = 0; c < NCH; ++c) pf[u][c].template load<kAuxNT>(rr, in_off[c]);
        }
    };
    if (blockIdx.x < p.T) prefetch(blockIdx.x);

    for (int64_t t = blockIdx.x; t < p.T; t += gridDim.x) {
        // weights start at zero: entries of rows a read's jobs do not cover stay so
        for (int i = threadIdx.x; i < n_q * L.ast / 4; i += blockDim.x)
            reinterpret_cast<u32x4*>(ap)[i] = u32x4{0u, 0u, 0u, 0u};

        // ---- the token's rows into LDS, their RMS scales -------------------------
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = wave + u * kBmWaves;
            if (i < n_rows) {
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    if (live[c]) *reinterpret_cast<u32x4*>(rows + (int64_t)i * dst + 8 * (c * 64 + ln)) = pf[u][c].v;
                float r;
                if (i < p.rinv_valid) {
                    r = cache[(int64_t)i * p.T + t];
                } else {
                    float sq = 0.f;
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        float x[8];
                        pf[u][c].to_float(x);
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
        __syncthreads();

        // ---- scores on the matrix cores ------------------------------------------
        BmJob jobs[kBmJobsPerWave];
        bool has[kBmJobsPerWave];
        f32x4 sc[kBmJobsPerWave][kBmJobTiles];
        const rsrc_t wr = make_rsrc(p.w, (uint64_t)n_q * d * 4);  // reads past n_q load zeros
#pragma unroll
        for (int q = 0; q < kBmJobsPerWave; ++q) {
#pragma unroll
            for (int u = 0; u < kBmJobTiles; ++u) sc[q][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            has[q] = bm_job(p, L.nrt, wave + kBmWaves * q, jobs[q]);
            if (!has[q]) continue;
            const BmJob J = jobs[q];
            const int jq = 16 * J.a + c16;  // this lane's query row (A operand)
            const uint32_t woff = jq < n_q ? (uint32_t)(jq * d + 8 * g) * 4u : kOOB;
            int roff[kBmJobTiles];  // this lane's row (B operand), clamped to a staged row
#pragma unroll
            for (int u = 0; u < kBmJobTiles; ++u) {
                int i = 16 * (J.b0 + u) + c16;
                i = i < n_rows ? i : n_rows - 1;
                roff[u] = i * dst + 8 * g;
            }
            switch (J.nb) {
                case 1: bm_scores<1>(wr, woff, rows, roff, d, sc[q]); break;
                case 2: bm_scores<2>(wr, woff, rows, roff, d, sc[q]); break;
                default: bm_scores<3>(wr, woff, rows, roff, d, sc[q]); break;
            }
        }

        // ---- softmax over each read's rows -----------------------------------------
        // lane (g, c16), register r of job tile u: read j = 16 a + 4 g + r, row
        // i = 16 (b0 + u) + c16; a 16-lane row of the wave holds one read's 16 rows
#pragma unroll
        for (int q = 0; q < kBmJobsPerWave; ++q) {
            if (!has[q]) continue;
            const BmJob J = jobs[q];
#pragma unroll
            for (int u = 0; u < kBmJobTiles; ++u) {
                if (u >= J.nb) continue;
                const int i = 16 * (J.b0 + u) + c16;
                const float ri = rs[i < n_rows ? i : n_rows - 1] * kLog2e;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J.a + 4 * g + r;
                    const bool sees = j < n_q && i <= p.q_begin + j;
                    const float s = sees ? ri * sc[q][u][r] : -INFINITY;
                    sc[q][u][r] = s;
                    const float mx = tg_max<16>(s);
                    if (c16 == 0 && j < n_q) pm[j * L.nrb + J.b0 + u] = mx;
                }
            }
        }
        __syncthreads();
        float Mr[kBmJobsPerWave][4];
#pragma unroll
        for (int q = 0; q < kBmJobsPerWave; ++q) {
            if (!has[q]) continue;
            const BmJob J = jobs[q];
            const int nb_a = bm_tile_rows(p, J.a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * J.a + 4 * g + r;
                // the row tiles' maxima, all loads issued at once (a clamped
                // index repeats the last tile, which leaves the max unchanged)
                const int jc = j < n_q ? j : n_q - 1;
                float M = -INFINITY;
#pragma unroll
                for (int b = 0; b < kBmMaxTiles; ++b) M = fmaxf(M, pm[jc * L.nrb + (b < nb_a ? b : nb_a - 1)]);
                Mr[q][r] = j < n_q ? M : 0.f;  // reads past n_q: any finite value (weights unused)
            }
#pragma unroll
            for (int u = 0; u < kBmJobTiles; ++u) {
                if (u >= J.nb) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J.a + 4 * g + r;
                    const float e = fast_exp2(sc[q][u][r] - Mr[q][r]);  // -inf -> 0
                    sc[q][u][r] = e;
                    const float sm = tg_sum<16>(e);
                    if (c16 == 0 && j < n_q) ps[j * L.nrb + J.b0 + u] = sm;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kBmJobsPerWave; ++q) {
            if (!has[q]) continue;
            const BmJob J = jobs[q];
            const int nb_a = bm_tile_rows(p, J.a);
            float inv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * J.a + 4 * g + r;
                const int jc = j < n_q ? j : n_q - 1;
                float Z = 0.f;  // the row tiles' sums in tile order, all loads issued at once
#pragma unroll
                for (int b = 0; b < kBmMaxTiles; ++b) {
                    const float v = ps[jc * L.nrb + (b < nb_a ? b : nb_a - 1)];
                    Z += b < nb_a ? v : 0.f;
                }
                if (j < n_q && J.b0 == 0 && c16 == 0 && p.lse != nullptr)
                    p.lse[(int64_t)j * p.T + t] = (Mr[q][r] + fast_log2(Z)) * kLn2;
                inv[r] = j < n_q ? 1.0f / Z : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kBmJobTiles; ++u) {
                if (u >= J.nb) continue;
                const int i = 16 * (J.b0 + u) + c16;
                const int kk = 32 * (i >> 5) + bm_kidx(i & 31);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * J.a + 4 * g + r;
                    if (j >= n_q) continue;
                    const float a = sc[q][u][r] * inv[r];
                    const uint32_t hp = pack_bf16x2(a, 0.f) & 0xffffu;
                    const uint32_t lp = pack_bf16x2(a - __uint_as_float(hp << 16), 0.f) & 0xffffu;
                    ap[(int64_t)j * L.ast + kk] = (uint16_t)hp;
                    ap[(int64_t)(n_q + j) * L.ast + kk] = (uint16_t)lp;
                    if (p.alpha != nullptr && i < p.n_hist)
                        p.alpha[((int64_t)j * p.n_hist + i) * p.T + t] = a;
                }
            }
        }
        if (p.alpha != nullptr) {  // rows past the tiles a read sees
            for (int k = threadIdx.x; k < n_q * p.n_hist; k += blockDim.x) {
                const int j = k / p.n_hist, i = k - j * p.n_hist;
                if (i >= 16 * bm_tile_rows(p, j / 16)) p.alpha[((int64_t)j * p.n_hist + i) * p.T + t] = 0.f;
            }
        }
        __syncthreads();

        // ---- outputs on the matrix cores --------------------------------------------
        // the next token's rows, in flight while this token's outputs are formed
        if (t + gridDim.x < p.T) prefetch(t + gridDim.x);
        // wave w takes the column tiles [w ne / 8, (w + 1) ne / 8) (16 columns each).
        // A column tile's row fragments are read once for every row step (lane
        // 4 e + q of lane group g fetches columns 4 q .. 4 q + 3 of row
        // 32 ks + 8 g + 2 e + s for read s; past the last row the last row, whose
        // weights are zero there or which no read tile uses), then each read tile
        // in turn multiplies the steps it needs into one accumulator and stores
        // it (a read past n_q reads the last read's weights and stores nothing).
        const int ne = d / 16;
        const int et0 = wave * ne / kBmWaves, et1 = (wave + 1) * ne / kBmWaves;
        int toff[kBmMaxKs][2];
#pragma unroll
        for (int ks = 0; ks < kBmMaxKs; ++ks)
#pragma unroll
            for (int sr = 0; sr < 2; ++sr) {
                const int i = 32 * ks + 8 * g + 2 * (c16 >> 2) + sr;
                toff[ks][sr] = (i < n_rows ? i : n_rows - 1) * dst + 4 * (c16 & 3);
            }
        const int aplane = n_q * L.ast;  // elements from a weight's hi part to its lo part
        for (int et = et0; et < et1; ++et) {
            const int e0 = 16 * et;
            bf16x8_t xa[kBmMaxKs];
#pragma unroll
            for (int ks = 0; ks < kBmMaxKs; ++ks) {
                const bm_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (bm_lds_v4s*)(const_cast<uint16_t*>(rows16) + toff[ks][0] + e0));
                const bm_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (bm_lds_v4s*)(const_cast<uint16_t*>(rows16) + toff[ks][1] + e0));
                xa[ks] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            for (int a = 0; a < L.nrt; ++a) {
                const int ks_last = (bm_tile_rows(p, a) * 16 - 1) / 32;
                const int j = 16 * a + c16;
                const int jc = j < n_q ? j : n_q - 1;
                const uint16_t* arow = ap + jc * L.ast + 8 * g;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < kBmMaxKs; ++ks) {
                    if (ks > ks_last) break;
#pragma unroll
                    for (int part = 0; part < 2; ++part) {
                        const u32x4 bv = *reinterpret_cast<const u32x4*>(arow + part * aplane + 32 * ks);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[ks], __builtin_bit_cast(bf16x8_t, bv), acc, 0,
                                                                      0, 0);
                    }
                }
                // lane (g, c16): columns e0 + 4 g .. + 3 of read j
                if (j < n_q) {
                    uint32_t* dstp = reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(p.out) + (int64_t)j * row_elems +
                                                                 t * d + e0 + 4 * g);
                    dstp[0] = pack_bf16x2(acc[0], acc[1]);
                    dstp[1] = pack_bf16x2(acc[2], acc[3]);
                }
            }
        }
        __syncthreads();  // the next token may overwrite the rows and weights
    }
}

template <int NCH>
hipError_t launch_bm(const FwdParams& p, int n_rows, size_t lds, hipStream_t stream) {
    const void* kern = (const void*)full_batch_mfma_kernel<NCH>;
    hipError_t e = prepare_dynamic_lds(kern, lds);
    if (e != hipSuccess) return e;
    // as many workgroups as the device holds at once, each looping over tokens
    int64_t slots = 0;
    if ((e = resident_workgroups(kern, 64 * kBmWaves, lds, &slots)) != hipSuccess) return e;
    const int64_t grid = p.T < slots ? p.T : slots;
    hipLaunchKernelGGL(full_batch_mfma_kernel<NCH>, dim3((unsigned)grid), dim3(64 * kBmWaves), lds, stream, p,
                       n_rows);
    return hipGetLastError();
}

// LDS bytes of a call the kernel takes, or 0
int64_t bm_plan(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt) {
    if (hist_dt != ATTNRES_BF16 || out_dt != ATTNRES_BF16) return 0;
    if (p.qtok != nullptr || p.normed != nullptr || p.n_q < kBmMinReads) return 0;
    if (p.d % 32 != 0 || p.nc > 4 * 64) return 0;
    const int n_rows = p.q_begin + p.n_q;
    // one round of row loads per wave covers the token
    const int nch = (p.nc + 63) / 64;
    const int rows_per_round = kBmWaves * (nch == 1   ? bm_rows_in_flight<1>()
                                           : nch == 2 ? bm_rows_in_flight<2>()
                                           : nch == 3 ? bm_rows_in_flight<3>()
                                                      : bm_rows_in_flight<4>());
    if (n_rows > rows_per_round) return 0;
    if (n_rows > 16 * kBmMaxTiles || p.n_q > 16 * kBmMaxTiles) return 0;
    if (p.T * 64 * kBmWaves >= ((int64_t)1 << 32)) return 0;
    const BmLayout L = bm_layout(n_rows, p.n_q, p.d);
    if (bm_num_jobs(p, L.nrt) > kBmWaves * kBmJobsPerWave) return 0;
    const int max_lds = device_max_lds();
    if (max_lds <= 0 || L.bytes > max_lds) return 0;
    return L.bytes;
}

}  // namespace

bool full_batch_mfma_applies(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt) {
    return bm_plan(p, hist_dt, out_dt) > 0;
}

int full_batch_mfma_prefix(const FwdParams& p, attnres_dtype hist_dt, attnres_dtype out_dt) {
    if (bm_plan(p, hist_dt, out_dt) > 0) return 0;  // the kernel takes the whole call
    FwdParams q = p;
    // the most reads whose rows (0 .. q_begin + n - 1) the kernel stages
    for (int n = std::min(p.n_q - 1, 16 * kBmMaxTiles - p.q_begin); n >= kBmMinReads; --n) {
        q.n_q = n;
        if (bm_plan(q, hist_dt, out_dt) > 0) return n;
    }
    return 0;
}

hipError_t launch_full_batch_mfma(const FwdParams& p, hipStream_t stream) {
    const int64_t lds = bm_plan(p, ATTNRES_BF16, ATTNRES_BF16);
    if (lds <= 0) return hipErrorInvalidValue;
    const int n_rows = p.q_begin + p.n_q;
    switch ((p.nc + 63) / 64) {
        case 1: return launch_bm<1>(p, n_rows, (size_t)lds, stream);
        case 2: return launch_bm<2>(p, n_rows, (size_t)lds, stream);
        case 3: return launch_bm<3>(p, n_rows, (size_t)lds, stream);
        case 4: return launch_bm<4>(p, n_rows, (size_t)lds, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attnres
