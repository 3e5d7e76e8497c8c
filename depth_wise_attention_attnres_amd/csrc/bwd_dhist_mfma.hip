// bwd_dhist_mfma.hip -- the backward's history gradient on the matrix cores.
//
// For one token t the history gradient (the derivative of the read of
// "DepthBench reading notes" sec. 2.3, block reading of sec. 2.5; the
// coefficients are formed by the coefficient kernels of bwd.hip) is
//   dv_i = sum_l A1[l][i] g_l + sum_l A2[l][i] w_l - sum_m coef(i, m) v_m,
// with coef(i, m) = C3[c] + K(max(i, m)) for rows i, m of one block c (v_0 a
// block of its own; K(m) the kappa of the reads whose partial sum holds row
// m, summed) and 0 across blocks.  Columns k of d are independent, so per
// token this is one small matrix product over K = reads (g), reads (w),
// rows (v):  D[k][i] = sum over K of Aop[k][K] B[K][i],  B = A1 ++ A2 ++ -coef.
// It runs on v_mfma_f32_32x32x16_bf16.  The history rows and upstream
// gradients are bf16 already; the fp32 coefficients enter as bf16 hi + lo
// and w as bf16 hi + mid, each exact to about 2^-17 relative (w's mid part
// meets A2's hi part only).  That is far below the bf16 rounding of the
// result, which is why only bf16 gradients take this kernel; fp32 gradients
// keep the fp32 vector kernel of bwd.hip.
//
// One workgroup of eight waves per token.  The token's B operands are split
// and laid out as matrix fragments in LDS once; K is packed (the four row
// sets back to back, padded only at the end).  The A operands are rows of
// dout, w and the history, read 16 rows (one 16-step) at a time: the waves
// load the step's rows for 512 columns of d together, one 1 KB row segment
// per load (a load that spans several rows, each in its own page, stalls the
// address unit), into an LDS tile; after a barrier every lane reads back the
// column it needs for its MFMA operand (a transposed read), and a second
// barrier frees the tile.  Wave w owns columns 64 w .. 64 w + 63 of each
// 512-column pass: two 32-column output tiles.  Loads run two steps ahead.
// The results leave the same way in reverse: 16 rows at a time through the
// tile, one 1 KB row segment per store (a store spanning 32 rows, one per
// lane pair, stalled like the loads).
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bm_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bm_v4s bm_lds_v4s;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDmWaves = 8;
constexpr int kDmMaxNT = 3;            // row tiles of 32 (at most 96 history rows)
constexpr int kDmMaxLds = 128 * 1024;  // LDS bytes a workgroup may use
constexpr int kDmRing = 2;             // 16-steps in flight per wave
constexpr int kDmCols = 64 * kDmWaves;  // columns of d per pass of a workgroup
constexpr int kDmRow = kDmCols + 8;     // bf16 per row of the LDS step tile (8 padding)

__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16x2(x, 0.f) & 0xffffu; }

// x = hi + lo + r with hi, lo bf16 (round to nearest even) and |r| <= 2^-17 |x|
__device__ __forceinline__ void split2(float x, uint32_t& hi, uint32_t& lo) {
    hi = bf16_bits(x);
    lo = bf16_bits(x - __uint_as_float(hi << 16));
}

__device__ __forceinline__ int block_of_row(int j, int S) { return j == 0 ? 0 : (j - 1) / S + 1; }

// w split into two bf16 parts, row-major: wsp[0] = hi, wsp[1] = mid
__global__ __launch_bounds__(256) void split_w2_kernel(const float* w, int64_t n, uint16_t* wsp) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    uint32_t hi, mid;
    split2(w[i], hi, mid);
    wsp[i] = (uint16_t)hi;
    wsp[n + i] = (uint16_t)mid;
}

template <int NT, int RING>
__global__ __launch_bounds__(512) void bwd_dhist_mfma_kernel(BwdParams p, int nsteps) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
    const int h = ln >> 5, m = ln & 31;
    const int64_t t = blockIdx.x;
    // K runs over the reads' dout rows, w's hi and mid rows, then the history
    // rows, packed (not padded per operand): nsteps 16-steps of K
    const int k_w = p.n_q, k_m = 2 * p.n_q, k_v = 3 * p.n_q;
    const int S = p.S;
    const int q_end = p.q_begin + p.n_q;

    extern __shared__ float lds[];
    u32x4* frag = reinterpret_cast<u32x4*>(lds);                   // [nsteps][NT][hi, lo][64 lanes]
    float* cf = lds + (size_t)nsteps * NT * 2 * 64 * 4;            // [n_hist] C3[block] + K(row)
    const int cf_floats = (p.n_hist + 3) & ~3;                     // then the step tile

    // ---- per-row coupling coefficient C3[c] + K(j) --------------------------
    const float* C3 = p.ws_c3 + t * p.n_blk;
    const float* kap = p.ws_kappa + t * p.n_q;
    for (int j = tid; j < p.n_hist; j += blockDim.x) {
        const int c = block_of_row(j, S);
        float K = 0.f;
        if (c > 0) {
            const int Lc = c * S - 1 < q_end - 1 ? c * S - 1 : q_end - 1;
            for (int l = j > p.q_begin ? j : p.q_begin; l <= Lc; ++l) K += kap[l - p.q_begin];
        }
        cf[j] = C3[c] + K;
    }
    __syncthreads();

    // ---- B operands: lane (hh, i) of fragment (ks, nt) holds K = 16 ks + 8 hh + j:
    // A1 (dout rows), A2 (w hi rows; w mid rows against A2's hi part only:
    // their lo fragment is 0), -coef (history rows)
    const float* A1 = p.ws_a1 + t * (int64_t)p.n_q * p.nh8;
    const float* A2 = p.ws_a2 + t * (int64_t)p.n_q * p.nh8;
    for (int e = tid; e < nsteps * NT * 64; e += blockDim.x) {
        const int L = e & 63, fn = e >> 6;
        const int nt = fn % NT, ks = fn / NT;
        const int hh = L >> 5, i = 32 * nt + (L & 31);
        const int ci = i < p.n_hist ? block_of_row(i, S) : -1;
        float v[8];
        bool lo_zero[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = 16 * ks + 8 * hh + j;
            float x = 0.f;
            if (ci >= 0) {
                if (k < k_w) {
                    x = A1[(int64_t)k * p.nh8 + i];
                } else if (k < k_v) {
                    x = A2[(int64_t)(k < k_m ? k - k_w : k - k_m) * p.nh8 + i];
                } else if (k - k_v < p.n_hist) {
                    const int r = k - k_v;
                    x = block_of_row(r, S) == ci ? -cf[r > i ? r : i] : 0.f;
                }
            }
            v[j] = x;
            lo_zero[j] = k >= k_m && k < k_v;
        }
        u32x4 hi4, lo4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t h0, l0, h1, l1;
            split2(v[2 * q], h0, l0);
            split2(v[2 * q + 1], h1, l1);
            if (lo_zero[2 * q]) l0 = 0u;
            if (lo_zero[2 * q + 1]) l1 = 0u;
            hi4[q] = h0 | (h1 << 16);
            lo4[q] = l0 | (l1 << 16);
        }
        frag[(fn * 2 + 0) * 64 + L] = hi4;
        frag[(fn * 2 + 1) * 64 + L] = lo4;
    }
    __syncthreads();

    // ---- A operands -----------------------------------------------------------
    // Wave w loads rows 2 w and 2 w + 1 of each 16-step across the pass; lane
    // (h, m) of output tile kk then takes column 64 w + 32 kk + m of the
    // step's rows 8 h .. 8 h + 7 (K = 8 h + j is row 8 h + j).
    const int64_t row_elems = p.T * (int64_t)p.d;
    const bf16_t* dout_t = static_cast<const bf16_t*>(p.dout) + t * p.d;
    const bf16_t* hist_t = static_cast<const bf16_t*>(p.hist) + t * p.d;
    const bf16_t* wsp = reinterpret_cast<const bf16_t*>(p.ws_wsplit2);  // [hi, mid][n_q][d]
    // the step tile: 16 rows x kDmCols bf16, rows padded to kDmRow (the two
    // half-waves read rows eight apart, 32 banks apart)
    uint16_t* tb = reinterpret_cast<uint16_t*>(cf + cf_floats);

    struct Slot {
        u32x4 x, y;  // this wave's two rows of the step
    };
    // Row k of K: dout row k, w hi / mid row, or history row.  A row past
    // the end of K, or a step past the last, gets an empty range (zeros);
    // columns past d read zeros from the row's range.
    const bf16_t* w_mid = wsp + (int64_t)p.n_q * p.d;
    const int k_end = k_v + p.n_hist;
    auto gather = [&](int k0, bool live, uint32_t coff, Slot& sl) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int k = k0 + 2 * wave + e;
            const bool ok = live && k < k_end;
            const bf16_t* base = k < k_w ? dout_t + (int64_t)k * row_elems
                                 : k < k_m ? wsp + (int64_t)(k - k_w) * p.d
                                 : k < k_v ? w_mid + (int64_t)(k - k_m) * p.d
                                           : hist_t + (int64_t)(k - k_v) * row_elems;
            const rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16_t*>(ok ? base : hist_t), (short)0, ok ? 2 * p.d : 0, (int)kRsrcWord3);
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr, coff, 0, 0);
            if (e == 0) sl.x = v; else sl.y = v;
        }
    };
    auto bfrag = [&](int ks, int nt, int part) {
        return __builtin_bit_cast(bf16x8_t, frag[((ks * NT + nt) * 2 + part) * 64 + ln]);
    };

    // nsteps 16-steps per pass.  A ring of RING register slots runs over all
    // passes: step sigma + RING is issued as soon as step sigma has gone to LDS.
    const int n_pass = (p.d + kDmCols - 1) / kDmCols;
    const int total = n_pass * nsteps;
    int i_pass = 0, i_st = 0;  // the next step to issue
    auto issue = [&](Slot& sl) {
        gather(16 * i_st, i_pass < n_pass, (uint32_t)(i_pass * kDmCols * 2 + 16 * ln), sl);
        const bool wrap = i_st == nsteps - 1;
        i_st = wrap ? 0 : i_st + 1;
        i_pass += wrap ? 1 : 0;
    };

    f32x16 acc[2][NT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[kk][nt][r] = 0.f;
    Slot ring[RING];
#pragma unroll
    for (int u = 0; u < RING; ++u) issue(ring[u]);
    bf16_t* dh_t = static_cast<bf16_t*>(p.dhist) + t * p.d;
    int c_pass = 0, c_st = 0;  // the step being consumed
    // whole rounds of RING steps; steps past the last one carry zeros
    for (int s0 = 0; s0 < total; s0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            *reinterpret_cast<u32x4*>(tb + (2 * wave) * kDmRow + 8 * ln) = ring[u].x;
            *reinterpret_cast<u32x4*>(tb + (2 * wave + 1) * kDmRow + 8 * ln) = ring[u].y;
            issue(ring[u]);
            __syncthreads();  // the step's 16 rows are in LDS
            bf16x8_t a[2];
            {
                // rows 8 h + 4 s + e (e = 0..3) of column 64 w + 32 kk + m from
                // transposing reads (ds_read_b64_tr_b16: within 16 lanes, lane c
                // receives element c mod 4 of the 8-byte chunks that lanes
                // 4 e + c / 4 fetch): lane 4 e + q of a 16-lane group fetches
                // columns 4 q .. 4 q + 3 of the group's 16 of row 8 h + 4 s + e
                bm_v4s tr[2][2];
                const int c16 = ln & 15;
                const uint16_t* tq = tb + (8 * h + (c16 >> 2)) * kDmRow + 64 * wave + 16 * ((ln >> 4) & 1) + 4 * (c16 & 3);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int sr = 0; sr < 2; ++sr)
                        tr[kk][sr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (bm_lds_v4s*)(const_cast<uint16_t*>(tq) + 4 * sr * kDmRow + 32 * kk));
                u32x4 t0 = __builtin_bit_cast(u32x4, __builtin_shufflevector(tr[0][0], tr[0][1], 0, 1, 2, 3, 4, 5, 6, 7));
                u32x4 t1 = __builtin_bit_cast(u32x4, __builtin_shufflevector(tr[1][0], tr[1][1], 0, 1, 2, 3, 4, 5, 6, 7));
                // the operands exist here (an empty statement the compiler
                // cannot move them across): every wave has read the tile when
                // the next barrier lets the next step write it
                asm volatile("" : "+v"(t0), "+v"(t1));
                a[0] = __builtin_bit_cast(bf16x8_t, t0);
                a[1] = __builtin_bit_cast(bf16x8_t, t1);
            }
            __syncthreads();
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    const bf16x8_t b = bfrag(c_st, nt, part);
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        acc[kk][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b, acc[kk][nt], 0, 0, 0);
                }
            if (c_st == nsteps - 1) {
                // The pass's rows leave one 1 KB row segment per store: in rounds of 16
                // rows through the step tile (free: every wave passed this step's second
                // barrier).  Lane (h, m), register r of tile kk holds column 64 w + 32 kk +
                // 8 (r / 4) + 4 h + r % 4 of row 32 nt + m.
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        if ((m >> 4) == half) {
#pragma unroll
                            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                                for (int g = 0; g < 4; ++g)
                                    *reinterpret_cast<uint2*>(tb + (m & 15) * kDmRow + 64 * wave + 32 * kk + 8 * g + 4 * h) =
                                        make_uint2(pack_bf16x2(acc[kk][nt][4 * g], acc[kk][nt][4 * g + 1]),
                                                   pack_bf16x2(acc[kk][nt][4 * g + 2], acc[kk][nt][4 * g + 3]));
                        }
                        __syncthreads();
#pragma unroll
                        for (int e = 0; e < 2; ++e) {  // tile rows 2 w, 2 w + 1
                            const int i = 32 * nt + 16 * half + 2 * wave + e;
                            const int col = c_pass * kDmCols + 8 * ln;
                            if (i < p.n_hist && col < p.d)
                                *reinterpret_cast<u32x4*>(dh_t + i * row_elems + col) =
                                    *reinterpret_cast<const u32x4*>(tb + (2 * wave + e) * kDmRow + 8 * ln);
                        }
                        __syncthreads();  // the tile is read before its next use
                    }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[kk][nt][r] = 0.f;
                c_st = 0;
                ++c_pass;
            } else {
                ++c_st;
            }
        }
    }
}

int dm_nt(const BwdParams& p) { return (p.n_hist + 31) / 32; }

int dm_steps(const BwdParams& p) { return (3 * p.n_q + p.n_hist + 15) / 16; }

size_t dm_lds(const BwdParams& p) {
    return (size_t)dm_steps(p) * dm_nt(p) * 2 * 64 * 16 + (size_t)((p.n_hist + 3) & ~3) * 4 +
           (size_t)16 * kDmRow * 2;
}

}  // namespace

int64_t bwd_wsplit2_elems(int64_t n_q, int64_t d) { return 2 * n_q * d; }

bool bwd_dhist_mfma_applies(const BwdParams& p) {
    if (p.hist_dt != ATTNRES_BF16 || p.dout_dt != ATTNRES_BF16 || p.dhist_dt != ATTNRES_BF16)
        return false;
    if (p.accumulate || p.n_q < 1 || dm_nt(p) > kDmMaxNT) return false;
    const size_t lds = dm_lds(p);
    return lds <= (size_t)kDmMaxLds && lds <= (size_t)device_max_lds();
}

hipError_t launch_bwd_dhist_mfma(const BwdParams& p, hipStream_t stream) {
    const int nsteps = dm_steps(p);
    const int64_t nw = (int64_t)p.n_q * p.d;
    hipLaunchKernelGGL(split_w2_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, stream, p.w,
                       nw, p.ws_wsplit2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = dm_lds(p);
    const void* kern;
    switch (dm_nt(p)) {
        case 1: kern = reinterpret_cast<const void*>(&bwd_dhist_mfma_kernel<1, kDmRing>); break;
        case 2: kern = reinterpret_cast<const void*>(&bwd_dhist_mfma_kernel<2, kDmRing>); break;
        default: kern = reinterpret_cast<const void*>(&bwd_dhist_mfma_kernel<3, kDmRing>); break;
    }
    e = prepare_dynamic_lds(kern, (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)p.T), block(64 * kDmWaves);
    switch (dm_nt(p)) {
        case 1: hipLaunchKernelGGL((bwd_dhist_mfma_kernel<1, kDmRing>), grid, block, lds, stream, p, nsteps); break;
        case 2: hipLaunchKernelGGL((bwd_dhist_mfma_kernel<2, kDmRing>), grid, block, lds, stream, p, nsteps); break;
        default: hipLaunchKernelGGL((bwd_dhist_mfma_kernel<3, kDmRing>), grid, block, lds, stream, p, nsteps); break;
    }
    return hipGetLastError();
}

}  // namespace attnres
