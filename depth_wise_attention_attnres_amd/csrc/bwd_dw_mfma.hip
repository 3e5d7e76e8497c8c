// bwd_dw_mfma.hip -- the backward's query gradient dw on the matrix cores
// (bf16 history).
//
// dw_l = sum over tokens t and rows i of A2T[t][i][l] v_{t,i} (the dw term of
// the read derivative; "DepthBench reading notes" sec. 2.3, block reading of
// sec. 2.5; A2T is formed by the coefficient kernels of bwd.hip).  Per chunk
// of 32 tokens this is the partial product
//   P[k][l] = sum over (t, i) of X[k][(t, i)] A2T[(t, i)][l],
// on v_mfma_f32_32x32x16_bf16 with K = 16 tokens of one row per step.  The
// history is bf16; each fp32 coefficient enters as three bf16 parts
// hi + mid + lo, which represent it exactly (24 significant bits), and every
// product of a part with a bf16 value is exact in the fp32 accumulator: the
// partial equals an fp32 contraction up to the order of the additions.  The
// partials go to the same buffer as those of the fp32 kernel in bwd.hip and
// are reduced by its fixed-order sum.
//
// One workgroup of eight waves per (chunk, 512-column pass); wave w owns
// columns 64 w .. 64 w + 63 of the pass (two 32-column tiles) and keeps its
// partials for all reads of the call (at most 64: two 32-read tiles) in
// registers across the chunk.  A step (row i, 16 tokens) is loaded by the
// whole workgroup: wave w loads the row segments of two tokens (1 KB each)
// into an LDS tile, every thread loads two coefficients and writes their
// split parts as matrix fragments; after a barrier each lane reads its
// column of the tile (a transposed read), a second barrier frees the tile.
// Loads run two steps ahead.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short dw_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dw_v4s dw_lds_v4s;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDwWaves = 8;
constexpr int kDwCols = 64 * kDwWaves;  // columns of d per workgroup
constexpr int kDwRow = kDwCols + 8;     // bf16 per row of the LDS tile (8 padding)
constexpr int kDwRing = 2;              // steps in flight per wave
constexpr int kDwMaxNL = 2;             // 32-read tiles (at most 64 reads)
constexpr int kDwChunk = 32;            // tokens per chunk (two 16-token steps per row)

__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16x2(x, 0.f) & 0xffffu; }

// x = hi + mid + lo exactly (round to nearest even at each stage)
__device__ __forceinline__ void split3(float x, uint32_t (&part)[3]) {
    part[0] = bf16_bits(x);
    const float r1 = x - __uint_as_float(part[0] << 16);
    part[1] = bf16_bits(r1);
    part[2] = bf16_bits(r1 - __uint_as_float(part[1] << 16));
}

template <int NL, int RING>
__global__ __launch_bounds__(512) void bwd_dw_mfma_kernel(BwdParams p) {
    static_assert(RING % 2 == 0, "the fragment block alternates with the step");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), ln = tid & 63;
    const int h = ln >> 5, m = ln & 31;
    // the passes of a chunk share an XCD: the chunk's coefficients come from
    // HBM once, then from that L2
    const int n_pass = (p.d + kDwCols - 1) / kDwCols;
    int64_t chunk64;
    int pass;
    xcd_group(blockIdx.x, n_pass, chunk64, pass);
    const int n_chunks = (int)((p.T + kDwChunk - 1) / kDwChunk);
    if (chunk64 >= n_chunks) return;  // the whole workgroup
    const int chunk = (int)chunk64;
    const int64_t t_lo = (int64_t)chunk * kDwChunk;
    const int n_tok = (int)(p.T - t_lo < kDwChunk ? p.T - t_lo : kDwChunk);
    const int64_t row_elems = p.T * (int64_t)p.d;
    const int64_t a2t_tok = (int64_t)p.n_hist * p.nq8;  // floats per token of A2T

    extern __shared__ float lds[];
    uint16_t* tile = reinterpret_cast<uint16_t*>(lds);                     // [16 tokens][kDwRow]
    uint32_t* bfr = reinterpret_cast<uint32_t*>(lds) + 16 * kDwRow / 2;  // [2][NL][3][64 lanes][4]
    constexpr int kBfrWords = NL * 3 * 64 * 4;

    // Steps: row i = s / 2, tokens 16 (s % 2) .. + 15 of the chunk.
    const int nr = p.q_begin + p.n_q;  // rows any read of the call sees (A2T is 0 past)
    const int n_steps = 2 * nr;

    // This thread's coefficient pair: (read tile lt, read n, lane half hh,
    // tokens j, j + 1 of the half's 8) -- fragment lane hh * 32 + n, dword j / 2.
    const int pr = tid < NL * 256 ? tid : 0;
    const bool pr_ok = tid < NL * 256;
    const int pj = 2 * (pr & 3), phh = (pr >> 2) & 1, pn = (pr >> 3) & 31, plt = pr >> 8;
    const int pl = 32 * plt + pn;  // the read
    const uint32_t tcol = (uint32_t)(pass * kDwCols * 2 + 16 * ln);  // tile load column offset
    const rsrc_t rcoef = make_rsrc(p.ws_a2t + t_lo * a2t_tok, (uint64_t)n_tok * a2t_tok * 4);

    struct Slot {
        u32x4 x, y;  // this wave's two token rows of the step
        float b0, b1;  // this thread's coefficient pair
    };
    auto issue = [&](int s, Slot& sl) {  // selects only: the four loads share one block
        const bool live = s < n_steps;
        const int i = live ? s >> 1 : 0;
        const int t0 = 16 * (live ? s & 1 : 0);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int tk = t0 + 2 * wave + k;  // token of the chunk
            const bool ok = live && tk < n_tok;
            const rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<void*>(static_cast<const void*>(static_cast<const bf16_t*>(p.hist) +
                                                          i * row_elems + (t_lo + (ok ? tk : 0)) * p.d)),
                (short)0, ok ? 2 * p.d : 0, (int)kRsrcWord3);
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr, tcol, 0, 0);
            if (k == 0) sl.x = v; else sl.y = v;
        }
        // coefficients of tokens t0 + 8 phh + pj (+ 1), row i, read pl: one
        // descriptor over the chunk's A2T, per-lane offsets
        const int tb = t0 + 8 * phh + pj;
        const bool cok = live && pr_ok && pl < p.nq8;
        const uint32_t coff = (uint32_t)(((int64_t)tb * a2t_tok + (int64_t)i * p.nq8 + pl) * 4);
        sl.b0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rcoef, cok && tb < n_tok ? coff : kOOB, 0, 0));
        sl.b1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rcoef, cok && tb + 1 < n_tok ? coff + (uint32_t)(a2t_tok * 4) : kOOB, 0, 0));
    };

    f32x16 acc[2][NL];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int lt = 0; lt < NL; ++lt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[kk][lt][r] = 0.f;
    Slot ring[RING];
#pragma unroll
    for (int u = 0; u < RING; ++u) issue(u, ring[u]);

    for (int s0 = 0; s0 < n_steps; s0 += RING) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const int s = s0 + u;
            // the step's token rows and split coefficients into LDS (the
            // fragment block alternates: its readers of two steps ago have
            // passed the barriers of the step between)
            uint32_t* bf = bfr + (u & 1) * kBfrWords;
            *reinterpret_cast<u32x4*>(tile + (2 * wave) * kDwRow + 8 * ln) = ring[u].x;
            *reinterpret_cast<u32x4*>(tile + (2 * wave + 1) * kDwRow + 8 * ln) = ring[u].y;
            if (pr_ok) {
                uint32_t p0[3], p1[3];
                split3(ring[u].b0, p0);
                split3(ring[u].b1, p1);
#pragma unroll
                for (int part = 0; part < 3; ++part)
                    bf[((plt * 3 + part) * 64 + phh * 32 + pn) * 4 + pj / 2] = p0[part] | (p1[part] << 16);
            }
            issue(s + RING, ring[u]);
            __syncthreads();  // the step is in LDS
            bf16x8_t a[2];
            {
                // tokens 8 h + 4 s + e (e = 0..3) of column 64 w + 32 kk + m from
                // transposing reads (ds_read_b64_tr_b16: within 16 lanes, lane c
                // receives element c mod 4 of the 8-byte chunks that lanes
                // 4 e + c / 4 fetch): lane 4 e + q of a 16-lane group fetches
                // columns 4 q .. 4 q + 3 of the group's 16 of token 8 h + 4 s + e
                dw_v4s tr[2][2];
                const int c16 = ln & 15;
                const uint16_t* tq = tile + (8 * h + (c16 >> 2)) * kDwRow + 64 * wave + 16 * ((ln >> 4) & 1) + 4 * (c16 & 3);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int sr = 0; sr < 2; ++sr)
                        tr[kk][sr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (dw_lds_v4s*)(const_cast<uint16_t*>(tq) + 4 * sr * kDwRow + 32 * kk));
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
            if (s < n_steps) {
#pragma unroll
                for (int lt = 0; lt < NL; ++lt)
#pragma unroll
                    for (int part = 0; part < 3; ++part) {
                        const bf16x8_t b = __builtin_bit_cast(
                            bf16x8_t, *reinterpret_cast<const u32x4*>(bf + ((lt * 3 + part) * 64 + ln) * 4));
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk)
                            acc[kk][lt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b, acc[kk][lt], 0, 0, 0);
                    }
            }
        }
    }

    // lane (h, m), register r of tile (kk, lt): column pass kDwCols + 64 w +
    // 32 kk + 8 (r / 4) + 4 h + r % 4, read 32 lt + m
#pragma unroll
    for (int lt = 0; lt < NL; ++lt) {
        const int l = 32 * lt + m;
        if (l < p.n_q) {
            float* part = p.ws_dwpart + ((int64_t)chunk * p.n_q + l) * p.d;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = pass * kDwCols + 64 * wave + 32 * kk + 8 * g + 4 * h;
                    if (col < p.d)
                        *reinterpret_cast<f32x4*>(part + col) = {acc[kk][lt][4 * g], acc[kk][lt][4 * g + 1],
                                                                 acc[kk][lt][4 * g + 2], acc[kk][lt][4 * g + 3]};
                }
        }
    }
}

int dw_nl(const BwdParams& p) { return (p.n_q + 31) / 32; }

size_t dw_lds(const BwdParams& p) {
    return (size_t)16 * kDwRow * 2 + (size_t)2 * dw_nl(p) * 3 * 64 * 16;
}

}  // namespace

bool bwd_dw_mfma_applies(const BwdParams& p) {
    if (p.hist_dt != ATTNRES_BF16 || p.n_q < 1 || dw_nl(p) > kDwMaxNL) return false;
    return dw_lds(p) <= (size_t)device_max_lds();
}

hipError_t launch_bwd_dw_mfma(const BwdParams& p, int chunk_tokens, hipStream_t stream) {
    if (chunk_tokens != kDwChunk) return hipErrorInvalidValue;  // the partials' chunking
    const int n_pass = (p.d + kDwCols - 1) / kDwCols;
    const int64_t n_chunks = (p.T + chunk_tokens - 1) / chunk_tokens;
    const unsigned blocks = (unsigned)((n_chunks + kNumXcd - 1) / kNumXcd) * kNumXcd * n_pass;
    const size_t lds = dw_lds(p);
    const void* kern = dw_nl(p) == 1 ? reinterpret_cast<const void*>(&bwd_dw_mfma_kernel<1, kDwRing>)
                                     : reinterpret_cast<const void*>(&bwd_dw_mfma_kernel<2, kDwRing>);
    hipError_t e = prepare_dynamic_lds(kern, (int)lds);
    if (e != hipSuccess) return e;
    if (dw_nl(p) == 1)
        hipLaunchKernelGGL((bwd_dw_mfma_kernel<1, kDwRing>), dim3(blocks), dim3(64 * kDwWaves), lds, stream, p);
    else
        hipLaunchKernelGGL((bwd_dw_mfma_kernel<2, kDwRing>), dim3(blocks), dim3(64 * kDwWaves), lds, stream, p);
    return hipGetLastError();
}

}  // namespace attnres
