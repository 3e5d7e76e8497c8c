// query_proj.hip -- the input-dependent query of the AttnRes ablation ("Kimi K3
// notes 2", sec. 6: a d x d projection of the current hidden state replaces
// the learned per-read query): q[j][t] = W[j] x[j][t] for every read j and
// token t.  A dense contraction over d, on the matrix cores:
// v_mfma_f32_32x32x16_bf16, D[32 tokens x 32 outputs] += A B with
//   A[i][k] = x[token t0 + i][k]   (lane j: token j % 32, k = 8 (j / 32) .. + 7)
//   B[k][n] = W[output o0 + n][k]  (lane j: output j % 32, same k)
// so both operands are 8 consecutive k of one row.  bf16 x bf16 products are
// exact in fp32 and each accumulator is one fp32 chain over d / 16 <= 256
// steps, so its rounding is that of a plain fp32 sum of d terms.
#include "device_common.hpp"
#include "launch.hpp"

namespace attnres {

namespace {
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
}  // namespace

// Workgroup tile: 256 tokens x 256 outputs; wave (wr, wc) of the 2 x 4 waves
// computes 128 x 64 as 4 x 2 fragments of 32 x 32, so each token fragment read
// from LDS feeds two matrix instructions and each W fragment four (6 LDS reads
// per 8 instructions).  K goes in stages of 32 elements through
// double-buffered LDS (80 KB, one workgroup of 8 waves per CU): the workgroup
// loads a stage's 256 token rows and 256 W rows (contiguous in k, 16 bytes per
// lane) three stages ahead of its multiplication; one barrier per stage.  The
// call is bound by moving the operands into the CUs, not by the matrix cores
// (timed without the matrix instructions it takes 95% as long, without the
// operand loads 60%): every token tile crosses L2 once per output tile and
// every W tile once per token tile, so the tile is as large as the registers
// allow (256 x 128 tiles: 2.78-2.92 ms; this tile 2.53-2.59 ms, on the L=32 /
// d=896 workload, all 65 reads).  Passing the fp32 results through LDS for
// 16-byte stores measured slower: one more barrier and round trip against
// 4-byte stores that already fill 128-byte lines per wave.
constexpr int kTileM = 256, kTileN = 256, kStageK = 32;
constexpr int kWavesM = 2, kWavesN = 4, kThreads = 64 * kWavesM * kWavesN;
// 32 x 32 fragments per wave along tokens and outputs
constexpr int kFa = kTileM / kWavesM / 32, kFb = kTileN / kWavesN / 32;
constexpr int kLdsRow = kStageK + 8;  // bf16 elements per LDS row (padded: staggers the banks)

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void query_proj_kernel(const bf16_t* x, const bf16_t* W, float* q, int64_t T, int d, int tiles_t,
                       int tiles_o, int64_t n_groups) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    auto lds_a = reinterpret_cast<bf16_t (*)[kTileM * kLdsRow]>(lds_raw);
    auto lds_b = reinterpret_cast<bf16_t (*)[kTileN * kLdsRow]>(lds_raw + 2 * kTileM * kLdsRow * sizeof(bf16_t));
    const int tid = threadIdx.x;
    const int wave = tid >> 6, ln = tid & 63;
    const int h = ln >> 5, m = ln & 31;
    const int wr = wave / kWavesN, wc = wave % kWavesN;
    // The tiles_o workgroups of one (read j, token tile) read the same token
    // rows, and the token tiles of one read share W_j: a group is numbered so
    // that its members run on one XCD, together, and consecutive groups on an
    // XCD take consecutive token tiles of the same read (numbered in XCD order
    // the members landed on different XCDs, each of whose L2 fetched the token
    // tile again: 8.9x the input bytes fetched).
    int64_t grp;
    int to;
    xcd_group(blockIdx.x, tiles_o, grp, to);
    if (grp >= n_groups) return;  // (the grid is rounded up to whole XCD rounds)
    const int tt = (int)(grp % tiles_t);
    const int64_t j = grp / tiles_t;
    const int64_t t0 = (int64_t)tt * kTileM;
    const int o0 = to * kTileN;
    const bf16_t* xj = x + j * T * d;
    const bf16_t* wj = W + j * (int64_t)d * d;

    // global -> LDS: thread tid moves the 16-byte chunks (row, kc) =
    // (idx / kCh, idx % kCh), idx = tid + kThreads c, of each operand tile
    constexpr int kCh = kStageK / 8;                 // 16-byte chunks per row
    constexpr int kPerA = kTileM * kCh / kThreads;   // chunks per thread of the token tile
    constexpr int kPerB = kTileN * kCh / kThreads;   // and of the W tile
    // Buffer loads over the tile's token rows and output rows: a chunk past T,
    // d or the last column loads zeros, without branches (a load inside a
    // branch makes every later wait drain all loads in flight).  Three register
    // slots: a stage's loads are issued two stages before its LDS store.
    const int n_tok = T - t0 < kTileM ? (int)(T - t0) : kTileM;
    const int n_out = d - o0 < kTileN ? d - o0 : kTileN;
    const rsrc_t ra_x = make_rsrc(xj + t0 * d, (uint64_t)n_tok * d * 2);
    const rsrc_t rb_w = make_rsrc(wj + (int64_t)o0 * d, (uint64_t)n_out * d * 2);
    u32x4 sa[3][kPerA], sb[3][kPerB];
    auto gload = [&](int slot, int k0) {
#pragma unroll
        for (int c = 0; c < kPerA; ++c) {
            const int idx = tid + kThreads * c;
            const int row = idx / kCh, kc = idx % kCh;
            const int k = k0 + 8 * kc;
            const uint32_t off = k < d ? (uint32_t)(row * d + k) * 2u : kOOB;
            sa[slot][c] = __builtin_amdgcn_raw_buffer_load_b128(ra_x, off, 0, 0);
            if (c < kPerB) sb[slot][c] = __builtin_amdgcn_raw_buffer_load_b128(rb_w, off, 0, 0);
        }
    };
    auto lstore = [&](int buf, int slot) {
#pragma unroll
        for (int c = 0; c < kPerA; ++c) {
            const int idx = tid + kThreads * c;
            const int row = idx / kCh, kc = idx % kCh;
            *reinterpret_cast<u32x4*>(&lds_a[buf][row * kLdsRow + 8 * kc]) = sa[slot][c];
            if (c < kPerB) *reinterpret_cast<u32x4*>(&lds_b[buf][row * kLdsRow + 8 * kc]) = sb[slot][c];
        }
    };

    f32x16 acc[kFa][kFb];
#pragma unroll
    for (int fa = 0; fa < kFa; ++fa)
#pragma unroll
        for (int fb = 0; fb < kFb; ++fb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fa][fb][r] = 0.f;

    const int n_stages = (d + kStageK - 1) / kStageK;
    // a wave whose output columns all lie past d (the last output tile when
    // d is not a multiple of the tile) only helps stage the operands
    const bool cols_live = o0 + (kTileN / kWavesN) * wc < d;
    gload(0, 0);
    gload(1, kStageK);  // past d: zeros, never stored
    gload(2, 2 * kStageK);
    lstore(0, 0);
    __syncthreads();
    // step st: slot st % 3 (stored already) takes stage st + 3's loads, the
    // MFMAs read buffer st % 2, then stage st + 1 goes from slot (st + 1) % 3
    // into the other buffer, last read before the previous barrier (unrolled
    // by 6 so that slots and buffers are compile-time registers and offsets)
    for (int st0 = 0; st0 < n_stages; st0 += 6) {
#pragma unroll
        for (int u = 0; u < 6; ++u) {
            const int st = st0 + u;
            if (st >= n_stages) break;
            gload(u % 3, (st + 3) * kStageK);
#pragma unroll
            for (int sub = 0; sub < kStageK / 16; ++sub) {
                if (!cols_live) break;  // (wave-uniform) this wave's outputs lie past d
                bf16x8_t fa_op[kFa], fb_op[kFb];
#pragma unroll
                for (int f = 0; f < kFa; ++f) {
                    const int ra = (kTileM / kWavesM) * wr + 32 * f + m;
                    fa_op[f] = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4*>(&lds_a[u % 2][ra * kLdsRow + 16 * sub + 8 * h]));
                }
#pragma unroll
                for (int f = 0; f < kFb; ++f) {
                    const int rb = (kTileN / kWavesN) * wc + 32 * f + m;
                    fb_op[f] = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4*>(&lds_b[u % 2][rb * kLdsRow + 16 * sub + 8 * h]));
                }
#pragma unroll
                for (int fa = 0; fa < kFa; ++fa)
#pragma unroll
                    for (int fb = 0; fb < kFb; ++fb)
                        acc[fa][fb] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_op[fa], fb_op[fb], acc[fa][fb], 0, 0, 0);
            }
            if (st + 1 < n_stages) {
                lstore((u + 1) % 2, (u + 1) % 3);
                __syncthreads();
            }
        }
    }
    // lane j, register r of fragment (fa, fb) holds token t0 + (kTileM / 2) wr +
    // 32 fa + i, output o0 + (kTileN / 2) wc + 32 fb + m, i = 8 (r / 4) + 4 h + r % 4
#pragma unroll
    for (int fa = 0; fa < kFa; ++fa)
#pragma unroll
        for (int fb = 0; fb < kFb; ++fb) {
            const int out = o0 + (kTileN / kWavesN) * wc + 32 * fb + m;
            if (out < d) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t ti = t0 + (kTileM / kWavesM) * wr + 32 * fa + 8 * (r / 4) + 4 * h + r % 4;
                    if (ti < T) q[(j * T + ti) * d + out] = acc[fa][fb][r];
                }
            }
        }
}

hipError_t launch_query_proj(const void* x, const void* W, float* q, int64_t n_q, int64_t T, int d,
                             hipStream_t stream) {
    const int tiles_t = (int)((T + kTileM - 1) / kTileM);
    const int tiles_o = (d + kTileN - 1) / kTileN;
    const int64_t n_groups = n_q * tiles_t;  // (read, token tile) pairs
    const int64_t blocks = (int64_t)kNumXcd * tiles_o * ((n_groups + kNumXcd - 1) / kNumXcd);
    constexpr size_t lds = (size_t)2 * (kTileM + kTileN) * kLdsRow * sizeof(bf16_t);
    const hipError_t e = prepare_dynamic_lds((const void*)query_proj_kernel, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(query_proj_kernel, dim3((unsigned)blocks), dim3(kThreads), lds, stream,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), q, T, d,
                       tiles_t, tiles_o, n_groups);
    return hipGetLastError();
}

}  // namespace attnres
