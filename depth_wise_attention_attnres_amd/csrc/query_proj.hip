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

// Workgroup tile: 128 tokens x 128 outputs; wave (wr, wc) of the 2 x 2 waves
// computes 64 x 64 as 2 x 2 fragments of 32 x 32, so each operand fragment
// read from LDS feeds two matrix instructions.  K goes in stages of 64
// elements through double-buffered LDS: the workgroup loads a stage's 128
// token rows and 128 W rows (contiguous in k, 16 bytes per lane) three stages
// ahead of its multiplication; one barrier per stage.  (Passing the fp32 results
// through LDS for 16-byte stores measured slower: one more barrier and round
// trip against 4-byte stores that already fill 128-byte lines per wave.)
constexpr int kTileM = 128, kTileN = 128, kStageK = 64;
constexpr int kLdsRow = kStageK + 8;  // bf16 elements per LDS row (padded: staggers the banks)

__global__ __launch_bounds__(256) void query_proj_kernel(const bf16_t* x, const bf16_t* W, float* q,
                                                         int64_t T, int d, int tiles_t, int tiles_o) {
    __shared__ __attribute__((aligned(16))) bf16_t lds_a[2][kTileM * kLdsRow];
    __shared__ __attribute__((aligned(16))) bf16_t lds_b[2][kTileN * kLdsRow];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, ln = tid & 63;
    const int h = ln >> 5, m = ln & 31;
    const int wr = wave >> 1, wc = wave & 1;
    // blockIdx.x = (read j, token tile, output tile), output tiles fastest so
    // that the workgroups sharing a token tile run together and reuse it in L2
    const int64_t blk = blockIdx.x;
    const int to = (int)(blk % tiles_o);
    const int64_t rest = blk / tiles_o;
    const int tt = (int)(rest % tiles_t);
    const int64_t j = rest / tiles_t;
    const int64_t t0 = (int64_t)tt * kTileM;
    const int o0 = to * kTileN;
    const bf16_t* xj = x + j * T * d;
    const bf16_t* wj = W + j * (int64_t)d * d;

    // global -> LDS: thread tid moves the 16-byte chunks (row, kc) =
    // (idx / kCh, idx % kCh), idx = tid + 256 c, of each operand tile
    constexpr int kCh = kStageK / 8;                 // 16-byte chunks per row
    constexpr int kPer = kTileM * kCh / 256;         // chunks per thread and operand
    // Buffer loads over the tile's token rows and output rows: a chunk past T,
    // d or the last column loads zeros, without branches (a load inside a
    // branch makes every later wait drain all loads in flight).  Three register
    // slots: a stage's loads are issued two stages before its LDS store.
    const int n_tok = T - t0 < kTileM ? (int)(T - t0) : kTileM;
    const int n_out = d - o0 < kTileN ? d - o0 : kTileN;
    const rsrc_t ra_x = make_rsrc(xj + t0 * d, (uint64_t)n_tok * d * 2);
    const rsrc_t rb_w = make_rsrc(wj + (int64_t)o0 * d, (uint64_t)n_out * d * 2);
    u32x4 sa[3][kPer], sb[3][kPer];
    auto gload = [&](int slot, int k0) {
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const int idx = tid + 256 * c;
            const int row = idx / kCh, kc = idx % kCh;
            const int k = k0 + 8 * kc;
            const uint32_t off = k < d ? (uint32_t)(row * d + k) * 2u : kOOB;
            sa[slot][c] = __builtin_amdgcn_raw_buffer_load_b128(ra_x, off, 0, 0);
            sb[slot][c] = __builtin_amdgcn_raw_buffer_load_b128(rb_w, off, 0, 0);
        }
    };
    auto lstore = [&](int buf, int slot) {
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const int idx = tid + 256 * c;
            const int row = idx / kCh, kc = idx % kCh;
            *reinterpret_cast<u32x4*>(&lds_a[buf][row * kLdsRow + 8 * kc]) = sa[slot][c];
            *reinterpret_cast<u32x4*>(&lds_b[buf][row * kLdsRow + 8 * kc]) = sb[slot][c];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int fa = 0; fa < 2; ++fa)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fa][fb][r] = 0.f;

    const int n_stages = (d + kStageK - 1) / kStageK;
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
                bf16x8_t fa_op[2], fb_op[2];
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const int ra = 64 * wr + 32 * f + m, rb = 64 * wc + 32 * f + m;
                    fa_op[f] = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4*>(&lds_a[u % 2][ra * kLdsRow + 16 * sub + 8 * h]));
                    fb_op[f] = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4*>(&lds_b[u % 2][rb * kLdsRow + 16 * sub + 8 * h]));
                }
#pragma unroll
                for (int fa = 0; fa < 2; ++fa)
#pragma unroll
                    for (int fb = 0; fb < 2; ++fb)
                        acc[fa][fb] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_op[fa], fb_op[fb], acc[fa][fb], 0, 0, 0);
            }
            if (st + 1 < n_stages) {
                lstore((u + 1) % 2, (u + 1) % 3);
                __syncthreads();
            }
        }
    }
    // lane j, register r of fragment (fa, fb) holds token t0 + 64 wr + 32 fa + i,
    // output o0 + 64 wc + 32 fb + m, with i = 8 (r / 4) + 4 h + r % 4
#pragma unroll
    for (int fa = 0; fa < 2; ++fa)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
            const int out = o0 + 64 * wc + 32 * fb + m;
            if (out < d) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t ti = t0 + 64 * wr + 32 * fa + 8 * (r / 4) + 4 * h + r % 4;
                    if (ti < T) q[(j * T + ti) * d + out] = acc[fa][fb][r];
                }
            }
        }
}

hipError_t launch_query_proj(const void* x, const void* W, float* q, int64_t n_q, int64_t T, int d,
                             hipStream_t stream) {
    const int tiles_t = (int)((T + kTileM - 1) / kTileM);
    const int tiles_o = (d + kTileN - 1) / kTileN;
    const int64_t blocks = n_q * tiles_t * (int64_t)tiles_o;
    hipLaunchKernelGGL(query_proj_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(W), q, T, d,
                       tiles_t, tiles_o);
    return hipGetLastError();
}

}  // namespace attnres
