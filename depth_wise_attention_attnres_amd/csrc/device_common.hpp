// device_common.hpp -- gfx950 device helpers shared by the AttnRes kernels.
//
// Data movement is in 16-byte chunks of 8 elements along d: a bf16 chunk is
// one dwordx4 load, an fp32 chunk two.  A "token group" (TG) of LPT lanes
// (LPT in {16, 32, 64}) owns one token; lane `ln` of the group owns chunks
// ln, ln + LPT, ln + 2 LPT, ... so that one load instruction of the group
// touches LPT * 16 contiguous bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// element types

struct bf16_t {
    uint16_t bits;
};

// native clang vectors (the nontemporal builtins need them)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// buffer addressing.  Every row access goes through a buffer resource whose
// base is wave-uniform (SGPRs) and whose range check turns out-of-range lanes
// into zero loads and dropped stores: a lane whose chunk lies past d, or whose
// token lies past T, is given the offset kOOB.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x40000000u;   // >= every num_records we build
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9-family raw buffer, 32-bit data
constexpr int kAuxNT = 2;                // non-temporal cache policy

// Read-only view of memory that a kernel never writes.  Loads through the
// constant address space with a wave-uniform address become scalar loads,
// which are counted apart from the vector loads, so waiting for them does
// not drain the vector loads in flight.
typedef const __attribute__((address_space(4))) float* cf32_ptr;
__device__ __forceinline__ cf32_ptr const_view(const float* p) { return (cf32_ptr)p; }

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes < kOOB ? (uint32_t)bytes : kOOB;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n,
                                             (int)kRsrcWord3);
}

// 8 elements of a history / gradient row
template <typename T> struct Chunk;

template <> struct Chunk<bf16_t> {
    u32x4 v;  // 8 bf16, little-endian pairs
    __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
    template <int AUX = 0>
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    }
    __device__ __forceinline__ void to_float(float (&f)[8]) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
        }
    }
};

template <> struct Chunk<float> {
    u32x4 a, b;
    __device__ __forceinline__ void zero() {
        a = u32x4{0u, 0u, 0u, 0u};
        b = a;
    }
    template <int AUX = 0>
    __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
        a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
        b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, AUX);
    }
    __device__ __forceinline__ void to_float(float (&f)[8]) const {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[q] = __uint_as_float(a[q]);
            f[4 + q] = __uint_as_float(b[q]);
        }
    }
};

// round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float float2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    float2_v f = {lo, hi};
    bf16x2_v b = __builtin_convertvector(f, bf16x2_v);
    return __builtin_bit_cast(uint32_t, b);
}

template <int AUX = 0>
__device__ __forceinline__ void store_chunk(bf16_t*, rsrc_t r, uint32_t off, const float (&f)[8]) {
    u32x4 v = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, AUX);
}

template <int AUX = 0>
__device__ __forceinline__ void store_chunk(float*, rsrc_t r, uint32_t off, const float (&f)[8]) {
    u32x4 a = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
               __float_as_uint(f[3])};
    u32x4 b = {__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
               __float_as_uint(f[7])};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, off, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, off + 16, 0, AUX);
}

__device__ __forceinline__ float load_f32(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void store_f32(rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// cross-lane sums inside a token group of LPT lanes (all lanes get the sum).
// Within a 16-lane row: DPP butterflies (xor 1, xor 2, half-row mirror, row
// mirror); across rows: the gfx950 row-swap permutes.

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

// sum over lanes l and l ^ 16 (rows 0<->1, 2<->3)
__device__ __forceinline__ float swap16_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// sum over lanes l and l ^ 32 (upper and lower half of the wave)
__device__ __forceinline__ float swap32_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int LPT>
__device__ __forceinline__ float tg_sum(float v) {
    static_assert(LPT == 16 || LPT == 32 || LPT == 64, "token group of 16, 32 or 64 lanes");
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    if constexpr (LPT >= 32) v = swap16_sum(v);
    if constexpr (LPT >= 64) v = swap32_sum(v);
    return v;
}

// max over a token group of LPT lanes (every lane gets the max)
__device__ __forceinline__ float swap16_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int LPT>
__device__ __forceinline__ float tg_max(float v) {
    static_assert(LPT == 16 || LPT == 32 || LPT == 64, "token group of 16, 32 or 64 lanes");
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    if constexpr (LPT >= 32) v = swap16_max(v);
    if constexpr (LPT >= 64) v = swap32_max(v);
    return v;
}

// ---------------------------------------------------------------------------
// sums over the wave of several values at once.  A transposing step over lane
// bit B (DPP control CTRL pairs lane i with lane i ^ (1 << B)): of each pair
// of values (v[2j], v[2j+1]) a lane keeps the one its bit selects and sends
// the other, so N values become N / 2, each summed over both lanes -- three
// operations per pair where plain butterflies take one per value and level.

constexpr int kDppRor8 = 0x128;  // row_ror:8 (lanes i and i ^ 8 of a 16-lane row)
constexpr int kDppShr4 = 0x114;  // row_shr:4 (lane i takes lane i - 4 of its row)

template <int CTRL, int B, int N>
__device__ __forceinline__ void transpose_step(const float (&v)[N], float (&o)[N / 2], int lane) {
    const bool hi = (lane >> B) & 1;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float keep = hi ? v[2 * j + 1] : v[2 * j];
        const float send = hi ? v[2 * j] : v[2 * j + 1];
        o[j] = keep + dpp<CTRL>(send);
    }
}

// Wave sums of P in {4, 8} values: value k ends in lane bits 0, 1 (and 3 when
// P = 8) equal to k; its total is complete in the lanes with bit 2 set and
// bits 4, 5 (and 3 when P = 4) clear: lanes 4..7 (and 12..15).
template <int P>
__device__ __forceinline__ bool wave_sum_holder(int lane) {
    return (lane & (P == 8 ? 0x34 : 0x3C)) == 0x04;
}
template <int P>
__device__ __forceinline__ int wave_sum_index(int lane) {
    return P == 8 ? (lane & 3) | (((lane >> 3) & 1) << 2) : (lane & 3);
}
template <int P>
__device__ __forceinline__ float wave_sum_transposed(const float (&v)[P], int lane) {
    static_assert(P == 4 || P == 8, "4 or 8 values");
    float v2[P / 2], v1[P / 4];
    transpose_step<kDppXor1, 0, P>(v, v2, lane);
    transpose_step<kDppXor2, 1, P / 2>(v2, v1, lane);
    float x;
    if constexpr (P == 8) {
        float v0[1];
        transpose_step<kDppRor8, 3, 2>(v1, v0, lane);
        x = v0[0];
    } else {
        x = v1[0];
        x += dpp<kDppRor8>(x);  // lanes i and i ^ 8
    }
    x += dpp<kDppShr4>(x);  // lane i takes i - 4: complete where bit 2 is set
    x = swap16_sum(x);
    x = swap32_sum(x);
    return x;
}

// Wave totals of KV values, as wave-uniform scalars: groups of up to 8 values
// share one transposing reduction; value k of a group is read from the lane
// that holds it (wave_sum_holder / wave_sum_index above).
template <int P>
__device__ __forceinline__ int holder_lane(int k) {
    return P == 8 ? (k & 3) | 4 | ((k >> 2) << 3) : 4 + k;
}
template <int BASE, int KV>
__device__ __forceinline__ void wave_totals(const float (&v)[KV], float (&tot)[KV], int lane) {
    constexpr int REM = KV - BASE;
    constexpr int P = REM > 4 ? 8 : 4;
    float g[P];
#pragma unroll
    for (int j = 0; j < P; ++j) g[j] = BASE + j < KV ? v[BASE + j < KV ? BASE + j : 0] : 0.f;
    const float t = wave_sum_transposed<P>(g, lane);
#pragma unroll
    for (int j = 0; j < P; ++j)
        if (BASE + j < KV)
            tot[BASE + j < KV ? BASE + j : 0] =
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), holder_lane<P>(j)));
    if constexpr (REM > 8) wave_totals<BASE + 8, KV>(v, tot, lane);
}

// XCD-aware workgroup numbering.  The dispatcher hands workgroups to the
// eight XCDs in turn (workgroup w runs on XCD w % 8), and each XCD has its own
// L2.  For work split into groups of `members` workgroups that read the same
// data, number the groups so that all members of a group share an XCD:
// group = 8 (w / (8 members)) + w % 8, member = (w / 8) % members.  A grid of
// 8 members ceil(groups / 8) workgroups covers every group; members of groups
// past the last one return.
constexpr int kNumXcd = 8;
__device__ __forceinline__ void xcd_group(int64_t w, int members, int64_t& group, int& member) {
    const int64_t q = w / kNumXcd;
    member = (int)(q % members);
    group = (q / members) * kNumXcd + w % kNumXcd;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

}  // namespace attnres
