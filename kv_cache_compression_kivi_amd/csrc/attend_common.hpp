// attend_common.hpp -- device code shared by the two decode-attention kernels:
// attend_kernel (attend.hip: one or two query heads per work-group, or four at
// d != 128, on the vector units) and attend_gqa_kernel (attend_gqa.hip: four
// query heads at d = 128 on the matrix cores). Both read the same block
// records, run the fp16 residual on the vector units with the same lane
// layout, and append the call's new token to the ring the same way.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace kivi {

// Four query heads per work-group at d = 128 on the matrix cores (b from
// a.g.bits): writes the splits' partial results when a.n_split > 1 (merged by
// the caller) or the output rows when a.n_split == 1.
hipError_t launch_attend_gqa(const AttendArgs& a, hipStream_t s);

namespace {

constexpr int kG = 32;   // tokens per key block
constexpr int kVG = 32;  // channels per value group

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ------------------------------------------------------------ lane reductions

// Lane i reads the lane the DPP control names; a source outside the row reads 0.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

constexpr int kSwap1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kSwap2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kMirror = 0x140;      // row_mirror
constexpr int kHalfMirror = 0x141;  // row_half_mirror
constexpr int kRor4 = 0x124;        // row_ror:4
constexpr int kRor8 = 0x128;        // row_ror:8

// Sum over each aligned group of N (4, 8, 16) contiguous lanes, in every lane of the group.
template <int N>
__device__ __forceinline__ float sum_cols(float x) {
    x += dpp<kSwap1>(x);
    x += dpp<kSwap2>(x);
    if constexpr (N >= 8) x += dpp<kHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kMirror>(x);
    return x;
}

// Sum / max of lane i and lanes i +- 16, i +- 32 (the same lane of the four rows).
__device__ __forceinline__ float rows_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

__device__ __forceinline__ float rows_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// Sum / max over the lanes that share (lane mod NW): the token lanes of one column.
template <int NW>
__device__ __forceinline__ float tok_sum(float x) {
    if constexpr (NW == 4) {
        x += dpp<kRor4>(x);
        x += dpp<kRor8>(x);
    } else if constexpr (NW == 8) {
        x += dpp<kRor8>(x);
    }
    return rows_sum(x);
}

template <int NW>
__device__ __forceinline__ float tok_max(float x) {
    if constexpr (NW == 4) {
        x = fmaxf(x, dpp<kRor4>(x));
        x = fmaxf(x, dpp<kRor8>(x));
    } else if constexpr (NW == 8) {
        x = fmaxf(x, dpp<kRor8>(x));
    }
    return rows_max(x);
}

__device__ __forceinline__ float wave_sum(float x) { return rows_sum(sum_cols<16>(x)); }

// Orders this wave's LDS stores before its later LDS loads by other lanes
// (and the loads before later stores); LDS executes a wave's accesses in order.
__device__ __forceinline__ void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

typedef int v4i32 __attribute__((ext_vector_type(4)));

// Maxima of non-negative floats taken on their bit patterns, which order
// like unsigned integers (no NaN quieting, unlike fmaxf): over each row of 16
// lanes, and over the wave (every lane holds the result).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t row_max_bits(uint32_t x) {
    x = umax(x, dpp_u<kSwap1>(x));
    x = umax(x, dpp_u<kSwap2>(x));
    x = umax(x, dpp_u<kHalfMirror>(x));
    return umax(x, dpp_u<kMirror>(x));
}
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t x) {
    x = row_max_bits(x);
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = umax(r[0], r[1]);
    auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return umax(t[0], t[1]);
}

// The 23-bit integer Q = rint(a b 2^-e) (|a b| < 2^(22+e)) as three signed
// bytes, (Q + 0x808080) ^ 0x808080 in bits 0..23. One fma with the magic
// 1.5 2^(23+e) rounds the exact product to a multiple of 2^e (ties to even),
// so the low 24 bits of the result's encoding hold (e & 1) << 23 (the
// exponent's low bit, as 150 + e has the parity of e) above 2^22 + Q; the
// bias 0x408080 - ((e & 1) << 23) turns them into Q + 0x808080.
struct DigitScale {
    float magic;
    uint32_t bias;
};
// e must be the same in every lane. Both values stay whole scalars: folded
// into the adds of digits3, the bias would cost a second add per value.
__device__ __forceinline__ DigitScale digit_scale(int e) {
    const float magic = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(ldexpf(1.5f, 23 + e))));
    uint32_t bias = __builtin_amdgcn_readfirstlane(0x408080u - ((uint32_t)(e & 1) << 23));
    asm("" : "+s"(bias));  // opaque: not reassociated into the adds
    return {magic, bias};
}
__device__ __forceinline__ uint32_t digits3(float a, float b, DigitScale ds) {
    return (__float_as_uint(fmaf(a, b, ds.magic)) + ds.bias) ^ 0x808080u;
}

// ------------------------------------------------------------ block records

// Record layout of one key block (see kivi.h): kcode [G][W] (token-major),
// vcode [D][BITS] (channel-major: a channel's 32 tokens in BITS words),
// ksz [D][2], vsz [G][D/32][2]; known at compile time from D and BITS.
template <int D, int BITS>
struct Rec {
    static constexpr int W = D * BITS / 32;
    static constexpr int kcode = 0;
    static constexpr int vcode = kG * W * 4;
    static constexpr int ksz = 2 * kG * W * 4;
    static constexpr int vsz = ksz + D * 8;
    static constexpr int bytes = vsz + kG * (D / kVG) * 8;
};

// One lane's share of a block record, loaded ahead of its use. Key side:
// lane = tl * NW + w holds key-code words of tokens tl + TL*i, column w
// (channels [CW w, CW w + CW)). Value side: lane L holds the value codes of
// channels L*CPV .. L*CPV + CPV - 1, all 32 tokens (BITS words per channel).
template <int D, int BITS, int CW = 16>
struct BlockRegs {
    static_assert(CW == 16 || CW == 32, "a score column is 16 or 32 channels");
    static constexpr int NW = D / CW, TL = 64 / NW, TPL = kG / TL, NWORD = CW * BITS / 32, CPL = D / 64;
    static constexpr int CPV = D / 64;  // value channels per lane
    float ksz[2 * CPL];          // (s, z) of channels lane*CPL .. lane*CPL + CPL - 1
    uint32_t kc[TPL][NWORD];     // key code words of this lane's tokens and column
    uint32_t vc[CPV * BITS];     // value code words of this lane's channels
    float2 vsz[TPL];             // (s, z) of each token's value group that holds column w
};

// `bytes` of records from `base` as one buffer: a unit's records, or one
// paged block's record (offsets past `bytes` read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t records(const uint8_t* base, uint64_t bytes) {
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)n, 0x00020000);
}

// The low / high fp16 half of a 32-bit word, as a float.
__device__ __forceinline__ float half_lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t x) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16)); }

// Copies the token t_new appended by this call of unit u into its ring slot:
// 16 bytes per lane, key row then value row (one wave).
template <int D>
__device__ __forceinline__ void write_new_token(const AttendArgs& a, int64_t u, int64_t t_new, const uint8_t* rbase) {
    constexpr int CH = D / 8;  // 16-byte chunks per fp16 row
    const int lane = threadIdx.x & 63;
    const int slot = (int)(t_new % a.g.ring_slots);
    for (int i = lane; i < 2 * CH; i += 64) {
        const int kv = i / CH, c = i % CH;
        const uint4 x = reinterpret_cast<const uint4*>((kv ? a.v_new : a.k_new) + u * D)[c];
        reinterpret_cast<uint4*>(const_cast<uint8_t*>(rbase) + (size_t)slot * 4 * D + (size_t)kv * 2 * D)[c] = x;
    }
}

}  // namespace
}  // namespace kivi
