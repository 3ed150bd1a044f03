// codec.hip -- gfx950 kernels that write the KIVI cache: quantize-and-pack of
// key blocks and value tokens, and the fp16 residual-ring append.
//
// The arithmetic follows the KIVI explainer page ("ICML 2024論文解説: KIVI —
// チューニング不要のKVキャッシュ2bit非対称量子化"):
//   section 量子化アルゴリズム: Q(X) = clamp(round((X - z)/s), 0, 2^b - 1),
//     D(X^) = s X^ + z, s = (max - min)/(2^b - 1), z = min per group;
//   section Per-Channel量子化 / Per-Token量子化: keys per channel (over a block
//     of 32 tokens here), values per token (over 32-channel groups here);
//   section アルゴリズム: s floored at 1e-8, round then clamp;
//   section 残差バッファ: the newest tokens stay fp16 in the ring.
//
// The codec runs in IEEE fp32 (correctly rounded division, round-half-even,
// no contraction: the library is built with -ffp-contract=off), so its bytes
// are reproducible on any IEEE machine.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "codec_math.hpp"
#include "launch.hpp"

namespace kivi {
namespace {

constexpr int kG = 32;   // tokens per key block
constexpr int kVG = 32;  // channels per value group

// The fp16 rows are read once and the packed records written once: both go
// through the non-temporal (streaming) path (measured on MI355X: about 4%
// faster prefill than plain loads and stores).
typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u2 __attribute__((ext_vector_type(2)));
typedef float nt_f2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ codec

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

// Minimum and maximum of the 2N fp16 values held as N pairs (exact: the
// extremes of fp16 values are fp16 values; which zero a tie of +0 and -0
// returns never shows, since z = min + 0 drops the sign and a zero range
// floors s). The IEEE 754-2019 minimum / maximum (-0 below +0, NaN kept)
// need no canonicalised operands, and gfx950 folds two steps into one
// three-input v_pk_minimum3 / v_pk_maximum3: 16 instructions for 16 pairs
// where minNum / maxNum took 46 (each operand quieted by a v_pk_max first).
template <int N>
__device__ __forceinline__ void minmax_pairs(const uint32_t (&p)[N], float& mn, float& mx) {
    half2_t lo = as_h2(p[0]), hi = lo;
#pragma unroll
    for (int i = 1; i < N; ++i) {
        lo = __builtin_elementwise_minimum(lo, as_h2(p[i]));
        hi = __builtin_elementwise_maximum(hi, as_h2(p[i]));
    }
    mn = fminf((float)lo[0], (float)lo[1]);
    mx = fmaxf((float)hi[0], (float)hi[1]);
}

// Scale and zero of a group from its extremes (the correctly rounded quotient
// of IEEE division, no contraction), and the two terms of the fast code path
// below: p = x rf + cf, with rf = rcp(s) and cf = -z rf rounded once. When
// |cf| > 32 that sum is not close enough to (x - z) / s for the path's tie
// test, and the group takes rf = 0, cf = 1/2 instead: every p is then exactly
// a half-integer, so each word with such a code takes the division path. A
// group of one value (max = min, also +0 and -0) takes rf = cf = 0: its
// codes are 0, as (x - z) / s = 0 says.
template <int BITS>
__device__ __forceinline__ void group_stats(float mn, float mx, float& s, float& z, float& rf, float& cf) {
    constexpr float kQmax = float((1 << BITS) - 1);
    s = div_by_levels(mx - mn, kQmax, 1.0f / kQmax);
    if (!(s >= 1e-8f)) s = 1e-8f;
    z = mn + 0.0f;  // -0 -> +0
    const float rs = __builtin_amdgcn_rcpf(s);
    const float c = -z * rs;
    if (mx == mn) {
        rf = 0.0f;
        cf = 0.0f;
    } else if (fabsf(c) <= 32.0f) {
        rf = rs;
        cf = c;
    } else {
        rf = 0.0f;
        cf = 0.5f;
    }
}

// x - z for the fp16 half `hi` (0: bits 0..15, 1: bits 16..31) of `pair`,
// rounded once to fp32: v_fma_mix_f32 widens the half exactly (subnormals
// included) and computes x * 1 - z with one rounding, the correctly rounded
// difference.
template <int HI>
__device__ __forceinline__ float half_minus(uint32_t pair, float z) {
    float r;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(z));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(z));
    return r;
}

// x rf + cf for the fp16 half `hi` of `pair`, rounded once to fp32 (the half
// widened exactly).
template <int HI>
__device__ __forceinline__ float half_fma(uint32_t pair, float rf, float cf) {
    float r;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(rf), "v"(cf));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(pair), "v"(rf), "v"(cf));
    return r;
}

// One packed word of N codes: code i = clamp(rint((x_i - z_i) / s_i), 0, 2^b - 1)
// at bits [b i, b i + b). xp(i) gives a 32-bit word whose half (i & 1) is the
// fp16 value x_i, fr(i) the fast path's pair (cf_i, rf_i) and sz(i) the pair
// (s_i, z_i).
//
// The bytes are those of the IEEE steps (q = RN(RN(x - z) / s), then rint),
// computed faster: p = RN(x rf + cf) in one mixed-precision fma. With rf
// within 1 ulp of 1/s, cf within 2^-24 |cf| <= 2^-19 of -z rf, and codes up
// to 15.5, p differs from (x - z)/s by at most 15.5 2^-23 + 2^-19 + 2^-20,
// and q from (x - z)/s by at most 15.5 2^-23: |p - q| < 2^-17. So rint(p) =
// rint(q) unless p lies within 2^-17 of a half integer. |p - rint(p)| is
// exact and at most 1/2; when its largest value over the word exceeds
// 1/2 - 2^-15 in some lane (ties included), the wave redoes the word by true
// division.
// The clamp of the definition never binds on this path: (x - z)/s lies in
// [0, 2^b - 1], so p lies within 2^-17 of that range and rint(p) in it (a
// p just below 0 rounds to -0, code 0). The division path keeps the clamp.
// Codes accumulate exactly in fp32, 16 bits per accumulator.
template <int BITS, int N, class XP, class FR, class SZ>
__device__ __forceinline__ uint32_t pack_codes(XP xp, FR fr, SZ sz) {
    constexpr float kQmax = float((1 << BITS) - 1);
    constexpr int H = 16 / BITS;  // codes per accumulator
    static_assert(N == 2 * H, "a word is two 16-bit halves");
    float acc[2] = {0.0f, 0.0f};
    float dmax = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float2 q = fr(i);
        const float p = (i & 1) ? half_fma<1>(xp(i), q.y, q.x) : half_fma<0>(xp(i), q.y, q.x);
        const float r = __builtin_rintf(p);
        dmax = fmaxf(dmax, fabsf(p - r));
        acc[i / H] = __builtin_fmaf(r, (float)(1 << (BITS * (i % H))), acc[i / H]);
    }
    if (__builtin_amdgcn_ballot_w64(dmax > 0.5f - 0x1p-15f)) {
        acc[0] = acc[1] = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float2 w = sz(i);
            const float t = (i & 1) ? half_minus<1>(xp(i), w.y) : half_minus<0>(xp(i), w.y);
            const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(t / w.x), 0.0f, kQmax);
            acc[i / H] = __builtin_fmaf(r, (float)(1 << (BITS * (i % H))), acc[i / H]);
        }
    }
    return (uint32_t)acc[0] | (uint32_t)acc[1] << 16;
}

// 16-byte chunk `idx` of the ring copy of tokens [t0, t1) of unit u (chunk
// c16 of the key, then the value row, token by token) from input row
// (t - in_t0) of k / v into the token's ring slot. False past the end.
template <int D>
__device__ __forceinline__ bool copy_ring_chunk(const CacheGeom& g, const uint16_t* k, const uint16_t* v, int64_t ntok,
                                                int64_t u, int64_t t0, int64_t t1, int64_t in_t0, int64_t idx) {
    constexpr int CPR = D / 8;
    if (idx >= (t1 - t0) * 2 * CPR) return false;
    const int c16 = (int)(idx % CPR);
    const int kv = (int)((idx / CPR) & 1);
    const int64_t tok = t0 + idx / (2 * CPR);
    const int64_t row = u * ntok + (tok - in_t0);
    const uint4* src = reinterpret_cast<const uint4*>((kv ? v : k) + row * D) + c16;
    uint8_t* slot = g.base + g.off_ring + (size_t)u * g.ring_unit_stride + (size_t)(tok % g.ring_slots) * 4 * D +
                    (size_t)kv * 2 * D;
    reinterpret_cast<uint4*>(slot)[c16] = *src;
    return true;
}

// One work-group per (key block j, unit): 2*D threads (with a row table, block
// j0[row] + blockIdx.x of the unit's batch row, if below j1[row]). The block's
// 32 key and value rows are staged in LDS, then each thread plays two roles:
//   channel thread c (tid < D): the statistics of key channel c over the
//     block, then the packed value words of channel c (the block's 32 tokens,
//     channel-major);
//   token thread (t, g) (tid >= D): the statistics of value group g of token
//     t, then the packed key words of token t's channels [32g, 32g + 32)
//     (token-major).
// Each thread's codes are built from the other role's statistics, so one
// barrier separates the two halves, and every word is packed in registers.
// (Measured on MI355X: a persistent variant that loads the next block's rows
// into registers while coding the current one ran 10% slower: its registers
// left four work-groups per CU instead of seven.)
template <int D, int BITS>
__global__ __launch_bounds__(2 * D) void quantize_kernel(const QuantArgs a) {
    constexpr int NG = D / kVG;
    constexpr int PER = 32 / BITS;  // codes per word
    constexpr int NWG = kG / PER;   // words per 32 codes (= BITS)
    constexpr int NT = 2 * D;
    constexpr int CPR = D / 8;      // 16-byte chunks per fp16 row
    // staged rows, padded by 16 bytes so that the 32 rows start on different banks
    constexpr int DP = D + 8;
    __shared__ __align__(16) uint16_t sk[kG * DP];
    __shared__ __align__(16) uint16_t sv[kG * DP];
    // statistics for the codes: the fast path's key (cf, rf) of channel c at
    // kzr[c + 2 (c / 32)] (the 32-channel groups, read together by the lanes
    // of a wave, start on different banks), key (s, z) for the division path;
    // value (cf, rf) and (s, z) per group and token (rows padded apart for the
    // same reason)
    __shared__ __align__(16) float2 kzr[D + 2 * NG];
    __shared__ __align__(16) float2 ksz[D];
    __shared__ __align__(16) float2 vzr[NG][kG + 2];
    __shared__ __align__(16) float2 vsz[NG][kG];

    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int64_t u = blockIdx.y;
    // the ring copy's work-groups (rows that agree): 8 tokens each
    if (a.ring_wgs && (int64_t)blockIdx.x >= a.j1 - a.j0) {
        const int64_t idx = ((int64_t)blockIdx.x - (a.j1 - a.j0)) * NT + tid;
        copy_ring_chunk<D>(g, a.k, a.v, a.ntok, u, a.ring_t0, a.ring_t1, a.ring_in_t0, idx);
        return;  // the whole work-group
    }
    // this unit's blocks and ring boundary: its batch row's, when rows differ
    // (units, rows and a sequence's tokens all fit in 32 bits)
    const int brow = (int)((uint32_t)blockIdx.y / (uint32_t)g.n_kv_heads);
    const int64_t j = (a.rows.n ? a.rows.j0[brow] : a.j0) + blockIdx.x;
    if (a.rows.n && j >= a.rows.j1[brow]) return;  // the whole work-group
    const int64_t ring_end = a.rows.n ? a.rows.ring_end[brow] : a.ring_end;

    // ring slot of the block's first token (one division per work-group)
    const int64_t tok0 = j * kG;
    const int rs0 = (int)((uint32_t)tok0 % (uint32_t)g.ring_slots);
    const uint8_t* ring = g.base + g.off_ring + (size_t)u * g.ring_unit_stride;
    const uint16_t* kin = a.k + (u * a.ntok - ring_end) * D;  // input row of token tok: kin + tok * D
    const uint16_t* vin = a.v + (u * a.ntok - ring_end) * D;
#pragma unroll
    for (int it = 0; it < kG * CPR / NT; ++it) {
        const int idx = tid + it * NT;
        const int t = idx / CPR, c16 = idx % CPR;
        const int64_t tok = tok0 + t;
        const uint4 *kp, *vp;
        if (tok < ring_end) {
            int slot = rs0 + t;  // t < 32 <= ring slots: one wrap at most
            slot -= slot >= (int)g.ring_slots ? (int)g.ring_slots : 0;
            const uint8_t* row = ring + (size_t)slot * 4 * D;
            kp = reinterpret_cast<const uint4*>(row) + c16;
            vp = reinterpret_cast<const uint4*>(row + 2 * D) + c16;
        } else {
            kp = reinterpret_cast<const uint4*>(kin + tok * D) + c16;
            vp = reinterpret_cast<const uint4*>(vin + tok * D) + c16;
        }
        *reinterpret_cast<nt_u4*>(&sk[t * DP + c16 * 8]) = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(kp));
        *reinterpret_cast<nt_u4*>(&sv[t * DP + c16 * 8]) = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(vp));
    }
    __syncthreads();

    uint8_t* rec = g.base + record_offset(g, u, j);
    const bool chan = tid < D;
    const int c = tid;                    // channel thread
    const int tg = tid - D;               // token thread: token t, group gg
    const int t = tg / NG, gg = tg % NG;
    if (chan) {
        // key channel c over the 32 tokens (token i paired with token i + 16)
        uint32_t p[kG / 2];
        const _Float16* hk = reinterpret_cast<const _Float16*>(sk);
#pragma unroll
        for (int i = 0; i < kG / 2; ++i) {
            const half2_t x = {hk[i * DP + c], hk[(i + 16) * DP + c]};
            p[i] = __builtin_bit_cast(uint32_t, x);
        }
        float mn, mx, s, z, rf, cf;
        minmax_pairs(p, mn, mx);
        group_stats<BITS>(mn, mx, s, z, rf, cf);
        kzr[c + 2 * (c / kVG)] = make_float2(cf, rf);
        ksz[c] = make_float2(s, z);
        __builtin_nontemporal_store(nt_f2{s, z}, reinterpret_cast<nt_f2*>(rec + g.rec_ksz) + c);
    } else {
        // value group gg of token t: 32 contiguous channels
        uint32_t p[kVG / 2];
        const uint4* row = reinterpret_cast<const uint4*>(&sv[t * DP + gg * kVG]);
#pragma unroll
        for (int i = 0; i < kVG / 8; ++i) {
            const uint4 x = row[i];
            p[4 * i] = x.x;
            p[4 * i + 1] = x.y;
            p[4 * i + 2] = x.z;
            p[4 * i + 3] = x.w;
        }
        float mn, mx, s, z, rf, cf;
        minmax_pairs(p, mn, mx);
        group_stats<BITS>(mn, mx, s, z, rf, cf);
        vzr[gg][t] = make_float2(cf, rf);
        vsz[gg][t] = make_float2(s, z);
        __builtin_nontemporal_store(nt_f2{s, z}, reinterpret_cast<nt_f2*>(rec + g.rec_vsz) + tg);
    }
    __syncthreads();

    // Codes, packed as the record layout of kivi.h has them (code i of a word
    // at bits [BITS*i, BITS*i + BITS)):
    //   value words channel-major: word k of channel c holds tokens [k*PER, (k+1)*PER);
    //   key words token-major: word w of token t holds channels [w*PER, (w+1)*PER).
    uint32_t words[NWG];
    if (chan) {
        const int grp = c / kVG;
        const uint16_t* col = &sv[c];
#pragma unroll
        for (int k = 0; k < NWG; ++k)
            words[k] = pack_codes<BITS, PER>(
                [&](int i) { return (uint32_t)col[(k * PER + i) * DP] << (16 * (i & 1)); },
                [&](int i) { return vzr[grp][k * PER + i]; }, [&](int i) { return vsz[grp][k * PER + i]; });
    } else {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(&sk[t * DP + gg * kVG]);
#pragma unroll
        for (int k = 0; k < NWG; ++k) {
            const int c0 = gg * kVG + k * PER;
            words[k] = pack_codes<BITS, PER>([&](int i) { return row[(k * PER + i) / 2]; },
                                             [&](int i) { return kzr[c0 + i + 2 * gg]; },
                                             [&](int i) { return ksz[c0 + i]; });
        }
    }
    // channel c's BITS value words, or token t's BITS key words of group gg
    // (words gg*BITS .. gg*BITS + BITS - 1 of the token's row): both contiguous
    uint32_t* dst = reinterpret_cast<uint32_t*>(rec + (chan ? g.rec_vcode : g.rec_kcode)) + (chan ? c : tg) * NWG;
    if constexpr (NWG == 2) {
        __builtin_nontemporal_store(nt_u2{words[0], words[1]}, reinterpret_cast<nt_u2*>(dst));
    } else {
        __builtin_nontemporal_store(nt_u4{words[0], words[1], words[2], words[3]}, reinterpret_cast<nt_u4*>(dst));
    }
}

// Copy tokens [t0, t1) of every unit into their ring slots (with a row table,
// each batch row's own range): one thread per 16-byte chunk of a key or value
// row.
template <int D>
__global__ __launch_bounds__(256) void ring_write_kernel(const RingArgs a) {
    const CacheGeom& g = a.g;
    const int64_t u = blockIdx.y;
    const int64_t brow = u / g.n_kv_heads;
    const int64_t t0 = a.rows.n ? a.rows.t0[brow] : a.t0;
    const int64_t t1 = a.rows.n ? a.rows.t1[brow] : a.t1;
    const int64_t in_t0 = a.rows.n ? a.rows.in_t0[brow] : a.in_t0;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    copy_ring_chunk<D>(g, a.k, a.v, a.ntok, u, t0, t1, in_t0, idx);
}

template <int D>
hipError_t quantize_d(const QuantArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.j1 - a.j0 + a.ring_wgs), (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
    if (a.g.bits == 2)
        quantize_kernel<D, 2><<<grid, 2 * D, 0, s>>>(a);
    else
        quantize_kernel<D, 4><<<grid, 2 * D, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
    switch (a.g.head_dim) {
        case 64: return quantize_d<64>(a, s);
        case 128: return quantize_d<128>(a, s);
        default: return quantize_d<256>(a, s);
    }
}

hipError_t launch_ring_write(const RingArgs& a, hipStream_t s) {
    const int64_t n = (a.t1 - a.t0) * 2 * (a.g.head_dim / 8);
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
    switch (a.g.head_dim) {
        case 64: ring_write_kernel<64><<<grid, 256, 0, s>>>(a); break;
        case 128: ring_write_kernel<128><<<grid, 256, 0, s>>>(a); break;
        default: ring_write_kernel<256><<<grid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace kivi
