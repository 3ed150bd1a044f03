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

#include "launch.hpp"

namespace kivi {
namespace {

constexpr int kG = 32;   // tokens per key block
constexpr int kVG = 32;  // channels per value group

// The fp16 rows are read once and the packed records written once: both go
// through the non-temporal (streaming) path (measured on MI355X: about 4%
// faster prefill than plain loads and stores).
typedef unsigned int nt_u4 __attribute__((ext_vector_type(4)));
typedef float nt_f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

// ------------------------------------------------------------------ codec

// One group of N values -> (s, z) and its codes.
//
// The bytes are those of the IEEE steps (s = (max - min) / (2^b - 1) by true
// division, code = rint((x - z) / s)), computed faster:
//   - min and max with v_min / v_max: which zero (+0 or -0) they return never
//     shows, since z = min + 0 drops the sign and a zero range clamps s;
//   - q' = (x - z) * rcp(s), where rcp is within 1 ulp of 1/s, differs from the
//     IEEE quotient q by at most (2^-23 + 2^-24) * 15.5 + 2^-20 < 2^-18 (codes
//     <= 15), so rint(q') = rint(q) unless q' lies within 2^-18 of a half
//     integer; within 2^-15 of one (ties included) the true division decides.
template <int N, int BITS>
__device__ __forceinline__ void quant_group(const float (&x)[N], float& s, float& z, uint8_t (&out)[N]) {
    constexpr float kQmax = float((1 << BITS) - 1);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    s = (mx - mn) / kQmax;
    if (!(s >= 1e-8f)) s = 1e-8f;
    z = mn + 0.0f;  // -0 -> +0
    const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float t = x[i] - z;
        float r = __builtin_rintf(t * rs);
        if (fabsf(fabsf(t * rs - r) - 0.5f) < 0x1p-15f) r = __builtin_rintf(t / s);
        r = r < 0.0f ? 0.0f : r;
        r = r > kQmax ? kQmax : r;
        out[i] = (uint8_t)r;
    }
}

// One work-group per (key block j, unit): 2*D threads (with a row table, block
// j0[row] + blockIdx.x of the unit's batch row, if below j1[row]). Threads [0, D) take
// one key channel each over the block's 32 tokens; threads [D, 2D) take one
// (token, 32-channel value group) each. Then all threads pack words.
template <int D, int BITS>
__global__ __launch_bounds__(2 * D) void quantize_kernel(const QuantArgs a) {
    constexpr int NG = D / kVG;
    constexpr int W = D * BITS / 32;
    constexpr int PER = 32 / BITS;
    constexpr int NT = 2 * D;
    constexpr int CPR = D / 8;  // 16-byte chunks per fp16 row
    // fp16 rows of the block; once read, the same memory holds the codes (bytes)
    __shared__ __align__(16) uint16_t sk[kG * D];
    __shared__ __align__(16) uint16_t sv[kG * D];
    uint8_t* const ck = reinterpret_cast<uint8_t*>(sk);
    uint8_t* const cv = reinterpret_cast<uint8_t*>(sv);

    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int64_t u = blockIdx.y;
    // this unit's blocks and ring boundary: its batch row's, when rows differ
    const int64_t brow = u / g.n_kv_heads;
    const int64_t j = (a.rows.n ? a.rows.j0[brow] : a.j0) + blockIdx.x;
    if (a.rows.n && j >= a.rows.j1[brow]) return;  // the whole work-group
    const int64_t ring_end = a.rows.n ? a.rows.ring_end[brow] : a.ring_end;

    for (int idx = tid; idx < kG * CPR; idx += NT) {
        const int t = idx / CPR, c16 = idx % CPR;
        const int64_t tok = j * kG + t;
        const uint4 *ks, *vs;
        if (tok < ring_end) {
            const uint8_t* slot = g.base + g.off_ring + (size_t)u * g.ring_unit_stride +
                                  (size_t)(tok % g.ring_slots) * 4 * D;
            ks = reinterpret_cast<const uint4*>(slot) + c16;
            vs = reinterpret_cast<const uint4*>(slot + 2 * D) + c16;
        } else {
            const int64_t row = u * a.ntok + (tok - ring_end);
            ks = reinterpret_cast<const uint4*>(a.k + row * D) + c16;
            vs = reinterpret_cast<const uint4*>(a.v + row * D) + c16;
        }
        reinterpret_cast<nt_u4*>(sk)[idx] = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(ks));
        reinterpret_cast<nt_u4*>(sv)[idx] = __builtin_nontemporal_load(reinterpret_cast<const nt_u4*>(vs));
    }
    __syncthreads();

    uint8_t* rec = g.base + record_offset(g, u, j);
    uint8_t codes[kG];  // kG == kVG
    if (tid < D) {
        const int c = tid;
        float x[kG];
#pragma unroll
        for (int t = 0; t < kG; ++t) x[t] = half_bits_to_float(sk[t * D + c]);
        float s, z;
        quant_group<kG, BITS>(x, s, z, codes);
        __builtin_nontemporal_store(nt_f2{s, z}, reinterpret_cast<nt_f2*>(rec + g.rec_ksz) + c);
    } else {
        const int idx = tid - D;
        const int t = idx / NG, grp = idx % NG;
        float x[kVG];
#pragma unroll
        for (int i = 0; i < kVG; ++i) x[i] = half_bits_to_float(sv[t * D + grp * kVG + i]);
        float s, z;
        quant_group<kVG, BITS>(x, s, z, codes);
        __builtin_nontemporal_store(nt_f2{s, z}, reinterpret_cast<nt_f2*>(rec + g.rec_vsz) + t * NG + grp);
    }
    __syncthreads();  // every thread is done reading the fp16 rows
    if (tid < D) {
#pragma unroll
        for (int t = 0; t < kG; ++t) ck[t * D + tid] = codes[t];
    } else {
        const int idx = tid - D;
        const int t = idx / NG, grp = idx % NG;
#pragma unroll
        for (int i = 0; i < kVG; i += 4)
            *reinterpret_cast<uint32_t*>(&cv[t * D + grp * kVG + i]) =
                (uint32_t)codes[i] | (uint32_t)codes[i + 1] << 8 | (uint32_t)codes[i + 2] << 16 |
                (uint32_t)codes[i + 3] << 24;
    }
    __syncthreads();

    // Pack (the record layout of kivi.h), code i of a word at bits [BITS*i, BITS*i + BITS):
    //   key words token-major, word w of token t holds channels [w*PER, (w+1)*PER);
    //   value words channel-major, word k of channel c holds tokens [k*PER, (k+1)*PER).
    uint32_t* kw = reinterpret_cast<uint32_t*>(rec + g.rec_kcode);
    uint32_t* vw = reinterpret_cast<uint32_t*>(rec + g.rec_vcode);
    for (int idx = tid; idx < 2 * kG * W; idx += NT) {
        uint32_t word = 0;
        if (idx < kG * W) {
            const int t = idx / W, w = idx % W;
            const uint8_t* cs = ck + t * D + w * PER;
#pragma unroll
            for (int i = 0; i < PER; ++i) word |= (uint32_t)cs[i] << (BITS * i);
            __builtin_nontemporal_store(word, kw + idx);
        } else {
            const int x = idx - kG * W;  // x = c * BITS + k
            const int c = x / BITS, k = x % BITS;
            const uint8_t* cs = cv + (k * PER) * D + c;
#pragma unroll
            for (int i = 0; i < PER; ++i) word |= (uint32_t)cs[i * D] << (BITS * i);
            __builtin_nontemporal_store(word, vw + x);
        }
    }
}

// Copy tokens [t0, t1) of every unit into their ring slots (with a row table,
// each batch row's own range): one thread per 16-byte chunk of a key or value
// row.
template <int D>
__global__ __launch_bounds__(256) void ring_write_kernel(const RingArgs a) {
    constexpr int CPR = D / 8;
    const CacheGeom& g = a.g;
    const int64_t u = blockIdx.y;
    const int64_t brow = u / g.n_kv_heads;
    const int64_t t0 = a.rows.n ? a.rows.t0[brow] : a.t0;
    const int64_t t1 = a.rows.n ? a.rows.t1[brow] : a.t1;
    const int64_t in_t0 = a.rows.n ? a.rows.in_t0[brow] : a.in_t0;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (t1 - t0) * 2 * CPR;
    if (idx >= n) return;
    const int c16 = (int)(idx % CPR);
    const int kv = (int)((idx / CPR) & 1);
    const int64_t tok = t0 + idx / (2 * CPR);
    const int64_t row = u * a.ntok + (tok - in_t0);
    const uint4* src = reinterpret_cast<const uint4*>((kv ? a.v : a.k) + row * D) + c16;
    uint8_t* slot = g.base + g.off_ring + (size_t)u * g.ring_unit_stride +
                    (size_t)(tok % g.ring_slots) * 4 * D + (size_t)kv * 2 * D;
    reinterpret_cast<uint4*>(slot)[c16] = *src;
}

template <int D>
hipError_t quantize_d(const QuantArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.j1 - a.j0), (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads));
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
