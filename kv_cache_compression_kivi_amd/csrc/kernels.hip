// kernels.hip -- gfx950 kernels of the KIVI cache: quantize-and-pack, ring
// append, split-K decode attention over packed codes plus the fp16 residual,
// and the log-sum-exp combine.
//
// The arithmetic follows the KIVI explainer page ("ICML 2024論文解説: KIVI —
// チューニング不要のKVキャッシュ2bit非対称量子化"):
//   section 量子化アルゴリズム: Q(X) = clamp(round((X - z)/s), 0, 2^b - 1),
//     D(X^) = s X^ + z, s = (max - min)/(2^b - 1), z = min per group;
//   section Per-Channel量子化 / Per-Token量子化: keys per channel (over a block
//     of 32 tokens here), values per token (over 32-channel groups here);
//   section アルゴリズム: s floored at 1e-8, round then clamp;
//   section 残差バッファ: attention is one softmax over the dequantized part
//     and the fp16 residual, scaled by 1/sqrt(d).
//
// The codec runs in IEEE fp32 (correctly rounded division, round-half-even,
// no contraction: the library is built with -ffp-contract=off), so its bytes
// are reproducible on any IEEE machine. Attention runs in fp32.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

#include "launch.hpp"

namespace kivi {
namespace {

constexpr int kG = 32;   // tokens per key block
constexpr int kVG = 32;  // channels per value group

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// ------------------------------------------------------------------ codec

// One group of N values -> (s, z) and codes written to out[i * stride].
template <int N, int BITS>
__device__ __forceinline__ void quant_group(const float (&x)[N], float& s, float& z, uint8_t* out,
                                            int stride) {
    constexpr float kQmax = float((1 << BITS) - 1);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) {
        mn = x[i] < mn ? x[i] : mn;
        mx = x[i] > mx ? x[i] : mx;
    }
    s = (mx - mn) / kQmax;
    if (!(s >= 1e-8f)) s = 1e-8f;
    z = mn + 0.0f;  // -0 -> +0
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float r = __builtin_rintf((x[i] - z) / s);
        r = r < 0.0f ? 0.0f : r;
        r = r > kQmax ? kQmax : r;
        out[i * stride] = (uint8_t)r;
    }
}

// One work-group per (key block j, unit): 2*D threads. Threads [0, D) take
// one key channel each over the block's 32 tokens; threads [D, 2D) take one
// (token, 32-channel value group) each. Then all threads pack words.
template <int D, int BITS>
__global__ __launch_bounds__(2 * D) void quantize_kernel(const QuantArgs a) {
    constexpr int NG = D / kVG;
    constexpr int W = D * BITS / 32;
    constexpr int PER = 32 / BITS;
    constexpr int NT = 2 * D;
    constexpr int CPR = D / 8;  // 16-byte chunks per fp16 row
    __shared__ __align__(16) uint16_t sk[kG * D];
    __shared__ __align__(16) uint16_t sv[kG * D];
    __shared__ __align__(16) uint8_t ck[kG * D];
    __shared__ __align__(16) uint8_t cv[kG * D];

    const CacheGeom& g = a.g;
    const int tid = threadIdx.x;
    const int64_t j = a.j0 + blockIdx.x;
    const int64_t u = blockIdx.y;

    for (int idx = tid; idx < kG * CPR; idx += NT) {
        const int t = idx / CPR, c16 = idx % CPR;
        const int64_t tok = j * kG + t;
        const uint4 *ks, *vs;
        if (tok < a.ring_end) {
            const uint8_t* slot = g.base + g.off_ring + (size_t)u * g.ring_unit_stride +
                                  (size_t)(tok % g.ring_slots) * 4 * D;
            ks = reinterpret_cast<const uint4*>(slot) + c16;
            vs = reinterpret_cast<const uint4*>(slot + 2 * D) + c16;
        } else {
            const int64_t row = u * a.ntok + (tok - a.ring_end);
            ks = reinterpret_cast<const uint4*>(a.k + row * D) + c16;
            vs = reinterpret_cast<const uint4*>(a.v + row * D) + c16;
        }
        reinterpret_cast<uint4*>(sk)[idx] = *ks;
        reinterpret_cast<uint4*>(sv)[idx] = *vs;
    }
    __syncthreads();

    uint8_t* rec = g.base + g.off_blocks + (size_t)u * g.unit_stride + (size_t)j * g.block_bytes;
    if (tid < D) {
        const int c = tid;
        float x[kG];
#pragma unroll
        for (int t = 0; t < kG; ++t) x[t] = half_bits_to_float(sk[t * D + c]);
        float s, z;
        quant_group<kG, BITS>(x, s, z, &ck[c], D);
        reinterpret_cast<float2*>(rec + g.rec_ksz)[c] = make_float2(s, z);
    } else {
        const int idx = tid - D;
        const int t = idx / NG, grp = idx % NG;
        float x[kVG];
#pragma unroll
        for (int i = 0; i < kVG; ++i) x[i] = half_bits_to_float(sv[t * D + grp * kVG + i]);
        float s, z;
        quant_group<kVG, BITS>(x, s, z, &cv[t * D + grp * kVG], 1);
        reinterpret_cast<float2*>(rec + g.rec_vsz)[t * NG + grp] = make_float2(s, z);
    }
    __syncthreads();

    uint32_t* kw = reinterpret_cast<uint32_t*>(rec + g.rec_kcode);
    uint32_t* vw = reinterpret_cast<uint32_t*>(rec + g.rec_vcode);
    for (int idx = tid; idx < 2 * kG * W; idx += NT) {
        const bool isv = idx >= kG * W;
        const int r = isv ? idx - kG * W : idx;  // r = t * W + w
        const int t = r / W, w = r % W;
        const uint8_t* cs = (isv ? cv : ck) + t * D + w * PER;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) word |= (uint32_t)cs[i] << (BITS * i);
        (isv ? vw : kw)[r] = word;
    }
}

// Copy tokens [t0, t1) of every unit into their ring slots: one thread per
// 16-byte chunk of a key or value row.
template <int D>
__global__ __launch_bounds__(256) void ring_write_kernel(const RingArgs a) {
    constexpr int CPR = D / 8;
    const CacheGeom& g = a.g;
    const int64_t u = blockIdx.y;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (a.t1 - a.t0) * 2 * CPR;
    if (idx >= n) return;
    const int c16 = (int)(idx % CPR);
    const int kv = (int)((idx / CPR) & 1);
    const int64_t tok = a.t0 + idx / (2 * CPR);
    const int64_t row = u * a.ntok + (tok - a.in_t0);
    const uint4* src = reinterpret_cast<const uint4*>((kv ? a.v : a.k) + row * D) + c16;
    uint8_t* slot = g.base + g.off_ring + (size_t)u * g.ring_unit_stride +
                    (size_t)(tok % g.ring_slots) * 4 * D + (size_t)kv * 2 * D;
    reinterpret_cast<uint4*>(slot)[c16] = *src;
}

// ------------------------------------------------------------------ attention

// Lane sums over aligned groups of N contiguous lanes.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < N; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

// Reduction across lanes that differ in bits >= log2(START).
template <int START>
__device__ __forceinline__ float across_sum(float x) {
#pragma unroll
    for (int o = START; o < 64; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

template <int START>
__device__ __forceinline__ float across_max(float x) {
#pragma unroll
    for (int o = START; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// 16 codes of one lane (channels [16w, 16w + 16)) -> floats in channel order.
template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t* wd, float (&cf)[16]) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t e = (wd[0] >> (2 * j)) & 0x03030303u;
#pragma unroll
            for (int k = 0; k < 4; ++k) cf[4 * k + j] = (float)((e >> (8 * k)) & 0xffu);
        }
    } else {
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t e = (wd[wi] >> (4 * j)) & 0x0f0f0f0fu;
#pragma unroll
                for (int k = 0; k < 4; ++k) cf[8 * wi + 2 * k + j] = (float)((e >> (8 * k)) & 0xffu);
            }
        }
    }
}

// Online-softmax update of one wave for one chunk of 32 tokens. sc holds the
// scores (base-2 log domain) of this lane's TPL tokens; on return p holds
// their weights relative to the running maximum m.
template <int QG, int TPL, int NW, int NC>
__device__ __forceinline__ void softmax_step(float (&sc)[QG][TPL], float (&p)[QG][TPL], float (&m)[QG],
                                             float (&l)[QG], float (&zacc)[QG], float (&o)[QG][NC]) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        float bm = sc[gq][0];
#pragma unroll
        for (int i = 1; i < TPL; ++i) bm = fmaxf(bm, sc[gq][i]);
        bm = across_max<NW>(bm);
        const float mn = fmaxf(m[gq], bm);
        if (mn > m[gq]) {
            const float alpha = exp2f(m[gq] - mn);
            l[gq] *= alpha;
            zacc[gq] *= alpha;
#pragma unroll
            for (int c = 0; c < NC; ++c) o[gq][c] *= alpha;
            m[gq] = mn;
        }
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            p[gq][i] = exp2f(sc[gq][i] - m[gq]);
            l[gq] += p[gq][i];
        }
    }
}

// One work-group (4 waves) per (split, unit, query chunk). A key split walks
// its key blocks, one block per wave at a time; the residual split walks the
// ring in chunks of 32 tokens. Lane = (token lane tl, column set w): w owns
// channels [16w, 16w + 16), tl owns tokens tl, tl + TL, ... of each chunk.
// Scores fold the key scale into the query, score = sum_c (q_c s_c) code_c +
// sum_c q_c z_c; values fold the token's scale into its weight,
// o_c += (p s_t) code_c, with sum_t p z_t added per lane at the end.
template <int D, int BITS, int QG>
__global__ __launch_bounds__(256) void attend_kernel(const AttendArgs a) {
    constexpr int NW = D / 16;   // column sets
    constexpr int TL = 64 / NW;  // token lanes
    constexpr int TPL = kG / TL; // tokens per lane per chunk
    constexpr int NWORD = BITS / 2;
    constexpr int W = D * BITS / 32;
    constexpr int NGV = D / kVG;
    const CacheGeom& g = a.g;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int w = lane % NW, tl = lane / NW;
    const int split = blockIdx.x;
    const int64_t u = blockIdx.y;
    const int group = g.n_q_heads / g.n_kv_heads;
    const int64_t b = u / g.n_kv_heads;
    const int h = (int)(u % g.n_kv_heads);
    const int qh0 = h * group + blockIdx.z * QG;

    float qv[QG][16];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        const uint16_t* qp = a.q + ((size_t)b * g.n_q_heads + qh0 + gq) * D + 16 * w;
        uint4 raw[2];
        raw[0] = reinterpret_cast<const uint4*>(qp)[0];
        raw[1] = reinterpret_cast<const uint4*>(qp)[1];
        const uint16_t* hv = reinterpret_cast<const uint16_t*>(raw);
#pragma unroll
        for (int c = 0; c < 16; ++c)
            qv[gq][c] = a.q_bf16 ? bf16_bits_to_float(hv[c]) : half_bits_to_float(hv[c]);
    }

    float m[QG], l[QG], zacc[QG], o[QG][16];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        m[gq] = -INFINITY;
        l[gq] = 0.f;
        zacc[gq] = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) o[gq][c] = 0.f;
    }

    if (split < a.n_key_splits) {
        const int64_t jb = (int64_t)split * a.blocks_per_split;
        const int64_t je = min(a.n_blocks, jb + a.blocks_per_split);
        const uint8_t* ubase = g.base + g.off_blocks + (size_t)u * g.unit_stride;
        for (int64_t j = jb + wave; j < je; j += 4) {
            const uint8_t* rec = ubase + (size_t)j * g.block_bytes;
            // key scales folded into the query, key zeros into a per-lane constant
            const float4* kszp = reinterpret_cast<const float4*>(rec + g.rec_ksz) + 8 * w;
            float qt[QG][16], zp[QG];
#pragma unroll
            for (int gq = 0; gq < QG; ++gq) zp[gq] = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 8; ++c2) {
                const float4 sz = kszp[c2];
#pragma unroll
                for (int gq = 0; gq < QG; ++gq) {
                    qt[gq][2 * c2] = qv[gq][2 * c2] * sz.x;
                    qt[gq][2 * c2 + 1] = qv[gq][2 * c2 + 1] * sz.z;
                    zp[gq] = fmaf(qv[gq][2 * c2], sz.y, zp[gq]);
                    zp[gq] = fmaf(qv[gq][2 * c2 + 1], sz.w, zp[gq]);
                }
            }
            const uint32_t* kc = reinterpret_cast<const uint32_t*>(rec + g.rec_kcode);
            float sc[QG][TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int t = tl + TL * i;
                uint32_t wd[NWORD];
#pragma unroll
                for (int n = 0; n < NWORD; ++n) wd[n] = kc[t * W + NWORD * w + n];
                float cf[16];
                unpack16<BITS>(wd, cf);
#pragma unroll
                for (int gq = 0; gq < QG; ++gq) {
                    float acc = zp[gq];
#pragma unroll
                    for (int c = 0; c < 16; ++c) acc = fmaf(qt[gq][c], cf[c], acc);
                    sc[gq][i] = group_sum<NW>(acc) * a.scale_log2;
                }
            }
            float p[QG][TPL];
            softmax_step<QG, TPL, NW, 16>(sc, p, m, l, zacc, o);
            const uint32_t* vcp = reinterpret_cast<const uint32_t*>(rec + g.rec_vcode);
            const float2* vsz = reinterpret_cast<const float2*>(rec + g.rec_vsz);
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int t = tl + TL * i;
                uint32_t wd[NWORD];
#pragma unroll
                for (int n = 0; n < NWORD; ++n) wd[n] = vcp[t * W + NWORD * w + n];
                const float2 sz = vsz[t * NGV + (w >> 1)];
                float cf[16];
                unpack16<BITS>(wd, cf);
#pragma unroll
                for (int gq = 0; gq < QG; ++gq) {
                    const float pt = p[gq][i] * sz.x;
                    zacc[gq] = fmaf(p[gq][i], sz.y, zacc[gq]);
#pragma unroll
                    for (int c = 0; c < 16; ++c) o[gq][c] = fmaf(pt, cf[c], o[gq][c]);
                }
            }
        }
    } else {
        // residual split: fp16 rows from the ring, in token order
        const int64_t nres = a.n_tokens - a.n_quant;
        const uint8_t* rbase = g.base + g.off_ring + (size_t)u * g.ring_unit_stride;
        const int64_t nchunk = (nres + kG - 1) / kG;
        for (int64_t ck = wave; ck < nchunk; ck += 4) {
            float sc[QG][TPL];
            bool valid[TPL];
            const uint8_t* rows[TPL];
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const int64_t idx = ck * kG + tl + TL * i;
                valid[i] = idx < nres;
                const int64_t slot = (a.n_quant + (valid[i] ? idx : 0)) % g.ring_slots;
                rows[i] = rbase + (size_t)slot * 4 * D;
                float kf[16];
                if (valid[i]) {
                    uint4 raw[2];
                    raw[0] = reinterpret_cast<const uint4*>(rows[i] + 32 * w)[0];
                    raw[1] = reinterpret_cast<const uint4*>(rows[i] + 32 * w)[1];
                    const uint16_t* hv = reinterpret_cast<const uint16_t*>(raw);
#pragma unroll
                    for (int c = 0; c < 16; ++c) kf[c] = half_bits_to_float(hv[c]);
                } else {
#pragma unroll
                    for (int c = 0; c < 16; ++c) kf[c] = 0.f;
                }
#pragma unroll
                for (int gq = 0; gq < QG; ++gq) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < 16; ++c) acc = fmaf(qv[gq][c], kf[c], acc);
                    acc = group_sum<NW>(acc) * a.scale_log2;
                    sc[gq][i] = valid[i] ? acc : -INFINITY;
                }
            }
            float p[QG][TPL];
            softmax_step<QG, TPL, NW, 16>(sc, p, m, l, zacc, o);
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                if (!valid[i]) continue;
                uint4 raw[2];
                raw[0] = reinterpret_cast<const uint4*>(rows[i] + 2 * D + 32 * w)[0];
                raw[1] = reinterpret_cast<const uint4*>(rows[i] + 2 * D + 32 * w)[1];
                const uint16_t* hv = reinterpret_cast<const uint16_t*>(raw);
#pragma unroll
                for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
                    for (int c = 0; c < 16; ++c) o[gq][c] = fmaf(p[gq][i], half_bits_to_float(hv[c]), o[gq][c]);
                }
            }
        }
    }

    // per-wave totals: fold the value zeros in, then sum over the token lanes
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        l[gq] = across_sum<NW>(l[gq]);
#pragma unroll
        for (int c = 0; c < 16; ++c) o[gq][c] = across_sum<NW>(o[gq][c] + zacc[gq]);
    }

    __shared__ float sm[4][QG], sl[4][QG];
    __shared__ float so[4][QG][D];
    if (tl == 0) {
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
            for (int c = 0; c < 16; ++c) so[wave][gq][16 * w + c] = o[gq][c];
            if (w == 0) {
                sm[wave][gq] = m[gq];
                sl[wave][gq] = l[gq];
            }
        }
    }
    __syncthreads();
    const size_t pstride = g.partial_stride / 4;
    float* pbase = reinterpret_cast<float*>(g.base + g.off_partial);
    for (int idx = threadIdx.x; idx < QG * D; idx += 256) {
        const int gq = idx / D, c = idx % D;
        float M = sm[0][gq];
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) M = fmaxf(M, sm[wv][gq]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
            if (sm[wv][gq] != -INFINITY) {
                const float f = exp2f(sm[wv][gq] - M);
                L = fmaf(sl[wv][gq], f, L);
                O = fmaf(so[wv][gq][c], f, O);
            }
        }
        float* rec = pbase + (((size_t)b * g.n_q_heads + qh0 + gq) * g.max_splits + split) * pstride;
        rec[c] = O;
        if (c == 0) {
            rec[D] = M;
            rec[D + 1] = L;
        }
    }

}

// Log-sum-exp merge of the splits of one (batch row, query head), in split
// order (deterministic). A separate launch: the kernel boundary makes every
// split's partial visible, where an in-kernel merge would need device-scope
// fences (full L2 write-back and invalidate on a multi-XCD part) in every
// work-group.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const AttendArgs a) {
    const CacheGeom& g = a.g;
    const size_t row = blockIdx.x;
    const int c = threadIdx.x;
    const size_t stride = g.partial_stride / 4;
    const float* rb = reinterpret_cast<const float*>(g.base + g.off_partial) + row * g.max_splits * stride;
    float M = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, rb[s * stride + D]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
        const float ms = rb[s * stride + D];
        if (ms != -INFINITY) {
            const float f = exp2f(ms - M);
            L = fmaf(rb[s * stride + D + 1], f, L);
            O = fmaf(rb[s * stride + c], f, O);
        }
    }
    a.out[row * D + c] = O / L;
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

template <int D, int BITS>
hipError_t attend_db(const AttendArgs& a, hipStream_t s) {
    const int group = a.g.n_q_heads / a.g.n_kv_heads;
    const int qg = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
    const dim3 grid((unsigned)a.n_split, (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads), (unsigned)(group / qg));
    if (qg == 4)
        attend_kernel<D, BITS, 4><<<grid, 256, 0, s>>>(a);
    else if (qg == 2)
        attend_kernel<D, BITS, 2><<<grid, 256, 0, s>>>(a);
    else
        attend_kernel<D, BITS, 1><<<grid, 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    combine_kernel<D><<<(unsigned)((int64_t)a.g.batch * a.g.n_q_heads), D, 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t attend_d(const AttendArgs& a, hipStream_t s) {
    return a.g.bits == 2 ? attend_db<D, 2>(a, s) : attend_db<D, 4>(a, s);
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

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
    switch (a.g.head_dim) {
        case 64: return attend_d<64>(a, s);
        case 128: return attend_d<128>(a, s);
        default: return attend_d<256>(a, s);
    }
}

}  // namespace kivi
