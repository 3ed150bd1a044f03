// attend.hip -- decode attention over the packed KIVI cache on gfx950.
//
// The KIVI explainer page ("ICML 2024論文解説: KIVI — チューニング不要のKVキャッシュ
// 2bit非対称量子化"), section 残差バッファ（Residual Buffer）: attention is one
// softmax of q . [D(K_quant); K_res]^T / sqrt(d) over every token, applied to
// [D(V_quant); V_res]; section 量子化アルゴリズム: D(x) = s x + z.
//
// Nothing is dequantized to memory. Per key block the key scales fold into
// the query (q~_c = q_c s_c, once per block and channel) and the key zeros
// into one constant (Z = sum_c q_c z_c), so a token's score is
// sum_c q~_c code_c + Z. Per value token the weight folds in the token's
// scale (p s_t) and the zeros accumulate as sum_t p z_t, added to every
// channel of the group at the end. One online softmax (base 2) runs over the
// key blocks and the fp16 residual of the work-group's share of the tokens;
// splits of a unit are merged by a log-sum-exp kernel afterwards.
//
// Lane layout inside a wave: lane = tl * NW + w. Column w owns channels
// [16w, 16w + 16) (one code word at b = 2, two at b = 4); token lane tl owns
// tokens tl, tl + TL, ... of every 32-token chunk. Reductions use DPP inside
// rows of 16 lanes and permlane swaps across rows: VALU only, no LDS traffic.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"
#include "split.hpp"

namespace kivi {
namespace {

constexpr int kG = 32;   // tokens per key block
constexpr int kVG = 32;  // channels per value group

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ------------------------------------------------------------ lane reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
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

// ------------------------------------------------------------ block records

// Record layout of one key block (see kivi.h): kcode [G][W], vcode [G][W],
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

// One lane's share of a block record, loaded ahead of its use.
template <int D, int BITS>
struct BlockRegs {
    static constexpr int NW = D / 16, TL = 64 / NW, TPL = kG / TL, NWORD = BITS / 2, CPL = D / 64;
    float ksz[2 * CPL];       // (s, z) of channels lane*CPL .. lane*CPL + CPL - 1
    uint32_t kc[TPL][NWORD];  // key code words of this lane's tokens and column
    uint32_t vc[TPL][NWORD];  // value code words
    float2 vsz[TPL];          // (s, z) of each token's value group that holds this column
};

template <int D, int BITS>
__device__ __forceinline__ void load_block(const uint8_t* rec, int lane, int w, int tl, BlockRegs<D, BITS>& r) {
    using B = BlockRegs<D, BITS>;
    using L = Rec<D, BITS>;
    const float* kszp = reinterpret_cast<const float*>(rec + L::ksz) + lane * 2 * B::CPL;
    if constexpr (B::CPL == 1) {
        const float2 v = *reinterpret_cast<const float2*>(kszp);
        r.ksz[0] = v.x;
        r.ksz[1] = v.y;
    } else {
#pragma unroll
        for (int k = 0; k < B::CPL / 2; ++k) {
            const float4 v = reinterpret_cast<const float4*>(kszp)[k];
            r.ksz[4 * k] = v.x;
            r.ksz[4 * k + 1] = v.y;
            r.ksz[4 * k + 2] = v.z;
            r.ksz[4 * k + 3] = v.w;
        }
    }
    const uint32_t* kc = reinterpret_cast<const uint32_t*>(rec + L::kcode);
    const uint32_t* vc = reinterpret_cast<const uint32_t*>(rec + L::vcode);
    const float2* vsz = reinterpret_cast<const float2*>(rec + L::vsz);
#pragma unroll
    for (int i = 0; i < B::TPL; ++i) {
        const int t = tl + B::TL * i;
        if constexpr (B::NWORD == 1) {
            r.kc[i][0] = kc[t * L::W + w];
            r.vc[i][0] = vc[t * L::W + w];
        } else {
            const uint2 kk = *reinterpret_cast<const uint2*>(kc + t * L::W + 2 * w);
            const uint2 vv = *reinterpret_cast<const uint2*>(vc + t * L::W + 2 * w);
            r.kc[i][0] = kk.x;
            r.kc[i][1] = kk.y;
            r.vc[i][0] = vv.x;
            r.vc[i][1] = vv.y;
        }
        r.vsz[i] = vsz[t * (D / kVG) + (w >> 1)];
    }
}

// Hides a value's bits from the optimizer, so that the byte conversions below
// stay one v_cvt_f32_ubyte{0..3} per code instead of a bit-field extract plus
// a conversion per code.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm("" : "+v"(x));
    return x;
}

// The 16 codes of one lane's column for one token, as floats in channel order:
// one mask isolates 4 codes, one per byte, then each byte converts directly.
template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t* wd, float (&cf)[16]) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t e = opaque((wd[0] >> (2 * j)) & 0x03030303u);
#pragma unroll
            for (int k = 0; k < 4; ++k) cf[4 * k + j] = (float)((e >> (8 * k)) & 0xffu);
        }
    } else {
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t e = opaque((wd[wi] >> (4 * j)) & 0x0f0f0f0fu);
#pragma unroll
                for (int k = 0; k < 4; ++k) cf[8 * wi + 2 * k + j] = (float)((e >> (8 * k)) & 0xffu);
            }
        }
    }
}

// ------------------------------------------------------------ online softmax

// New scores sc (base-2 log domain) of this lane's TPL tokens for each query:
// raise the running maximum if the chunk's maximum exceeds it (rescaling the
// accumulators), then turn the scores into weights p.
template <int QG, int TPL, int NW>
__device__ __forceinline__ void softmax_update(const float (&sc)[QG][TPL], float (&p)[QG][TPL], float (&m)[QG],
                                               float (&l)[QG], float (&zacc)[QG], float (&o)[QG][16]) {
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        float bm = sc[gq][0];
#pragma unroll
        for (int i = 1; i < TPL; ++i) bm = fmaxf(bm, sc[gq][i]);
        bm = tok_max<NW>(bm);  // the same in every lane of the wave
        if (bm > m[gq]) {
            const float alpha = __builtin_amdgcn_exp2f(m[gq] - bm);
            l[gq] *= alpha;
            zacc[gq] *= alpha;
#pragma unroll
            for (int c = 0; c < 16; ++c) o[gq][c] *= alpha;
            m[gq] = bm;
        }
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            p[gq][i] = __builtin_amdgcn_exp2f(sc[gq][i] - m[gq]);
            l[gq] += p[gq][i];
        }
    }
}

// ------------------------------------------------------------ kernel

template <int D, int BITS, int QG, int NWAVES>
__global__ __launch_bounds__(64 * NWAVES) void attend_kernel(const AttendArgs a) {
    using B = BlockRegs<D, BITS>;
    constexpr int NW = B::NW, TL = B::TL, TPL = B::TPL, CPL = B::CPL;
    constexpr int NT = 64 * NWAVES;
    __shared__ __align__(16) float s_q[QG][D];             // the query heads, fp32
    __shared__ __align__(16) float s_qt[NWAVES][QG][D];    // each wave's folded query q*s
    __shared__ float s_m[NWAVES][QG], s_l[NWAVES][QG];

    const CacheGeom& g = a.g;
    const int lane = threadIdx.x & 63;
    // the wave index is uniform across the wave: keep it (and every block
    // address derived from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = lane % NW, tl = lane / NW;
    const int split = blockIdx.x;
    const int64_t u = blockIdx.y;
    const int group = g.n_q_heads / g.n_kv_heads;
    const int64_t b = u / g.n_kv_heads;
    const int h = (int)(u % g.n_kv_heads);
    const size_t row0 = (size_t)b * g.n_q_heads + (size_t)h * group + (size_t)blockIdx.z * QG;
    const float scale = a.scale_log2;

    for (int idx = threadIdx.x; idx < QG * D; idx += NT) {
        const uint16_t v = a.q[row0 * D + idx];
        s_q[idx / D][idx % D] = a.q_bf16 ? bf2f(v) : h2f(v);
    }
    __syncthreads();
    float qf[QG][CPL];  // query at this lane's fold channels
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
        for (int k = 0; k < CPL; ++k) qf[gq][k] = s_q[gq][lane * CPL + k];

    // this work-group's and this wave's share of the tokens
    const int64_t nres = a.n_tokens - a.n_quant;
    const int64_t nrc = (nres + kG - 1) / kG;
    const int64_t cost = residual_chunk_cost(BITS);
    int64_t b0, b1;
    split_range(a.n_blocks, nrc, cost, a.n_split, split, &b0, &b1);
    const int64_t rc = split == a.n_split - 1 ? nrc : 0;
    const int64_t j0 = b0 + wave_start(b1 - b0, rc, cost, NWAVES, wave);
    const int64_t j1 = b0 + wave_start(b1 - b0, rc, cost, NWAVES, wave + 1);

    float m[QG], l[QG], zacc[QG], o[QG][16];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        m[gq] = -INFINITY;
        l[gq] = 0.f;
        zacc[gq] = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) o[gq][c] = 0.f;
    }

    const uint8_t* ubase = g.base + g.off_blocks + (size_t)u * g.unit_stride;
    B ra, rb;
    if (j0 < j1) load_block<D, BITS>(ubase + (size_t)j0 * Rec<D, BITS>::bytes, lane, w, tl, ra);

    // residual chunks: fp16 rows from the ring, in token order
    const uint8_t* rbase = g.base + g.off_ring + (size_t)u * g.ring_unit_stride;
    for (int64_t ck = wave; ck < rc; ck += NWAVES) {
        uint4 kraw[TPL][2];
        bool valid[TPL];
        const uint8_t* rows[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int64_t idx = ck * kG + tl + TL * i;
            valid[i] = idx < nres;
            const int64_t slot = (a.n_quant + (valid[i] ? idx : 0)) % g.ring_slots;
            rows[i] = rbase + (size_t)slot * 4 * D + 32 * w;
            const uint4* kp = reinterpret_cast<const uint4*>(rows[i]);
            kraw[i][0] = kp[0];
            kraw[i][1] = kp[1];
        }
        float sc[QG][TPL];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float qv[16];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_q[gq][16 * w + 4 * c4]);
                qv[4 * c4] = x.x;
                qv[4 * c4 + 1] = x.y;
                qv[4 * c4 + 2] = x.z;
                qv[4 * c4 + 3] = x.w;
            }
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const uint16_t* kh = reinterpret_cast<const uint16_t*>(kraw[i]);
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc = fmaf(qv[c], h2f(kh[c]), acc);
                acc = sum_cols<NW>(acc) * scale;
                sc[gq][i] = valid[i] ? acc : -INFINITY;
            }
        }
        uint4 vraw[TPL][2];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const uint4* vp = reinterpret_cast<const uint4*>(rows[i] + 2 * D);
            vraw[i][0] = vp[0];
            vraw[i][1] = vp[1];
        }
        float p[QG][TPL];
        softmax_update<QG, TPL, NW>(sc, p, m, l, zacc, o);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const uint16_t* vh = reinterpret_cast<const uint16_t*>(vraw[i]);
#pragma unroll
            for (int gq = 0; gq < QG; ++gq) {
                const float pw = valid[i] ? p[gq][i] : 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) o[gq][c] = fmaf(pw, h2f(vh[c]), o[gq][c]);
            }
        }
    }

    // key blocks: two register sets alternate, so the loads of the next block
    // are in flight while the current one is computed
    auto block_math = [&](const B& r) {
        float Z[QG];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float zp = 0.f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                s_qt[wave][gq][lane * CPL + k] = qf[gq][k] * r.ksz[2 * k];
                zp = fmaf(qf[gq][k], r.ksz[2 * k + 1], zp);
            }
            Z[gq] = wave_sum(zp);
        }
        wave_lds_order();
        float sc[QG][TPL];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float qt[16];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_qt[wave][gq][16 * w + 4 * c4]);
                qt[4 * c4] = x.x;
                qt[4 * c4 + 1] = x.y;
                qt[4 * c4 + 2] = x.z;
                qt[4 * c4 + 3] = x.w;
            }
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float cf[16];
                unpack16<BITS>(r.kc[i], cf);
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc = fmaf(qt[c], cf[c], acc);
                sc[gq][i] = (sum_cols<NW>(acc) + Z[gq]) * scale;
            }
        }
        wave_lds_order();
        float p[QG][TPL];
        softmax_update<QG, TPL, NW>(sc, p, m, l, zacc, o);
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            float cf[16];
            unpack16<BITS>(r.vc[i], cf);
#pragma unroll
            for (int gq = 0; gq < QG; ++gq) {
                const float pt = p[gq][i] * r.vsz[i].x;
                zacc[gq] = fmaf(p[gq][i], r.vsz[i].y, zacc[gq]);
#pragma unroll
                for (int c = 0; c < 16; ++c) o[gq][c] = fmaf(pt, cf[c], o[gq][c]);
            }
        }
    };
    for (int64_t j = j0; j < j1; j += 2) {
        if (j + 1 < j1) load_block<D, BITS>(ubase + (size_t)(j + 1) * Rec<D, BITS>::bytes, lane, w, tl, rb);
        block_math(ra);
        if (j + 1 >= j1) break;
        if (j + 2 < j1) load_block<D, BITS>(ubase + (size_t)(j + 2) * Rec<D, BITS>::bytes, lane, w, tl, ra);
        block_math(rb);
    }

    // per-wave totals: the value zeros join their channels, then the token lanes sum
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        l[gq] = tok_sum<NW>(l[gq]);
#pragma unroll
        for (int c = 0; c < 16; ++c) o[gq][c] = tok_sum<NW>(o[gq][c] + zacc[gq]);
    }
    __syncthreads();  // every wave is done with s_qt
    if (tl == 0) {
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
            for (int c = 0; c < 16; ++c) s_qt[wave][gq][16 * w + c] = o[gq][c];
            if (w == 0) {
                s_m[wave][gq] = m[gq];
                s_l[wave][gq] = l[gq];
            }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < QG * D; idx += NT) {
        const int gq = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < NWAVES; ++wv) M = fmaxf(M, s_m[wv][gq]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int wv = 0; wv < NWAVES; ++wv) {
            if (s_m[wv][gq] != -INFINITY) {
                const float f = __builtin_amdgcn_exp2f(s_m[wv][gq] - M);
                L = fmaf(s_l[wv][gq], f, L);
                O = fmaf(s_qt[wv][gq][c], f, O);
            }
        }
        if (a.n_split == 1) {
            a.out[(row0 + gq) * D + c] = O / L;
        } else {
            float* rec = reinterpret_cast<float*>(g.base + g.off_partial +
                                                  ((row0 + gq) * g.max_splits + split) * g.partial_stride);
            rec[c] = O;
            if (c == 0) {
                rec[D] = M;
                rec[D + 1] = L;
            }
        }
    }
}

// Log-sum-exp merge of the splits of one (batch row, query head), in split order.
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
            const float f = __builtin_amdgcn_exp2f(ms - M);
            L = fmaf(rb[s * stride + D + 1], f, L);
            O = fmaf(rb[s * stride + c], f, O);
        }
    }
    a.out[row * D + c] = O / L;
}

template <int D, int BITS, int QG, int NWAVES>
hipError_t attend_launch(const AttendArgs& a, hipStream_t s) {
    const int group = a.g.n_q_heads / a.g.n_kv_heads;
    const dim3 grid((unsigned)a.n_split, (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads), (unsigned)(group / QG));
    attend_kernel<D, BITS, QG, NWAVES><<<grid, 64 * NWAVES, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    combine_kernel<D><<<(unsigned)((int64_t)a.g.batch * a.g.n_q_heads), D, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int BITS>
hipError_t attend_db(const AttendArgs& a, hipStream_t s) {
    switch (a.nwaves * 8 + a.qg) {
        case 4 * 8 + 4: return attend_launch<D, BITS, 4, 4>(a, s);
        case 4 * 8 + 2: return attend_launch<D, BITS, 2, 4>(a, s);
        case 8 * 8 + 2: return attend_launch<D, BITS, 2, 8>(a, s);
        case 8 * 8 + 1: return attend_launch<D, BITS, 1, 8>(a, s);
        default: return attend_launch<D, BITS, 1, 16>(a, s);
    }
}

template <int D>
hipError_t attend_d(const AttendArgs& a, hipStream_t s) {
    static_assert(Rec<D, 2>::bytes == 2 * kG * D * 2 / 32 * 4 + D * 8 + kG * (D / kVG) * 8, "record layout");
    return a.g.bits == 2 ? attend_db<D, 2>(a, s) : attend_db<D, 4>(a, s);
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
    // the kernel takes the record layout from (D, BITS); it must be the one the cache uses
    const int W = a.g.head_dim * a.g.bits / 32;
    if (a.g.rec_kcode != 0 || a.g.rec_vcode != (size_t)kG * W * 4 || a.g.rec_ksz != (size_t)2 * kG * W * 4 ||
        a.g.rec_vsz != a.g.rec_ksz + (size_t)a.g.head_dim * 8 ||
        a.g.block_bytes != a.g.rec_vsz + (size_t)kG * (a.g.head_dim / kVG) * 8)
        return hipErrorInvalidValue;
    switch (a.g.head_dim) {
        case 64: return attend_d<64>(a, s);
        case 128: return attend_d<128>(a, s);
        default: return attend_d<256>(a, s);
    }
}

}  // namespace kivi
