// attend.hip -- decode attention over the packed KIVI cache on gfx950: the
// vector-unit kernel (one, two or four query heads per work-group), the merge
// of the splits, and the dispatch (four query heads at d = 128 go to the
// matrix-core kernel of attend_gqa.hip).
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
// Codes are never converted one by one. One AND of a packed word with a mask
// leaves one code in each 16-bit half, inside the mantissa field of an fp16
// subnormal, so the half reads exactly as code * 2^(b*j - 24) for the code's
// bit position b*j in the half; v_fma_mix_f32 takes that half as an operand
// of an fp32 FMA (the half widens exactly, one rounding as in an fp32 FMA).
// Half the positions of a half-word are masked in place and half after one
// shift right by 8 bits, so b*j < 8 and the code never reaches the exponent
// field. The powers of two go into the query (key side: q_c 2^(-b j(c)), and
// 2^24 into the score scale) and into the value weights (value side:
// 2^(24 - b j(t)) per token).
//
// Lane layout inside a wave: lane = tl * NW + w. Column w owns channels
// [CW w, CW w + CW) (CW = 32 at d = 128, else 16: CW b / 32 code words); token
// lane tl owns tokens tl, tl + TL, ... of every 32-token chunk. Reductions use DPP inside
// rows of 16 lanes and permlane swaps across rows: VALU only, no LDS traffic.
// Block records are read with buffer loads: the unit's records are one
// buffer (paged blocks: each block's page record is one), the block offset is
// a scalar and each lane's offsets are constants, so no vector instruction
// goes to address arithmetic.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "attend_common.hpp"
#include "kivi.h"
#include "split.hpp"

namespace kivi {
namespace {

// ------------------------------------------------------------ block loads

// A lane's byte offsets inside any record: its key-code word of token tl
// (token tl + TL*i at i*TL*W*4 more), its value-code words, its key (s, z)
// and its value (s, z) of token tl.
struct LaneOffsets {
    int code, vcode, ksz, vsz;
};

template <int D, int BITS, int CW>
__device__ __forceinline__ LaneOffsets lane_offsets(int lane, int w, int tl) {
    using B = BlockRegs<D, BITS, CW>;
    using L = Rec<D, BITS>;
    LaneOffsets o;
    o.code = (tl * L::W + w * B::NWORD) * 4;
    o.vcode = L::vcode + lane * B::CPV * BITS * 4;
    o.ksz = L::ksz + lane * 2 * B::CPL * 4;
    o.vsz = L::vsz + (tl * (D / kVG) + w * CW / kVG) * 8;
    return o;
}

template <int D, int BITS, int CW>
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rs, uint32_t soff, const LaneOffsets& lo,
                                           BlockRegs<D, BITS, CW>& r) {
    using B = BlockRegs<D, BITS, CW>;
    using L = Rec<D, BITS>;
    const int so = __builtin_amdgcn_readfirstlane((int)soff);  // uniform: the block's offset
    if constexpr (B::CPL == 1) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.ksz, so, 2);
        r.ksz[0] = __uint_as_float(v[0]);
        r.ksz[1] = __uint_as_float(v[1]);
    } else {
#pragma unroll
        for (int k = 0; k < B::CPL / 2; ++k) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lo.ksz + 16 * k, so, 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.ksz[4 * k + e] = __uint_as_float(v[e]);
        }
    }
#pragma unroll
    for (int i = 0; i < B::TPL; ++i) {
        const int toff = i * B::TL * L::W * 4;
        if constexpr (B::NWORD == 1) {
            r.kc[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.code + toff, so, 2);
        } else if constexpr (B::NWORD == 2) {
            const auto kk = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.code + toff, so, 2);
            r.kc[i][0] = kk[0];
            r.kc[i][1] = kk[1];
        } else {
            const auto kk = __builtin_amdgcn_raw_buffer_load_b128(rs, lo.code + toff, so, 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.kc[i][e] = kk[e];
        }
        const auto sz = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.vsz + i * B::TL * (D / kVG) * 8, so, 2);
        r.vsz[i] = make_float2(__uint_as_float(sz[0]), __uint_as_float(sz[1]));
    }
    constexpr int NV = B::CPV * BITS;  // 2, 4, 8 or 16 words, contiguous
    if constexpr (NV == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.vcode, so, 2);
        r.vc[0] = v[0];
        r.vc[1] = v[1];
    } else {
#pragma unroll
        for (int k = 0; k < NV / 4; ++k) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lo.vcode + 16 * k, so, 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.vc[4 * k + e] = v[e];
        }
    }
}

// ------------------------------------------------------------ codes as fp16 halves

// Where the code of column channel ch sits once masked: codes per 16-bit half
// PH = 16 / b; the first ND = PH / 2 of a half are masked in place, the rest
// after a shift right by 8, so the code lands at bit b * jpos(ch) of its half.
template <int BITS>
struct CodePos {
    static constexpr int PH = 16 / BITS;
    static constexpr int ND = PH / 2;
    static constexpr int NWORD = BITS / 2;
    __device__ static constexpr int jpos(int ch) { return (ch % PH) % ND; }
};

// The codes of NWD packed words as exact floats, in code order: word k holds
// codes [P k, P (k + 1)) (P = 32 / b), code P k + i at bits [b i, b i + b), and
// cf[P k + i] = code * 2^(b * jpos(i) - 24). Key side: one token's channels
// of a column (CW b / 32 words); value side: one word of a channel's tokens.
// Each cf feeds an FMA directly (v_fma_mix_f32 reads the half).
template <int BITS, int NWD>
__device__ __forceinline__ void code_halves(const uint32_t* wd, float (&cf)[NWD * 32 / BITS]) {
    using P = CodePos<BITS>;
    constexpr uint32_t M = (1u << BITS) - 1;
#pragma unroll
    for (int k = 0; k < NWD; ++k) {
        const uint32_t sh = wd[k] >> 8;
#pragma unroll
        for (int p = 0; p < P::PH; ++p) {
            const int j = p % P::ND;
            const uint32_t x = (p < P::ND ? wd[k] : sh) & ((M << (BITS * j)) | (M << (16 + BITS * j)));
            cf[2 * P::PH * k + p] = half_lo(x);
            cf[2 * P::PH * k + P::PH + p] = half_hi(x);
        }
    }
}

// ------------------------------------------------------------ online softmax

// New scores sc (base-2 log domain) of this lane's TPL tokens for each query:
// raise the running maximum if the chunk's maximum exceeds it (rescaling the
// accumulators), then turn the scores into weights p.
template <int QG, int TPL, int NW, int NO>
__device__ __forceinline__ void softmax_update(const float (&sc)[QG][TPL], float (&p)[QG][TPL], float (&m)[QG],
                                               float (&l)[QG], float (&zacc)[QG], float (&o)[QG][NO]) {
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
            for (int c = 0; c < NO; ++c) o[gq][c] *= alpha;
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

// Channels per score column of attend_kernel: 32 at d = 128 (4 columns x 16
// token lanes, 2 tokens per lane: a token's score needs 2 cross-lane sums
// instead of 3, and the softmax and weight steps run over 2 tokens a lane
// instead of 4), else 16.
constexpr int attend_cw(int D) { return D == 128 ? 32 : 16; }

// Key blocks computed together by one wave: two with one query head at
// d <= 128 (their LDS round trips and cross-lane reductions are shared, and
// the two blocks' independent work interleaves), else one.
constexpr int attend_pair(int D, int QG) { return QG == 1 && D <= 128 ? 2 : 1; }

// Key blocks each wave keeps in registers: the NP being computed and the
// next NP in flight (two blocks in flight with one query head at d <= 128;
// measured on MI355X, more buys nothing once the HBM queue is full), else
// the one being computed and one in flight.
constexpr int attend_prefetch(int D, int QG) { return 2 * attend_pair(D, QG); }

// Two lane layouts per wave. Key side: lane = tl * NW + w scores tokens
// tl + TL*i against channels [CW w, CW w + CW). Value side: lane L accumulates
// channels [L*CPV, L*CPV + CPV) over all 32 tokens of a chunk, with the
// chunk's weights passed through a wave-private LDS slot (one row of 32
// weights per value group, the group's scale and the code-half factor folded in).
template <int D, int BITS, int QG, int NWAVES, bool RAGGED>
__global__ __launch_bounds__(64 * NWAVES) void attend_kernel(const AttendArgs a) {
    constexpr int CW = attend_cw(D);
    using B = BlockRegs<D, BITS, CW>;
    using P = CodePos<BITS>;
    using L = Rec<D, BITS>;
    constexpr int NW = B::NW, TL = B::TL, TPL = B::TPL, CPL = B::CPL, CPV = B::CPV;
    constexpr int NG = D / kVG;  // value groups of a token
    constexpr int NACC = 2;      // partial sums per value channel (shorter dependency chains)
    constexpr int NT = 64 * NWAVES;
    __shared__ __align__(16) float s_q[QG][D];              // the query heads, fp32
    constexpr int NP = attend_pair(D, QG);                        // key blocks computed together
    __shared__ __align__(16) float s_qt[NWAVES][NP][QG][D];      // each wave's folded queries; at the end its output
    __shared__ __align__(16) float s_p[NWAVES][NP][QG][NG][kG];  // each wave's value weights of NP chunks
    __shared__ float s_m[NWAVES][QG], s_l[NWAVES][QG], s_z[NWAVES][QG][NG];

    const CacheGeom& g = a.g;
    const int lane = threadIdx.x & 63;
    // the wave index is uniform across the wave: keep it (and every block
    // offset derived from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = lane % NW, tl = lane / NW;
    const int cv0 = lane * CPV, vgrp = cv0 / kVG;  // this lane's value channels and their group
    const int wgrp = w * CW / kVG;                 // the value group of column w
    const bool wlead = w * CW % kVG == 0;          // writes its group's value weights
    const int split = blockIdx.x;
    const int64_t u = dispatch_unit<RAGGED>(a, blockIdx.y);
    const int group = g.n_q_heads / g.n_kv_heads;
    const int64_t b = u / g.n_kv_heads;
    const int h = (int)(u % g.n_kv_heads);
    const size_t row0 = (size_t)b * g.n_q_heads + (size_t)h * group + (size_t)blockIdx.z * QG;
    const float scale = a.scale_log2;
    const float scale_q = ldexpf(a.scale_log2, 24);  // for scores summed in units of 2^-24

    // this work-group's and this wave's share of the tokens (kernel arguments only)
    // this unit's counters (its batch row's, when the rows differ in length)
    const RowCounts cnt = row_counts<RAGGED>(a, b);
    if constexpr (RAGGED)
        if (split >= cnt.n_split) return;  // an idle split of a shorter row (the whole work-group)
    const int64_t nres = cnt.n_tokens - cnt.n_quant;
    const int64_t nrc = (nres + kG - 1) / kG;
    const int64_t cost = kResidualChunkCost;
    int64_t b0, b1;
    split_range(cnt.n_blocks, nrc, cost, cnt.n_split, split, &b0, &b1);
    const int rc = (int)(split == cnt.n_split - 1 ? nrc : 0);
    // this wave's key blocks: j0, j0 + NWAVES, ... below j1 (round robin). Block
    // indices of a unit fit in 32 bits (its records are one buffer of < 4 GiB);
    // readfirstlane keeps them, and each block offset, in scalar registers
    const int j0 = __builtin_amdgcn_readfirstlane((int)b0 + wave);
    const int j1 = __builtin_amdgcn_readfirstlane((int)b1);

    // the first NP key blocks go in flight before anything waits
    constexpr int PF = attend_prefetch(D, QG);
    const uint8_t* ubase = g.base + g.off_blocks + (size_t)u * g.unit_stride;
    const __amdgpu_buffer_rsrc_t rs = records(ubase, (uint64_t)cnt.n_blocks * L::bytes);
    const LaneOffsets lo = lane_offsets<D, BITS, CW>(lane, w, tl);
    // key block j into r: an offset into the unit's records, or (paged blocks,
    // built with a row table) its own page's record. A wave issues its blocks
    // in order, j0, j0 + NWAVES, ...: each block's table entry was read one
    // call earlier, and the call reads the next one, so no call waits on it.
    int32_t pg_next = 0;
    if constexpr (RAGGED)
        if (g.table && j0 < j1) pg_next = table_entry(g, b, j0);
    auto issue = [&](int j, B& r) {
        if constexpr (RAGGED) {
            if (g.table) {
                const int32_t p = pg_next;
                if (j + NWAVES < j1) pg_next = table_entry(g, b, j + NWAVES);
                load_block<D, BITS>(records(g.base + page_offset(g, p, h), L::bytes), 0u, lo, r);
                return;
            }
        }
        load_block<D, BITS>(rs, (uint32_t)(j * L::bytes), lo, r);
    };
    B rr[PF];
#pragma unroll
    for (int k = 0; k < NP; ++k)
        if (j0 + k * NWAVES < j1) issue(j0 + k * NWAVES, rr[k]);

    // residual chunks (fp16 rows from the ring) are computed first, while the
    // first blocks are in flight (memory is idle once the last block lands, so
    // work left after it lengthens the tail); a wave's first chunk is loaded now
    const uint8_t* rbase = g.base + g.off_ring + (size_t)u * g.ring_unit_stride;
    const int ring = (int)g.ring_slots;
    const int slot0 = (int)(cnt.n_quant % g.ring_slots);
    const int ck0 = NWAVES - 1 - wave;  // chunk ck goes to wave NWAVES - 1 - ck % NWAVES
    constexpr int VRW = (CPV + 1) / 2;  // words of fp16 value pairs per token
    uint4 kraw[TPL][CW / 8];            // key rows of this lane's tokens, column w
    uint32_t vr[kG][VRW];               // value rows of this lane's channels, all 32 tokens
    bool valid[TPL];
    auto load_chunk = [&](int ck) {
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int idx = ck * kG + tl + TL * i;
            valid[i] = idx < (int)nres;
            const int ie = valid[i] ? idx : (int)nres - 1;  // past the end: the last token's row
            int slot = slot0 + ie;  // ie < ring: one wrap at most
            slot -= slot >= ring ? ring : 0;
            // the token appended by this call comes from its input row
            const uint4* kp = cnt.n_quant + ie == cnt.t_new
                                  ? reinterpret_cast<const uint4*>(a.k_new + u * D + CW * w)
                                  : reinterpret_cast<const uint4*>(rbase + (size_t)slot * 4 * D + 2 * CW * w);
#pragma unroll
            for (int e = 0; e < CW / 8; ++e) kraw[i][e] = kp[e];
        }
#pragma unroll
        for (int t = 0; t < kG; ++t) {
            // tokens past the residual's end (weight 0) read the last token's
            // row, which is finite: it is in the ring, or it is the new token's
            // input row (the first residual slot is not written yet when the
            // new token is the only one)
            const int idx = ck * kG + t;
            const int ie = idx < (int)nres ? idx : (int)nres - 1;
            int slot = slot0 + ie;
            slot -= slot >= ring ? ring : 0;
            const uint8_t* vp = cnt.n_quant + ie == cnt.t_new
                                    ? reinterpret_cast<const uint8_t*>(a.v_new + u * D + cv0)
                                    : rbase + (size_t)slot * 4 * D + 2 * D + 2 * cv0;
            if constexpr (CPV == 1) {
                vr[t][0] = *reinterpret_cast<const uint16_t*>(vp);
            } else if constexpr (CPV == 2) {
                vr[t][0] = *reinterpret_cast<const uint32_t*>(vp);
            } else {
                const uint2 x = *reinterpret_cast<const uint2*>(vp);
                vr[t][0] = x.x;
                vr[t][1] = x.y;
            }
        }
    };
    constexpr bool kEarly = D <= 128;  // d = 256: a chunk and the first blocks take too many registers
    if (kEarly && ck0 < rc) load_chunk(ck0);
    if (cnt.t_new >= 0 && split == cnt.n_split - 1 && blockIdx.z == 0 && wave == 0)
        write_new_token<D>(a, u, cnt.t_new, rbase);

    for (int idx = threadIdx.x; idx < QG * D; idx += NT) {
        const uint16_t v = a.q[row0 * D + idx];
        s_q[idx / D][idx % D] = a.q_bf16 ? bf2f(v) : h2f(v);
    }
    __syncthreads();
    // the query at this lane's fold channels, pre-scaled for the code halves
    // (key scales) and into units of 2^-24 (key zeros)
    float qf[QG][CPL], qz[QG][CPL];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = lane * CPL + k;
            qf[gq][k] = ldexpf(s_q[gq][c], -BITS * P::jpos(c % 16));
            qz[gq][k] = ldexpf(s_q[gq][c], -24);
        }
    // the code-half factor of this lane's key-side tokens tl + TL*i, folded
    // into their value weights: 2^(24 - b jpos(token))
    float tf[TPL];
#pragma unroll
    for (int i = 0; i < TPL; ++i) tf[i] = ldexpf(1.0f, 24 - BITS * P::jpos(tl + TL * i));

    float m[QG], l[QG], zacc[QG], o[QG][CPV * NACC];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        m[gq] = -INFINITY;
        l[gq] = 0.f;
        zacc[gq] = 0.f;
#pragma unroll
        for (int c = 0; c < CPV * NACC; ++c) o[gq][c] = 0.f;
    }

    // one residual chunk (rows loaded by load_chunk)
    auto chunk_math = [&]() {
        float sc[QG][TPL];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float qv[CW];
#pragma unroll
            for (int c4 = 0; c4 < CW / 4; ++c4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_q[gq][CW * w + 4 * c4]);
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
                for (int c = 0; c < CW; ++c) acc = fmaf(qv[c], h2f(kh[c]), acc);
                acc = sum_cols<NW>(acc) * scale;
                sc[gq][i] = valid[i] ? acc : -INFINITY;
            }
        }
        float p[QG][TPL];
        softmax_update<QG, TPL, NW, CPV * NACC>(sc, p, m, l, zacc, o);
        if (w == 0) {
#pragma unroll
            for (int gq = 0; gq < QG; ++gq)
#pragma unroll
                for (int i = 0; i < TPL; ++i) s_p[wave][0][gq][0][tl + TL * i] = valid[i] ? p[gq][i] : 0.f;
        }
        wave_lds_order();
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float pv[kG];
#pragma unroll
            for (int t4 = 0; t4 < kG / 4; ++t4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_p[wave][0][gq][0][4 * t4]);
                pv[4 * t4] = x.x;
                pv[4 * t4 + 1] = x.y;
                pv[4 * t4 + 2] = x.z;
                pv[4 * t4 + 3] = x.w;
            }
#pragma unroll
            for (int k = 0; k < CPV; ++k)
#pragma unroll
                for (int t = 0; t < kG; ++t) {
                    const float v = (k & 1) ? half_hi(vr[t][k / 2]) : half_lo(vr[t][k / 2]);
                    o[gq][k * NACC + t % NACC] = fmaf(pv[t], v, o[gq][k * NACC + t % NACC]);
                }
        }
        wave_lds_order();
    };

    // key blocks, NB (one or two) at a time: their folds and value weights go
    // through the LDS together, and one softmax update covers all their tokens
    auto blocks_math = [&](auto nb_tag, const B* r) {
        constexpr int NB = decltype(nb_tag)::value;
        float Z[NB][QG];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int gq = 0; gq < QG; ++gq) {
                float zp = 0.f;
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    s_qt[wave][bb][gq][lane * CPL + k] = qf[gq][k] * r[bb].ksz[2 * k];
                    zp = fmaf(qz[gq][k], r[bb].ksz[2 * k + 1], zp);
                }
                Z[bb][gq] = wave_sum(zp);
            }
        wave_lds_order();
        // scores: token by token, every query against the same CW code halves
        float sc[QG][NB * TPL];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            float qt[QG][CW];
#pragma unroll
            for (int gq = 0; gq < QG; ++gq)
#pragma unroll
                for (int c4 = 0; c4 < CW / 4; ++c4) {
                    const float4 x = *reinterpret_cast<const float4*>(&s_qt[wave][bb][gq][CW * w + 4 * c4]);
                    qt[gq][4 * c4] = x.x;
                    qt[gq][4 * c4 + 1] = x.y;
                    qt[gq][4 * c4 + 2] = x.z;
                    qt[gq][4 * c4 + 3] = x.w;
                }
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                float cf[CW];
                code_halves<BITS, B::NWORD>(r[bb].kc[i], cf);
#pragma unroll
                for (int gq = 0; gq < QG; ++gq) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < CW; ++c) acc = fmaf(qt[gq][c], cf[c], acc);
                    sc[gq][bb * TPL + i] = (sum_cols<NW>(acc) + Z[bb][gq]) * scale_q;
                }
            }
        }
        float p[QG][NB * TPL];
        softmax_update<QG, NB * TPL, NW, CPV * NACC>(sc, p, m, l, zacc, o);
        // value weights p s_t 2^(24 - b jpos(t)) of token t in its group's row;
        // the value zeros accumulate per lane as sum p z_t
        if (wlead) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int gq = 0; gq < QG; ++gq)
#pragma unroll
                    for (int i = 0; i < TPL; ++i) {
                        s_p[wave][bb][gq][wgrp][tl + TL * i] = p[gq][bb * TPL + i] * (r[bb].vsz[i].x * tf[i]);
                        zacc[gq] = fmaf(p[gq][bb * TPL + i], r[bb].vsz[i].y, zacc[gq]);
                    }
        }
        wave_lds_order();
        // values: one code word (32/b tokens) of one channel at a time, against each query's weights
        constexpr int PW = 32 / BITS;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int k = 0; k < CPV; ++k)
#pragma unroll
                for (int wd = 0; wd < BITS; ++wd) {
                    float cf[PW];
                    code_halves<BITS, 1>(&r[bb].vc[k * BITS + wd], cf);
#pragma unroll
                    for (int gq = 0; gq < QG; ++gq) {
                        float pv[PW];
#pragma unroll
                        for (int t4 = 0; t4 < PW / 4; ++t4) {
                            const float4 x =
                                *reinterpret_cast<const float4*>(&s_p[wave][bb][gq][vgrp][PW * wd + 4 * t4]);
                            pv[4 * t4] = x.x;
                            pv[4 * t4 + 1] = x.y;
                            pv[4 * t4 + 2] = x.z;
                            pv[4 * t4 + 3] = x.w;
                        }
#pragma unroll
                        for (int t = 0; t < PW; ++t)
                            o[gq][k * NACC + t % NACC] = fmaf(pv[t], cf[t], o[gq][k * NACC + t % NACC]);
                    }
                }
        wave_lds_order();
    };
    for (int ck = ck0; ck < rc; ck += NWAVES) {
        if (!kEarly || ck != ck0) load_chunk(ck);
        chunk_math();
    }
    // a ring of PF = 2 NP register sets: the NP blocks being computed, and the
    // next NP in flight (issued just before)
    for (int j = j0; j < j1; j += PF * NWAVES) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int jj = j + h * NP * NWAVES;
            if (jj >= j1) break;
            // issue priority by work left: the SIMD favours older waves, so
            // without it the younger waves of a work-group finish last
            {
                const int left = (j1 - jj + NWAVES - 1) / NWAVES;
                if (left >= 6) __builtin_amdgcn_s_setprio(3);
                else if (left >= 4) __builtin_amdgcn_s_setprio(2);
                else if (left >= 2) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
#pragma unroll
            for (int e = 0; e < NP; ++e) {
                const int jn = jj + (NP + e) * NWAVES;
                if (jn < j1) issue(jn, rr[(1 - h) * NP + e]);
            }
            if (NP == 2 && jj + NWAVES < j1)
                blocks_math(std::integral_constant<int, NP>(), &rr[h * NP]);
            else
                blocks_math(std::integral_constant<int, 1>(), &rr[h * NP]);
        }
    }

    // per-wave totals: the weight sum and each group's value-zero sum over the
    // token lanes; the zero sum joins every channel of its group
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        l[gq] = tok_sum<NW>(l[gq]);
        const float zt = tok_sum<NW>(zacc[gq]);
        if (tl == 0 && wlead) s_z[wave][gq][wgrp] = zt;
    }
    wave_lds_order();
    float ov[QG][CPV];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
        for (int k = 0; k < CPV; ++k) {
            float acc = s_z[wave][gq][vgrp];
#pragma unroll
            for (int e = 0; e < NACC; ++e) acc += o[gq][k * NACC + e];
            ov[gq][k] = acc;
        }
    __syncthreads();  // every wave is done with s_qt
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
#pragma unroll
        for (int k = 0; k < CPV; ++k) s_qt[wave][0][gq][cv0 + k] = ov[gq][k];
        if (lane == 0) {
            s_m[wave][gq] = m[gq];
            s_l[wave][gq] = l[gq];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < QG * D; idx += NT) {
        const int gq = idx / D, c = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < NWAVES; ++wv) M = fmaxf(M, s_m[wv][gq]);
        float Lsum = 0.f, O = 0.f;
#pragma unroll
        for (int wv = 0; wv < NWAVES; ++wv) {
            if (s_m[wv][gq] != -INFINITY) {
                const float f = __builtin_amdgcn_exp2f(s_m[wv][gq] - M);
                Lsum = fmaf(s_l[wv][gq], f, Lsum);
                O = fmaf(s_qt[wv][0][gq][c], f, O);
            }
        }
        if (a.n_split == 1) {
            a.out[(row0 + gq) * D + c] = O / Lsum;
        } else {
            float* rec = reinterpret_cast<float*>(g.partial + ((row0 + gq) * g.partial_splits + split) * g.partial_stride);
            rec[c] = O;
            if (c == 0) {
                rec[D] = M;
                rec[D + 1] = Lsum;
            }
        }
    }
}

// Log-sum-exp merge of the splits of one (batch row, query head), in split
// order. The splits' (m, l, o) are read 16 at a time in one round of loads
// (a second round waiting on the first would double the kernel's latency);
// a group's maximum rescales the sums of the groups before it.
template <int D, bool RAGGED>
__global__ __launch_bounds__(D) void combine_kernel(const AttendArgs a) {
    constexpr int CH = 16;
    const CacheGeom& g = a.g;
    const size_t row = blockIdx.x;
    const int c = threadIdx.x;
    const size_t stride = g.partial_stride / 4;
    const float* rb = reinterpret_cast<const float*>(g.partial) + row * g.partial_splits * stride;
    const int n_split = (int)row_counts<RAGGED>(a, (int64_t)(row / g.n_q_heads)).n_split;  // this batch row's splits
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += CH) {
        float ms[CH], ls[CH], os[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const bool in = s0 + i < n_split;
            const float* r = rb + (size_t)(in ? s0 + i : s0) * stride;  // split s0 stands in past the end
            ms[i] = r[D];
            ls[i] = r[D + 1];
            os[i] = r[c];
            if (!in) ms[i] = -INFINITY;
        }
        float Mc = M;
#pragma unroll
        for (int i = 0; i < CH; ++i) Mc = fmaxf(Mc, ms[i]);
        if (M != -INFINITY && Mc != M) {
            const float f = __builtin_amdgcn_exp2f(M - Mc);
            L *= f;
            O *= f;
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (ms[i] != -INFINITY) {
                const float f = __builtin_amdgcn_exp2f(ms[i] - Mc);
                L = fmaf(ls[i], f, L);
                O = fmaf(os[i], f, O);
            }
        }
        M = Mc;
    }
    a.out[row * D + c] = O / L;
}

// Merges the splits after an attention kernel wrote them (n_split > 1).
template <int D>
hipError_t merge_splits(hipError_t e, const AttendArgs& a, hipStream_t s) {
    if (e != hipSuccess || a.n_split == 1) return e;
    const dim3 grid((unsigned)((int64_t)a.g.batch * a.g.n_q_heads));
    if (a.rows.n)
        combine_kernel<D, true><<<grid, D, 0, s>>>(a);
    else
        combine_kernel<D, false><<<grid, D, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int BITS, int QG, int NWAVES>
hipError_t attend_launch(const AttendArgs& a, hipStream_t s) {
    const int group = a.g.n_q_heads / a.g.n_kv_heads;
    const dim3 grid((unsigned)a.n_split, (unsigned)((int64_t)a.g.batch * a.g.n_kv_heads), (unsigned)(group / QG));
    if (a.rows.n)
        attend_kernel<D, BITS, QG, NWAVES, true><<<grid, 64 * NWAVES, 0, s>>>(a);
    else
        attend_kernel<D, BITS, QG, NWAVES, false><<<grid, 64 * NWAVES, 0, s>>>(a);
    return merge_splits<D>(hipGetLastError(), a, s);
}

template <int D, int BITS>
hipError_t attend_db(const AttendArgs& a, hipStream_t s) {
    // the host plans (qg, nwaves) with the same attend_waves()
    switch (a.qg) {
        case 4:
            if constexpr (D == 128) return merge_splits<D>(launch_attend_gqa(a, s), a, s);
            else return attend_launch<D, BITS, 4, attend_waves(4, D)>(a, s);
        case 2: return attend_launch<D, BITS, 2, attend_waves(2, D)>(a, s);
        default: return attend_launch<D, BITS, 1, attend_waves(1, D)>(a, s);
    }
}

template <int D>
hipError_t attend_d(const AttendArgs& a, hipStream_t s) {
    static_assert(Rec<D, 2>::bytes == 2 * kG * D * 2 / 32 * 4 + D * 8 + kG * (D / kVG) * 8, "record layout");
    return a.g.bits == 2 ? attend_db<D, 2>(a, s) : attend_db<D, 4>(a, s);
}

// Split partials of kivi_attend_decode_noalloc: device memory the library
// brings itself, for callers that cannot allocate. Each GPU the library runs
// on holds its own copy until the process ends; every call on a GPU shares it.
static __device__ __align__(256) uint8_t scratch[KIVI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

}  // namespace

// In host code `scratch` names a host-side stand-in, not device memory: the
// device copy's address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and is the only form passed to kernels.
hipError_t static_scratch(void** ptr) {
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

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
