// attend_gqa.hip -- decode attention for four query heads per KV head
// (grouped-query attention) at d = 128, on the gfx950 matrix cores.
//
// It computes what attend_kernel computes (the KIVI explainer page ("ICML
// 2024論文解説: KIVI — チューニング不要のKVキャッシュ2bit非対称量子化"), section
// 残差バッファ（Residual Buffer）: one softmax of q . [D(K_quant); K_res]^T /
// sqrt(d) over every token, applied to [D(V_quant); V_res]; section
// 量子化アルゴリズム: D(x) = s x + z), for the four query heads that share a KV
// head, so a block record is read once for all four.
//
// With four query heads per KV head both contractions of a block are small
// matrix products, and they run exactly on the int8 matrix cores:
//   scores  S[g][t] = sum_c q~[g][c] kcode[t][c]   (q~ = q s, per block and channel)
//   values  O[g][c] = sum_t p~[g][t] vcode[t][c]   (p~ = p s_t, per token and value group)
// The codes are int8 operands as they are. q~ and p~ are rounded to 23-bit
// integers against powers of two (|q| < 2^Eq per query and s < 2^Es per
// block for q~; for p~, p <= 1 and a running bound 2^ew on s_t, within 2^2 of
// the block's own) and split into three signed 8-bit digits, so every product
// and sum is exact in int32; the only rounding is that of q~ and p~ to 2^-22
// of their bounds. The digits of query (or weight)
// row g sit in rows 4g .. 4g + 2 of a 16-row tile operand; row 4g + 3 is never
// written: its products land in result row 4g + 3, which is never read.
// Scores: v_mfma_i32_16x16x64_i8, 16 rows (query, digit) x 16 tokens x 64
// channels, so a lane's four results are the digit sums of one query and one
// token (lane / 16 and lane % 16).
// Values: v_mfma_i32_16x16x32_i8, 16 rows x 16 channels x the block's 32 tokens,
// accumulated in int32 from block to block and folded into fp32 only when
// the running maximum or the weights' bound moves.
// The fp16 residual runs on the vector units as in attend_kernel.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "attend_common.hpp"
#include "split.hpp"

namespace kivi {
namespace {

// One lane's shares of a block record, read from its LDS slot before the block's math.
template <int D, int BITS>
struct GqaRegs {
    static constexpr int KC = D / 64;  // 64-channel chunks
    static constexpr int KW = BITS / 2;
    static constexpr int VT = D / 16;  // 16-channel value tiles
    uint32_t kc[2][KC][KW];            // key words of score column l%16 of tile tt, lane group l/16 of each chunk
    float ksz[KC][4][2];               // (s, z) of the digit producer's channels
    float2 vsz[2][4];                  // (s, z) of the tokens of columns 4((l%16)/4) + r, value group l%4
    uint32_t vc[VT];                   // value word of channel 16 vt + l%16 used by lane group l/16
};

// Bytes d of four words, as one word (byte k from word k).
__device__ __forceinline__ uint32_t bytes_d(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, int d) {
    const uint32_t lo = __builtin_amdgcn_perm(v1, v0, (uint32_t)(d | (4 + d) << 8 | 0x0c << 16 | 0x0c << 24));
    const uint32_t hi = __builtin_amdgcn_perm(v3, v2, (uint32_t)(0x0c | 0x0c << 8 | d << 16 | (4 + d) << 24));
    return lo | hi;
}

// The three digit words of four values: word d holds byte d of v0 .. v3
// (byte k from v_k). Bytes 0 and 1 go through two pair words, byte 2 directly.
__device__ __forceinline__ void digit_words(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3, uint32_t (&w)[3]) {
    constexpr uint32_t kPair = 0 | 4 << 8 | 1 << 16 | 5 << 24;  // [a.b0, b.b0, a.b1, b.b1]
    const uint32_t p01 = __builtin_amdgcn_perm(v1, v0, kPair);
    const uint32_t p23 = __builtin_amdgcn_perm(v3, v2, kPair);
    w[0] = __builtin_amdgcn_perm(p23, p01, 0 | 1 << 8 | 4 << 16 | 5 << 24);
    w[1] = __builtin_amdgcn_perm(p23, p01, 2 | 3 << 8 | 6 << 16 | 7 << 24);
    w[2] = bytes_d(v0, v1, v2, v3, 2);
}

// d0 + 2^8 d1 + 2^16 d2 of three int32 digit sums (the matrix cores' results:
// read them only from compiled code, which waits out the result hazard).
__device__ __forceinline__ int digit_sum3(int d0, int d1, int d2) { return (d2 << 16) + ((d1 << 8) + d0); }

// quad_perm broadcasts of lane k of each quad
constexpr int kQuadBcast[4] = {0x00, 0x55, 0xAA, 0xFF};

// Staging of the four-query kernel's blocks: each wave streams its next
// blocks from HBM straight into a ring of LDS slots (buffer loads with the LDS
// bit, a record copied as it is, 16 bytes per lane per load), so the blocks in
// flight hold no registers. The loads are asm, so the compiler tracks none of
// them: each slot is read after an explicit s_waitcnt vmcnt(N), N the staging
// loads issued after it (vector-memory loads retire in order; loads the
// compiler issues later only make the wait stricter), and a slot is refilled
// after an s_waitcnt lgkmcnt(0), once its reads have returned. M0 holds the
// LDS destination of each load (one SALU write and a wait state before it);
// nothing else in this kernel keeps a value in M0.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ uint32_t lds_address(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int NL>
__device__ __forceinline__ void stage_record(__amdgpu_buffer_rsrc_t rs, uint32_t soff, uint32_t slot, uint32_t voff) {
    const int so = __builtin_amdgcn_readfirstlane((int)soff);
    const uint32_t m = __builtin_amdgcn_readfirstlane(slot);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int c = 0; c < NL; ++c)
        asm volatile(
            "s_mov_b32 m0, %[m]\n\t"
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %[v], %[rs], %[so] offen nt lds"
            :
            : [m] "s"(m + 1024u * c), [v] "v"(voff + 1024u * c), [rs] "s"(rs), [so] "s"(so)
            : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%[n])" : : [n] "i"(N) : "memory");
}

// Waits until the staged block with `later` staged blocks after it has landed.
template <int NL, int NS>
__device__ __forceinline__ void wait_staged(int later) {
    static_assert(NS >= 1 && NS <= 3, "two later stages at most");
    if (NS > 2 && later >= 2) wait_vmem<2 * NL>();
    else if (NS > 1 && later >= 1) wait_vmem<NL>();
    else wait_vmem<0>();
}

// Issue priority by the blocks a wave has left. A SIMD issues from its oldest
// wave first, so of the two work-groups that share a CU the one dispatched
// first runs ahead, and the other ends alone at half the CU's memory
// parallelism (measured on MI355X: in every CU the later work-group took
// 14-23 us longer). Near its end a wave steps its priority down, so the
// waves of the other work-group, which have more blocks left, catch up.
__device__ __forceinline__ void take_turn(int left) {
    if (left >= 12) __builtin_amdgcn_s_setprio(3);
    else if (left >= 8) __builtin_amdgcn_s_setprio(2);
    else if (left >= 4) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// Two 4-wave work-groups per CU (up to 256 VGPRs a lane: the value digit
// sums stay in matrix-core accumulators across blocks).
template <int D, int BITS, int NWAVES, bool RAGGED>
__global__ __launch_bounds__(64 * NWAVES, 8 / NWAVES) void attend_gqa_kernel(const AttendArgs a) {
    constexpr int QG = 4;
    using B = BlockRegs<D, BITS>;
    using R = GqaRegs<D, BITS>;
    using L = Rec<D, BITS>;
    constexpr int NW = B::NW, TL = B::TL, TPL = B::TPL, CPV = B::CPV, KC = R::KC, VT = R::VT;
    constexpr int NG = D / kVG;
    static_assert(NG == 4 && CPV == 2, "the four lanes of a quad take the four value groups");
    constexpr int NACC = 2;
    constexpr int NT = 64 * NWAVES;
    __shared__ __align__(16) float s_q[QG][D];
    __shared__ __align__(16) float s_p[NWAVES][QG][kG];  // residual weights
    __shared__ float s_m[NWAVES][QG], s_l[NWAVES][QG], s_z[NWAVES][QG][NG];

    const CacheGeom& g = a.g;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // vector layout (residual): key rows of tokens tl + TL*i, column w; value channels cv0, cv0 + 1
    const int w = lane % NW, tl = lane / NW;
    const int cv0 = lane * CPV;
    // matrix layout: n = column (scores) / row (values) / channel in a tile, rho = lane group
    const int n = lane & 15, rho = lane >> 4;
    const int gl = n >> 2, dq = n & 3;  // the query of score columns 4gl .. 4gl+3, and a value group
    const int group = g.n_q_heads / g.n_kv_heads;
    // (split, unit, chunk of four query heads) of this work-group: with one
    // chunk per KV head, blockIdx = (split, unit). With zc > 1 chunks the grid
    // is flat and the zc chunks of one (split, unit), which read the same key
    // blocks, take ids 8 apart: work-groups go to the 8 XCDs in turn, so
    // they run on one XCD at about the same time, and the later ones find the
    // blocks in its L2 instead of HBM (padding ids past the last pair exit).
    const int zc = group / QG;
    int split, zq;
    int64_t uy;
    if (zc == 1) {
        split = blockIdx.x;
        uy = blockIdx.y;
        zq = 0;
    } else {
        const int64_t id = blockIdx.x, per = 8 * (int64_t)zc;
        const int64_t pair = 8 * (id / per) + id % 8;
        if (pair >= (int64_t)a.n_split * g.batch * g.n_kv_heads) return;
        zq = (int)(id % per / 8);
        split = (int)(pair % a.n_split);
        uy = pair / a.n_split;
    }
    const int64_t u = dispatch_unit<RAGGED>(a, uy);
    const int64_t b = u / g.n_kv_heads;
    const int h = (int)(u % g.n_kv_heads);
    const size_t row0 = (size_t)b * g.n_q_heads + (size_t)h * group + (size_t)zq * QG;
    const float scale = a.scale_log2;

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
    const int j0 = __builtin_amdgcn_readfirstlane((int)b0 + wave);
    const int j1 = __builtin_amdgcn_readfirstlane((int)b1);

    const uint8_t* ubase = g.base + g.off_blocks + (size_t)u * g.unit_stride;
    const __amdgpu_buffer_rsrc_t rs = records(ubase, (uint64_t)cnt.n_blocks * L::bytes);
    // per-lane byte offsets of the block shares: a base per share plus
    // compile-time steps (which become the loads' immediate offsets)
    const int rt = gqa_row_token<BITS>(n);       // token of score column n in its tile
    const int ob_kw = (rt * L::W + (BITS == 2 ? rho : 2 * rho)) * 4;
    const int ob_vc = L::vcode + (n * BITS + (BITS == 2 ? rho / 2 : rho)) * 4;
    auto kw_off = [&](int tt, int kc) { return ob_kw + (16 * tt * L::W + (BITS == 2 ? 4 : 8) * kc) * 4; };
    // Key (s, z): the lane's k-th pair is that of byte k' = (k + kq) mod 4 of
    // the digit word it produces (kq = n >> 2, the word's lane group), so the
    // 16 lanes of a 64-bit LDS read hit 32 distinct banks (in byte order they
    // would share 8); the digit words are rotated back by kq bytes before
    // they are stored.
    const int kq = n >> 2;
    constexpr int KS_STEP = gqa_channel<BITS>(0, 0, 1) * 8;  // bytes from the pair of byte k to that of k + 1
    const int ks_a = L::ksz + (gqa_channel<BITS>(0, kq, 4 * (n & 3)) + gqa_channel<BITS>(0, 0, kq)) * 8;
    const int ks_b = ks_a - 4 * KS_STEP;  // where k + kq wraps past byte 3
    auto ks_off = [&](int kc, int k) {
        return (k + kq >= 4 ? ks_b : ks_a) + KS_STEP * k + gqa_channel<BITS>(kc, 0, 0) * 8;
    };
    auto vs_off = [&](int tt, int r) {
        return L::vsz + ((16 * tt + gqa_row_token<BITS>(4 * gl + r)) * NG + dq) * 8;
    };
    // staged blocks: NS slots per wave (two 4-wave work-groups per CU, set by
    // registers; measured on MI355X: no faster with 4 slots)
    constexpr int NS = 3;
    constexpr int NL = L::bytes / 1024;  // staging loads per block
    static_assert(L::bytes % 1024 == 0, "a record is a whole number of 1 KB wave loads");
    __shared__ __align__(16) uint8_t s_stage[NWAVES][NS][L::bytes];
    const uint32_t stage_lds = lds_address(s_stage[wave][0]);
    // The matrix operands of the block being computed live in the slot it was
    // read from (its next load goes out after the block's math): score
    // operands [chunk][lane group][row][word] in the first 2 KB, weight
    // operands [group][lane group][row][word] in the next 2 KB. Rows are
    // XOR-swizzled by lane group (scores) or by group and lane group
    // (weights), so that a wave's stores, lanes spread over lane group and
    // row, hit distinct banks (32 or 64), and each lane's 16-byte (8-byte)
    // operand read stays contiguous.
    static_assert(KC * 4 * 64 * 4 + NG * 4 * 16 * 2 * 4 <= L::bytes, "the operands fit in one slot");
    auto kb_at = [&](int k, int kc, int q, int row, int wd) -> uint32_t& {
        return reinterpret_cast<uint32_t*>(s_stage[wave][k])[(kc * 4 + q) * 64 + ((row * 4 + wd) ^ (q * 4))];
    };
    auto va_at = [&](int k, int gr, int q, int row, int wd) -> uint32_t& {
        return reinterpret_cast<uint32_t*>(
            s_stage[wave][k])[KC * 4 * 64 + gr * 128 + (((q * 16 + row) * 2 + wd) ^ (gr * 2) ^ ((q & 1) << 4))];
    };
    // a wave's output rows at the end, in its first slot (no staging load is in flight then)
    auto s_o = [&](int wv) { return reinterpret_cast<float(*)[D]>(&s_stage[wv][0][0]); };
    static_assert(QG * D * 4 <= L::bytes, "the output rows fit in one slot");
    // paged blocks (built with a row table): the block's own page. A wave
    // stages its blocks in order, j0, j0 + NWAVES, ...: each block's table
    // entry was read one call earlier, and the call reads the next one.
    int32_t pg_next = 0;
    if constexpr (RAGGED)
        if (g.table && j0 < j1) pg_next = table_entry(g, b, j0);
    auto stage = [&](int j, int k) {
        if constexpr (RAGGED) {
            if (g.table) {
                const int32_t p = pg_next;
                if (j + NWAVES < j1) pg_next = table_entry(g, b, j + NWAVES);
                stage_record<NL>(records(g.base + page_offset(g, p, h), L::bytes), 0u, stage_lds + k * L::bytes,
                                 16u * lane);
                return;
            }
        }
        stage_record<NL>(rs, (uint32_t)j * L::bytes, stage_lds + k * L::bytes, 16u * lane);
    };
    // this lane's shares of a staged block
    auto read_slot = [&](int k, R& r) {
        const uint8_t* sb = s_stage[wave][k];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                if constexpr (BITS == 2) {
                    r.kc[tt][kc][0] = *reinterpret_cast<const uint32_t*>(sb + kw_off(tt, kc));
                } else {
                    const uint2 x = *reinterpret_cast<const uint2*>(sb + kw_off(tt, kc));
                    r.kc[tt][kc][0] = x.x;
                    r.kc[tt][kc][1] = x.y;
                }
            }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                const float2 x = *reinterpret_cast<const float2*>(sb + ks_off(kc, k2));
                r.ksz[kc][k2][0] = x.x;
                r.ksz[kc][k2][1] = x.y;
            }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) r.vsz[tt][rr] = *reinterpret_cast<const float2*>(sb + vs_off(tt, rr));
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) r.vc[vt] = *reinterpret_cast<const uint32_t*>(sb + ob_vc + 16 * vt * BITS * 4);
    };
    // the query first, while nothing else is in flight (its wait counts every
    // load issued before it), then the first blocks' staging loads
    for (int idx = threadIdx.x; idx < QG * D; idx += NT) {
        const uint16_t v = a.q[row0 * D + idx];
        s_q[idx / D][idx % D] = a.q_bf16 ? bf2f(v) : h2f(v);
    }
#pragma unroll
    for (int k = 0; k < NS; ++k)
        if (j0 + k * NWAVES < j1) stage(j0 + k * NWAVES, k);
    __syncthreads();
    // per-query bounds |q| < 2^Eq; the producer's query (rho) at its channels,
    // scaled to 2^22 of the bound (digits) and as it is (key zeros)
    int Eq[QG];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        uint32_t mx = 0;  // |q| as bit patterns
#pragma unroll
        for (int c = lane; c < D; c += 64) mx = umax(mx, __float_as_uint(s_q[gq][c]) & 0x7fffffffu);
        Eq[gq] = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(__uint_as_float(wave_max_bits(mx))));
    }
    const int eq_mine = rho == 0 ? Eq[0] : (rho == 1 ? Eq[1] : (rho == 2 ? Eq[2] : Eq[3]));
    float qn[KC][4], qv[KC][4];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float x = s_q[rho][gqa_channel<BITS>(kc, kq, 4 * (n & 3) + ((k + kq) & 3))];
            qn[kc][k] = ldexpf(x, 22 - eq_mine);
            qv[kc][k] = x;
        }

    // running state, two parts merged at the end. Residual (vector layout): m,
    // l_res and o_res per query. Blocks (matrix layout, query rho = lane / 16):
    // running max m_b, weight sum l_b of this lane's tokens, value-zero sum z_b
    // of group dq over the tokens of quad gl, o_blk[vt] (folded from acc_v) for
    // channel 16vt + n.
    float m[QG], l_res[QG], o_res[QG][CPV * NACC], o_blk[VT];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        m[gq] = -INFINITY;
        l_res[gq] = 0.f;
#pragma unroll
        for (int c = 0; c < CPV * NACC; ++c) o_res[gq][c] = 0.f;
    }
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) o_blk[vt] = 0.f;
    float m_b = -INFINITY, l_b = 0.f, z_b = 0.f;
    // value digit sums of the blocks since the last fold, per tile (rows 4 rho
    // + d), accumulated on the matrix cores; the weights' digits are taken
    // against 2^ew (ew wave-uniform, moved only at a fold)
    v4i32 acc_v[VT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) acc_v[vt] = v4i32{0, 0, 0, 0};
    int ew = INT_MIN / 2;
    // blocks added to acc_v since the last wave-wide fold: kGqaFoldBlocks
    // bounds it, so the int32 sums cannot overflow however long the wave's
    // share (a fold of some rows only, on a new maximum, leaves it counting;
    // it stays wave-uniform, in a scalar register)
    int since_fold = 0;
    // o_blk += 2^(ew - 22) sum_d 2^(8d) acc_v[d], then the sums restart
    auto fold = [&]() {
        const float vs = ldexpf(1.0f, ew - 22);
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const float comb = fmaf((float)acc_v[vt][2], 65536.0f, fmaf((float)acc_v[vt][1], 256.0f, (float)acc_v[vt][0]));
            o_blk[vt] = fmaf(comb, vs, o_blk[vt]);
            acc_v[vt] = v4i32{0, 0, 0, 0};
        }
    };
    // multiply the residual accumulators of query gq by alpha (a new running maximum)
    auto rescale = [&](int gq, float alpha) {
        l_res[gq] *= alpha;
#pragma unroll
        for (int c = 0; c < CPV * NACC; ++c) o_res[gq][c] *= alpha;
    };

    // residual chunks (vector units, as in attend_kernel): computed after the
    // key blocks, once no staging load is in flight, so that their loads (whose
    // waits count every earlier load) do not wait for the staged blocks, and
    // the kernel's first loads are the query and the staged blocks only
    const uint8_t* rbase = g.base + g.off_ring + (size_t)u * g.ring_unit_stride;
    const int ring = (int)g.ring_slots;
    const int slot0 = (int)(cnt.n_quant % g.ring_slots);
    if (cnt.t_new >= 0 && split == cnt.n_split - 1 && zq == 0 && wave == 0)
        write_new_token<D>(a, u, cnt.t_new, rbase);
    // scores, softmax, weight digits of one block
    auto key_math = [&](const R& r, int k_slot) {
        // 1. digits of the folded query: rint(q 2^(22-Eq) * s 2^-Es)
        uint32_t smax = 0;  // scales are positive: their bit patterns order like the values
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
            for (int k = 0; k < 4; ++k) smax = umax(smax, __float_as_uint(r.ksz[kc][k][0]));
        smax = row_max_bits(smax);  // each row of 16 lanes covers every channel
        const int es = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(__uint_as_float(smax)));
        const DigitScale dk = digit_scale(es);
        float zp = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint32_t vq[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vq[k] = digits3(qn[kc][k], r.ksz[kc][k][0], dk);
                zp = fmaf(qv[kc][k], r.ksz[kc][k][1], zp);
            }
            uint32_t wq[3];
            digit_words(vq[0], vq[1], vq[2], vq[3], wq);
#pragma unroll
            for (int d = 0; d < 3; ++d) kb_at(k_slot, kc, kq, 4 * rho + d, n & 3) = __builtin_rotateleft32(wq[d], 8 * kq);
        }
        // key zeros: Z = sum_c q[rho][c] z[c], summed over row rho (all its lanes hold it)
        const float zs = sum_cols<16>(zp) * scale;
        // bound of the block's value scales, for the weight digits
        uint32_t vmax = 0;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) vmax = umax(vmax, __float_as_uint(r.vsz[tt][r2].x));
        // each row of 16 lanes reads every (token, group) scale of the block once
        // (gqa_row_token is a permutation of a tile's 16 tokens; lane n reads
        // group n % 4 of the tokens of columns 4 (n / 4) .. 4 (n / 4) + 3)
        const int ev = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(__uint_as_float(row_max_bits(vmax))));
        // the weights' exponent follows the block's bound when it grows, or
        // when the bound falls more than 2 below it (at most 2 of the digits'
        // 22 bits left unused)
        if (ev > ew || ev < ew - 2) {
            fold();
            ew = ev;
            since_fold = 0;
        }
        wave_lds_order();
        // 2. scores of query rho and token rt of each tile: the digit sums of
        //    rows 4 rho .. 4 rho + 2 land in this lane's accumulators 0 .. 2
        const float ks = ldexpf(scale, eq_mine + es - 22);  // sum Q code = 2^(22 - Eq - Es) sum q s code
        float sc[2];
        // both tiles' products interleave on the matrix core; the digit
        // operand of a chunk serves both
        v4i32 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const uint4 bb = *reinterpret_cast<const uint4*>(&kb_at(k_slot, kc, rho, n, 0));
            v4i32 qd;
            qd[0] = (int)bb.x;
            qd[1] = (int)bb.y;
            qd[2] = (int)bb.z;
            qd[3] = (int)bb.w;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                v4i32 cv;
                if constexpr (BITS == 2) {
                    const uint32_t x = r.kc[tt][kc][0];
                    cv[0] = (int)(x & 0x03030303u);
                    cv[1] = (int)((x >> 2) & 0x03030303u);
                    cv[2] = (int)((x >> 4) & 0x03030303u);
                    cv[3] = (int)((x >> 6) & 0x03030303u);
                } else {
                    const uint32_t x0 = r.kc[tt][kc][0], x1 = r.kc[tt][kc][1];
                    cv[0] = (int)(x0 & 0x0F0F0F0Fu);
                    cv[1] = (int)((x0 >> 4) & 0x0F0F0F0Fu);
                    cv[2] = (int)(x1 & 0x0F0F0F0Fu);
                    cv[3] = (int)((x1 >> 4) & 0x0F0F0F0Fu);
                }
                acc[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qd, cv, acc[tt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float comb;
            if constexpr (BITS == 2) {
                // |sums| <= 128 * 3 * 128 (digits 0, 1) and 128 * 3 * 64 (digit 2): exact in int32
                comb = (float)digit_sum3(acc[tt][0], acc[tt][1], acc[tt][2]);
            } else {
                comb = fmaf((float)acc[tt][2], 65536.0f, fmaf((float)acc[tt][1], 256.0f, (float)acc[tt][0]));
            }
            sc[tt] = fmaf(comb, ks, zs);
        }
        // 3. online softmax of query rho over the row's 32 tokens
        float bm = fmaxf(sc[0], sc[1]);
        bm = fmaxf(bm, dpp<kSwap1>(bm));
        bm = fmaxf(bm, dpp<kSwap2>(bm));
        bm = fmaxf(bm, dpp<kHalfMirror>(bm));
        bm = fmaxf(bm, dpp<kMirror>(bm));
        if (bm > m_b) {
            const float alpha = __builtin_amdgcn_exp2f(m_b - bm);
            l_b *= alpha;
            z_b *= alpha;
            fold();
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) o_blk[vt] *= alpha;
            m_b = bm;
        }
        float pt[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            pt[tt] = __builtin_amdgcn_exp2f(sc[tt] - m_b);
            l_b += pt[tt];
        }
        const DigitScale dv = digit_scale(ew - 22);
        // 4. weights p s_t of value group dq for the tokens of quad gl (gathered
        //    from its four lanes), as digits: rows 4 rho + d of the value operand,
        //    one word per tile (lane group 2tt + gl/2, word gl%2)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float pq[4];
            pq[0] = dpp<kQuadBcast[0]>(pt[tt]);
            pq[1] = dpp<kQuadBcast[1]>(pt[tt]);
            pq[2] = dpp<kQuadBcast[2]>(pt[tt]);
            pq[3] = dpp<kQuadBcast[3]>(pt[tt]);
            uint32_t vp[4];
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) {
                z_b = fmaf(pq[r2], r.vsz[tt][r2].y, z_b);
                vp[r2] = digits3(pq[r2], r.vsz[tt][r2].x, dv);
            }
            uint32_t wp[3];
            digit_words(vp[0], vp[1], vp[2], vp[3], wp);
#pragma unroll
            for (int d = 0; d < 3; ++d)
                va_at(k_slot, dq, 2 * tt + gl / 2, 4 * rho + d, gl % 2) = wp[d];
        }
        wave_lds_order();
    };
    // values of one block: acc_v[vt] += sum_t P[g][t] code[t][c] (digit rows)
    auto value_math = [&](const R& r, int k_slot) {
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            const uint2 pa = *reinterpret_cast<const uint2*>(&va_at(k_slot, vt / 2, rho, n, 0));
            const uint32_t x = r.vc[vt];
            uint32_t b0, b1;
            if constexpr (BITS == 2) {
                const int sh = 4 * (rho % 2);  // tokens 2(q%2) + e of each quartet
                b0 = (x >> sh) & 0x03030303u;
                b1 = (x >> (sh + 2)) & 0x03030303u;
            } else {
                b0 = x & 0x0F0F0F0Fu;
                b1 = (x >> 4) & 0x0F0F0F0Fu;
            }
            const long av = (long)(((uint64_t)pa.y << 32) | pa.x);
            const long bv = (long)(((uint64_t)b1 << 32) | b0);
            acc_v[vt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, acc_v[vt], 0, 0, 0);
        }
        wave_lds_order();
    };
    // a block is read from its slot into registers, its math runs with the
    // matrix operands in that slot, and then the slot is refilled with the
    // block NS further on
    for (int j = j0; j < j1; j += NS * NWAVES) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {  // slot k: its address offsets are constants
            const int jj = j + k * NWAVES;
            if (jj >= j1) break;
            wait_staged<NL, NS>((j1 - 1 - jj) / NWAVES);
            R r;
            read_slot(k, r);
            wave_lds_order();  // the slot's reads stay before the operand stores into it
            key_math(r, k);
            value_math(r, k);
            if (++since_fold == (int)kGqaFoldBlocks) {
                fold();
                since_fold = 0;
            }
            if (jj + NS * NWAVES < j1) stage(jj + NS * NWAVES, k);
            take_turn((j1 - 1 - jj) / NWAVES);
        }
    }
    fold();

    for (int ck = NWAVES - 1 - wave; ck < rc; ck += NWAVES) {
        uint4 kraw[TPL][2];
        bool valid[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int idx = ck * kG + tl + TL * i;
            valid[i] = idx < (int)nres;
            const int ie = valid[i] ? idx : (int)nres - 1;  // past the end: the last token's row
            int slot = slot0 + ie;
            slot -= slot >= ring ? ring : 0;
            const uint4* kp = cnt.n_quant + ie == cnt.t_new
                                  ? reinterpret_cast<const uint4*>(a.k_new + u * D + 16 * w)
                                  : reinterpret_cast<const uint4*>(rbase + (size_t)slot * 4 * D + 32 * w);
            kraw[i][0] = kp[0];
            kraw[i][1] = kp[1];
        }
        uint32_t vr[kG];  // fp16 values of channels cv0, cv0 + 1, token t
#pragma unroll
        for (int t = 0; t < kG; ++t) {
            // tokens past the residual's end (weight 0) read the last token's
            // row, which is finite (the first residual slot is not written yet
            // when the new token is the only one)
            const int idx = ck * kG + t;
            const int ie = idx < (int)nres ? idx : (int)nres - 1;
            int slot = slot0 + ie;
            slot -= slot >= ring ? ring : 0;
            vr[t] = cnt.n_quant + ie == cnt.t_new
                        ? *reinterpret_cast<const uint32_t*>(a.v_new + u * D + cv0)
                        : *reinterpret_cast<const uint32_t*>(rbase + (size_t)slot * 4 * D + 2 * D + 2 * cv0);
        }
        float sc[QG][TPL];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float qq[16];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_q[gq][16 * w + 4 * c4]);
                qq[4 * c4] = x.x;
                qq[4 * c4 + 1] = x.y;
                qq[4 * c4 + 2] = x.z;
                qq[4 * c4 + 3] = x.w;
            }
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                const uint16_t* kh = reinterpret_cast<const uint16_t*>(kraw[i]);
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc = fmaf(qq[c], h2f(kh[c]), acc);
                acc = sum_cols<NW>(acc) * scale;
                sc[gq][i] = valid[i] ? acc : -INFINITY;
            }
        }
        float p[QG][TPL];
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float bm = sc[gq][0];
#pragma unroll
            for (int i = 1; i < TPL; ++i) bm = fmaxf(bm, sc[gq][i]);
            bm = tok_max<NW>(bm);
            if (bm > m[gq]) {
                rescale(gq, __builtin_amdgcn_exp2f(m[gq] - bm));
                m[gq] = bm;
            }
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                p[gq][i] = valid[i] ? __builtin_amdgcn_exp2f(sc[gq][i] - m[gq]) : 0.f;
                l_res[gq] += p[gq][i];
            }
        }
        if (w == 0) {
#pragma unroll
            for (int gq = 0; gq < QG; ++gq)
#pragma unroll
                for (int i = 0; i < TPL; ++i) s_p[wave][gq][tl + TL * i] = p[gq][i];
        }
        wave_lds_order();
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) {
            float pv[kG];
#pragma unroll
            for (int t4 = 0; t4 < kG / 4; ++t4) {
                const float4 x = *reinterpret_cast<const float4*>(&s_p[wave][gq][4 * t4]);
                pv[4 * t4] = x.x;
                pv[4 * t4 + 1] = x.y;
                pv[4 * t4 + 2] = x.z;
                pv[4 * t4 + 3] = x.w;
            }
#pragma unroll
            for (int t = 0; t < kG; ++t) {
                o_res[gq][t % NACC] = fmaf(pv[t], half_lo(vr[t]), o_res[gq][t % NACC]);
                o_res[gq][NACC + t % NACC] = fmaf(pv[t], half_hi(vr[t]), o_res[gq][NACC + t % NACC]);
            }
        }
        wave_lds_order();
    }

    // per-wave totals. Block part of query rho (row rho): its max m_b, weight
    // sum, value-zero sums of group dq; residual part per query: m, l_res, o_res
    const float lb = sum_cols<16>(l_b);
    float zb = z_b + dpp<kRor4>(z_b);
    zb += dpp<kRor8>(zb);  // over the quads of the row: (query rho, group dq)
    const float mr = rho == 0 ? m[0] : (rho == 1 ? m[1] : (rho == 2 ? m[2] : m[3]));
    const float mt = fmaxf(mr, m_b);  // this wave's max of query rho
    const float fb = m_b == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_b - mt);
    float mq[QG], fr[QG];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
        mq[gq] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mt), 16 * gq));
        fr[gq] = m[gq] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[gq] - mq[gq]);
    }
    float lq[QG];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
        lq[gq] = tok_sum<NW>(l_res[gq]) * fr[gq] +
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lb * fb), 16 * gq));
    if (gl == 0) s_z[wave][rho][dq] = zb * fb;
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
#pragma unroll
        for (int k = 0; k < CPV; ++k) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < NACC; ++e) acc += o_res[gq][k * NACC + e];
            s_o(wave)[gq][cv0 + k] = acc * fr[gq];
        }
    wave_lds_order();
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
        const int c = 16 * vt + n;
        s_o(wave)[rho][c] += fmaf(o_blk[vt], fb, s_z[wave][rho][c / kVG]);
    }
#pragma unroll
    for (int gq = 0; gq < QG; ++gq)
        if (lane == 0) {
            s_m[wave][gq] = mq[gq];
            s_l[wave][gq] = lq[gq];
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
                O = fmaf(s_o(wv)[gq][c], f, O);
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

// Rows that agree: two 4-wave work-groups per CU. With a row table (rows of
// different lengths, paged blocks): one 8-wave work-group per CU, so that a
// long row left running alone on its CU still has two waves per SIMD
// (measured on MI355X: 1.5% faster on a 64-row serving batch, 5% paged).
template <int BITS>
hipError_t gqa_launch(const AttendArgs& a, hipStream_t s) {
    constexpr int NW = attend_waves(4, 128);
    constexpr int NWR = attend_waves_rows(4, 128);
    const int zc = a.g.n_q_heads / a.g.n_kv_heads / 4;
    const int64_t units = (int64_t)a.g.batch * a.g.n_kv_heads;
    // one chunk of four query heads: (split, unit); more: flat, the chunks of a
    // (split, unit) 8 ids apart, the pairs padded to a multiple of 8
    const dim3 grid = zc == 1 ? dim3((unsigned)a.n_split, (unsigned)units, 1u)
                              : dim3((unsigned)(8 * (int64_t)zc * ((a.n_split * units + 7) / 8)), 1u, 1u);
    if (a.rows.n)
        attend_gqa_kernel<128, BITS, NWR, true><<<grid, 64 * NWR, 0, s>>>(a);
    else
        attend_gqa_kernel<128, BITS, NW, false><<<grid, 64 * NW, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_gqa(const AttendArgs& a, hipStream_t s) {
    return a.g.bits == 2 ? gqa_launch<2>(a, s) : gqa_launch<4>(a, s);
}

}  // namespace kivi
