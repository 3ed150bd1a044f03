// split.hpp -- how decode attention divides one unit's tokens among
// work-groups (splits) and among the waves of a work-group. Shared by the
// kernel and the host-side tests, so both use one definition.
//
// Work items are the unit's key blocks (G = 32 quantized tokens each) and its
// residual chunks (up to 32 fp16 tokens each). Splits are balanced by cost,
// and the residual goes to the last split.
#pragma once

#include <cstdint>

#ifdef __HIPCC__
#define KIVI_HD __host__ __device__
#else
#define KIVI_HD
#endif

namespace kivi {

// Cost of one residual chunk, in key blocks: a chunk of 32 fp16 tokens moves
// 16 KB (four 2-bit blocks at d = 128) but runs no decoding; measured on
// MI355X it takes about as long as 1.5 packed blocks at b = 2 or b = 4, and
// costs are whole blocks.
constexpr int64_t kResidualChunkCost = 2;

// Key blocks [*b0, *b1) of split s (of n) for a unit with nb key blocks and
// nrc residual chunks; the last split (which also owns the residual) ends at nb.
KIVI_HD inline void split_range(int64_t nb, int64_t nrc, int64_t cost, int64_t n, int64_t s, int64_t* b0,
                                int64_t* b1) {
    const int64_t total = nb + cost * nrc;
    const int64_t lo = s * total / n;
    const int64_t hi = (s + 1) * total / n;
    *b0 = lo < nb ? lo : nb;
    *b1 = s == n - 1 ? nb : (hi < nb ? hi : nb);
}

// Cost of a unit's attention work, in key blocks: nb key blocks and the
// residual's chunks of 32 tokens.
KIVI_HD inline int64_t unit_cost(int64_t nb, int64_t n_resid) { return nb + kResidualChunkCost * ((n_resid + 31) / 32); }

// Splits of one batch row when the rows differ in length: n splits for the
// costliest row (cost_max), and for a row of cost c the share of n its cost
// calls for, so that every split of every row holds about cost_max / n
// (rounded up, at least 1). Splits s >= this count of a row are idle.
KIVI_HD inline int64_t row_split_count(int64_t cost, int64_t cost_max, int64_t n) {
    const int64_t k = (n * cost + cost_max - 1) / cost_max;
    return k < 1 ? 1 : k;
}

// Inside a work-group of nw waves, wave w takes the split's key blocks
// b0 + w, b0 + w + nw, b0 + w + 2 nw, ... (round robin), so the waves sweep
// the split's records together, and residual chunk c goes to wave
// residual_wave(c, nw): the last waves first, which hold one block fewer
// whenever nw does not divide the split's block count.
KIVI_HD inline int64_t residual_wave(int64_t c, int64_t nw) { return nw - 1 - c % nw; }

// Waves per work-group of the attention kernel for qg query heads per
// work-group: 8, except 4 where a lane's registers allow two waves per SIMD
// at most (four query heads, on the matrix cores at d = 128 or the vector
// path otherwise; two query heads at d = 256). Two 4-wave work-groups then
// share a CU, so one's start overlaps the other's end (measured on MI355X:
// 2% faster than one 8-wave work-group for the four-query kernel).
KIVI_HD constexpr int attend_waves(int qg, int head_dim) {
    return qg == 4 ? 4 : (qg == 2 && head_dim > 128 ? 4 : 8);
}

// Waves per work-group of the attention kernels launched with a row table
// (rows of different lengths, paged blocks): 8 for the four-query kernel at
// d = 128 (one work-group per CU), else as attend_waves.
KIVI_HD constexpr int attend_waves_rows(int qg, int head_dim) {
    return qg == 4 && head_dim == 128 ? 8 : attend_waves(qg, head_dim);
}

// The four-query kernel keeps its value digit sums in int32 from block to
// block. One block adds at most 128 (a signed digit) * 15 (a 4-bit code) * 32
// (tokens) = 61440 to a sum in magnitude, so the sums are folded into fp32 at
// least every kGqaFoldBlocks blocks: 32768 * 61440 < 2^31.
constexpr int64_t kGqaFoldBlocks = 32768;
constexpr int64_t kGqaBlockDigitSumMax = 128 * 15 * 32;
static_assert(kGqaFoldBlocks * kGqaBlockDigitSumMax < (int64_t)1 << 31, "value digit sums stay in int32");

// Operand layouts of the four-query kernel (attend_gqa.hip), here so that the
// host-side tests can check them.
// Channel of byte s of a score operand, for lane group q of 64-channel chunk kc:
// masking a token's key word by (w >> b*j) & 0x0303..03 / 0x0F0F..0F gives one
// code per byte; these formulas follow that byte order.
template <int BITS>
KIVI_HD constexpr int gqa_channel(int kc, int q, int s) {
    if constexpr (BITS == 2) {
        return 64 * kc + 16 * q + 4 * (s % 4) + s / 4;  // word 4kc + q, s = 4j + k -> channel 4k + j
    } else {
        return 64 * kc + 16 * q + 8 * (s / 8) + 2 * (s % 4) + (s / 4) % 2;  // words 8kc + 2q + e, s = 8e + 4j + k
    }
}

// Token of byte s of a value operand, for lane group q: masking a channel's
// value word in the same way. b = 2: word q/2, bytes (w >> 2(2(q%2) + e)) ->
// tokens 16(q/2) + 4k + 2(q%2) + e (s = 4e + k); b = 4: word q, (w >> 4e) ->
// tokens 8q + 2k + e.
// Score columns are assigned to tokens so that the four lanes 4c .. 4c + 3 of
// a row (columns of one quad) hold exactly the tokens of bytes 4e .. 4e + 3 of
// one value operand (q = 2 tt + c/2, e = c % 2): their weights then pack into
// one word.
template <int BITS>
KIVI_HD constexpr int gqa_row_token(int m) {  // token (within its 16-token tile) of score column m
    if constexpr (BITS == 2) {
        return m / 4 + 4 * (m % 4);
    } else {
        return 8 * ((m / 4) / 2) + (m / 4) % 2 + 2 * (m % 4);
    }
}

// Key blocks wave w of nw holds out of nbw.
KIVI_HD inline int64_t wave_blocks(int64_t nbw, int64_t nw, int64_t w) { return nbw / nw + (w < nbw % nw ? 1 : 0); }

}  // namespace kivi
