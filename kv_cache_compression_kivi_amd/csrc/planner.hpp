// planner.hpp -- host-side layout and scheduling of the KIVI cache.
//
// Pure C++ (no HIP): validation of a kivi_config, the device-memory layout,
// and the bookkeeping of the fp16 residual ring (which tokens a call
// quantizes, which it copies into the ring), plus the split-K plan of the
// decode attention. Everything here runs on the host before any launch.
//
// Ring semantics follow the KIVI explainer page ("ICML 2024論文解説: KIVI"),
// section 残差バッファ（Residual Buffer） and section Per-Token量子化（Value Cache）:
// the newest tokens stay fp16 and a whole group of G tokens is quantized once
// it leaves the newest R. Reading used here: a ring of R + G slots; a token
// arriving at a full ring first quantizes the oldest G residual tokens; an
// explicit flush quantizes floor((n_res - R) / G) * G of them. The closed forms
// below give the same counters as that token-by-token rule.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "kivi.h"
#include "split.hpp"

namespace kivi {

constexpr int32_t kDefaultMaxSplits = 256;
// Compute units assumed when no device can be asked (an MI355X has 256).
constexpr int32_t kDefaultCUs = 256;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Returns KIVI_OK or an error code with a message in `err`.
inline int validate_config(const kivi_config* c, std::string& err) {
    if (!c) { err = "config is NULL"; return KIVI_E_INVAL; }
    if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->max_tokens < 1) {
        err = "batch, n_kv_heads, n_q_heads and max_tokens must be >= 1";
        return KIVI_E_INVAL;
    }
    if (c->n_q_heads % c->n_kv_heads != 0) {
        err = "n_q_heads must be a multiple of n_kv_heads";
        return KIVI_E_INVAL;
    }
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) {
        err = "head_dim must be 64, 128 or 256";
        return KIVI_E_UNSUPPORTED;
    }
    if (c->bits != 2 && c->bits != 4) { err = "bits must be 2 or 4"; return KIVI_E_UNSUPPORTED; }
    if (c->k_block != 32 || c->v_group != 32) {
        err = "k_block and v_group must be 32";
        return KIVI_E_UNSUPPORTED;
    }
    if (c->residual < 0 || c->residual % c->k_block != 0) {
        err = "residual must be a non-negative multiple of k_block";
        return KIVI_E_INVAL;
    }
    if (c->max_splits != 0 && (c->max_splits < 2 || c->max_splits > 4096)) {
        err = "max_splits must be 0 or in [2, 4096]";
        return KIVI_E_INVAL;
    }
    // units index grid dimension y of the launches (at most 65535)
    int64_t units = (int64_t)c->batch * c->n_kv_heads;
    if (units > 65535 || (int64_t)c->batch * c->n_q_heads > ((int64_t)1 << 30)) {
        err = "batch * n_kv_heads must be <= 65535";
        return KIVI_E_INVAL;
    }
    // the attention kernel addresses one sequence's key-block records as one
    // buffer with 32-bit offsets
    if (c->n_pages < 0) {
        err = "n_pages must be >= 0";
        return KIVI_E_INVAL;
    }
    if (c->squat_rank < 0) {
        err = "squat_rank must be >= 0";
        return KIVI_E_INVAL;
    }
    if (c->squat_rank > 0 && (c->head_dim > 128 || c->squat_rank > 32 || c->squat_rank > c->head_dim)) {
        err = "the SQuat-style key coder needs head_dim 64 or 128 and squat_rank <= min(32, head_dim)";
        return KIVI_E_UNSUPPORTED;
    }
    const int64_t W = (int64_t)c->head_dim * c->bits / 32;
    const int64_t block_bytes = 2 * 32 * W * 4 + (int64_t)c->head_dim * 8 + 32 * (c->head_dim / 32) * 8;
    if ((int64_t)(c->max_tokens / c->k_block) * block_bytes > (int64_t)0xffffffff) {
        err = "max_tokens too large: one sequence's quantized blocks must fit in 4 GiB";
        return KIVI_E_UNSUPPORTED;
    }
    return KIVI_OK;
}

inline void compute_layout(const kivi_config* c, kivi_layout* L) {
    const size_t d = (size_t)c->head_dim, G = (size_t)c->k_block;
    const size_t W = d * (size_t)c->bits / 32;
    const int64_t units = (int64_t)c->batch * c->n_kv_heads;
    L->rec_kcode = 0;
    L->rec_vcode = G * W * 4;
    L->rec_ksz = L->rec_vcode + G * W * 4;
    L->rec_vsz = L->rec_ksz + d * 8;
    L->block_bytes = L->rec_vsz + G * (d / (size_t)c->v_group) * 8;
    L->max_blocks = c->max_tokens / c->k_block;
    L->off_blocks = 0;
    L->n_pages = c->n_pages;
    size_t blocks_bytes;
    if (c->n_pages > 0) {  // a pool of pages, each one block of every KV head of a sequence
        L->unit_stride = 0;
        L->page_bytes = (size_t)c->n_kv_heads * L->block_bytes;
        blocks_bytes = (size_t)c->n_pages * L->page_bytes;
    } else {
        L->unit_stride = align_up((size_t)L->max_blocks * L->block_bytes);
        L->page_bytes = 0;
        blocks_bytes = (size_t)units * L->unit_stride;
    }
    L->ring_slots = (int64_t)c->residual + c->k_block;
    L->off_ring = align_up(L->off_blocks + blocks_bytes);
    L->ring_unit_stride = align_up((size_t)L->ring_slots * 4 * d);
    L->off_partial = align_up(L->off_ring + (size_t)units * L->ring_unit_stride);
    L->max_splits = c->max_splits ? c->max_splits : kDefaultMaxSplits;
    L->partial_stride = (d + 4) * 4;
    L->off_squat = align_up(L->off_partial + (size_t)c->batch * c->n_q_heads * (size_t)L->max_splits *
                                                 L->partial_stride);
    L->squat_r8 = (c->squat_rank + 7) / 8 * 8;
    L->squat_unit_bytes = (size_t)2 * d * (size_t)L->squat_r8 * 4;
    L->total_bytes = L->off_squat + align_up((size_t)units * L->squat_unit_bytes);
}

// What one kivi_append(ntok) does, as closed forms of the token-by-token rule.
struct AppendPlan {
    int64_t nt0, nq0;   // counters before
    int64_t nt1, nq1;   // counters after
    int64_t ring_t0;    // tokens [ring_t0, nt1) are copied into the ring
};

inline AppendPlan plan_append(int64_t nt, int64_t nq, int64_t ntok, int64_t R, int64_t G) {
    const int64_t C = R + G;
    const int64_t total = (nt - nq) + ntok;  // residual tokens if nothing were flushed
    // each implicit flush removes G tokens and happens only while the ring is full,
    // so the count is the fewest flushes that bring the residual back to <= C
    const int64_t flushes = total > C ? (total - C + G - 1) / G : 0;
    AppendPlan p;
    p.nt0 = nt;
    p.nq0 = nq;
    p.nt1 = nt + ntok;
    p.nq1 = nq + flushes * G;
    p.ring_t0 = p.nq1 > nt ? p.nq1 : nt;
    return p;
}

// Tokens an explicit flush quantizes.
inline int64_t plan_flush(int64_t nt, int64_t nq, int64_t R, int64_t G) {
    const int64_t n_res = nt - nq;
    return n_res < R ? 0 : ((n_res - R) / G) * G;
}

struct AttendPlan {
    int32_t n_split;          // work-groups per (unit, query chunk) along the tokens
    int32_t blocks_per_split; // key blocks per split, about (informational)
    int32_t qg;               // query heads per work-group
    int32_t nwaves;           // waves per work-group
};

// Query heads per work-group: the largest of 4, 2, 1 dividing the GQA group
// (the kernel keeps qg x 16 accumulators per lane); waves per work-group from
// attend_waves(), which the kernel's dispatch uses too.
inline void attend_shape(int32_t group, int32_t head_dim, int32_t* qg, int32_t* nwaves) {
    *qg = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
    *nwaves = attend_waves(*qg, head_dim);
}

// Waves per CU the split plans aim for: one 8-wave work-group or two 4-wave
// ones on every compute unit.
constexpr int64_t kWavesPerCU = 8;

// Split-K plan. Enough work-groups for 8 waves on each of the device's `cus`
// compute units (one 8-wave work-group or two 4-wave ones per CU), at least 2
// key blocks per wave in every split, at most max_splits partials per query
// head; no split (and no merge launch) when the units alone fill the chip.
// forced > 0 fixes the split count instead.
inline AttendPlan plan_attend(int64_t units, int32_t group, int32_t head_dim, int64_t n_blocks,
                              int32_t max_splits, int32_t forced, int32_t cus) {
    AttendPlan p;
    attend_shape(group, head_dim, &p.qg, &p.nwaves);
    const int64_t wgs_per_split = units * (group / p.qg);
    int64_t n;
    if (forced > 0) {
        n = forced;
    } else {
        const int64_t target_waves = (int64_t)(cus > 0 ? cus : 1) * kWavesPerCU;
        n = (target_waves + wgs_per_split * p.nwaves - 1) / (wgs_per_split * p.nwaves);
        const int64_t cap = n_blocks / (2 * p.nwaves);
        if (n > cap) n = cap;
    }
    if (n > max_splits) n = max_splits;
    if (n < 1) n = 1;
    p.n_split = (int32_t)n;
    p.blocks_per_split = (int32_t)((n_blocks + n - 1) / n);
    return p;
}

// Split plan of a batch whose rows differ in length (cost[r]: unit_cost of
// row r; nb_max: the longest row's key blocks). n is the split count of the
// costliest row and each row takes its share (row_split_count), so that the
// work-groups carry about equal work. n is the largest count whose work-groups
// still fit one round over the `cus` CUs (as for rows that agree: 8 waves a CU), at
// least 1: then every work-group starts at once, and the costliest rows'
// work-groups, dispatched first, pair with short ones on their CUs (measured
// on MI355X: more splits, with a second round of work-groups and the merge,
// were 15-40% slower on a 64-row serving batch). At least 2 key blocks per
// wave in the costliest row's splits, at most max_splits; forced > 0 fixes n.
inline AttendPlan plan_attend_rows(int64_t n_kv_heads, int32_t group, int32_t head_dim, int64_t rows,
                                   const int64_t* cost, int64_t nb_max, int32_t max_splits, int32_t forced,
                                   int32_t cus, int64_t* cost_max) {
    AttendPlan p;
    attend_shape(group, head_dim, &p.qg, &p.nwaves);
    p.nwaves = attend_waves_rows(p.qg, head_dim);
    const int64_t wgs_per_row = n_kv_heads * (group / p.qg);  // work-groups of one split of one row
    int64_t cmax = 1;
    for (int64_t r = 0; r < rows; ++r) cmax = cost[r] > cmax ? cost[r] : cmax;
    auto wgs = [&](int64_t n) {
        int64_t w = 0;
        for (int64_t r = 0; r < rows; ++r) w += row_split_count(cost[r], cmax, n);
        return w * wgs_per_row;
    };
    int64_t n;
    if (forced > 0) {
        n = forced;
    } else {
        const int64_t target_wgs = (int64_t)(cus > 0 ? cus : 1) * kWavesPerCU / p.nwaves;
        int64_t hi = nb_max / (2 * p.nwaves);
        if (hi > max_splits) hi = max_splits;
        // the largest n in [1, hi] with wgs(n) <= target (wgs grows with n)
        n = 1;
        while (n < hi) {
            const int64_t mid = (n + hi + 1) / 2;
            if (wgs(mid) <= target_wgs) n = mid;
            else hi = mid - 1;
        }
    }
    if (n > max_splits) n = max_splits;
    if (n < 1) n = 1;
    p.n_split = (int32_t)n;
    p.blocks_per_split = (int32_t)((nb_max + n - 1) / n);
    *cost_max = cmax;
    return p;
}

}  // namespace kivi
