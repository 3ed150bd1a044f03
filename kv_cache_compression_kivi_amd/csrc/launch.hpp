// launch.hpp -- arguments of the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "split.hpp"

namespace kivi {

// Geometry shared by every kernel of one cache.
struct CacheGeom {
    uint8_t* base;            // start of the cache memory
    size_t off_blocks, unit_stride, block_bytes;
    size_t rec_kcode, rec_vcode, rec_ksz, rec_vsz;
    size_t off_ring, ring_unit_stride;
    int64_t ring_slots;
    // split-K partials of (batch row, query head) r, split s at
    // partial + (r * partial_splits + s) * partial_stride (bytes): the cache's
    // partial region, or the library's static scratch (kivi_attend_decode_noalloc)
    uint8_t* partial;
    size_t partial_stride;
    int32_t partial_splits;
    int32_t batch, n_kv_heads, n_q_heads, head_dim, bits;
    // paged blocks: the caller's block table [batch][table_stride] of page
    // indices into a pool of n_pages pages (Hkv records each); null when each
    // unit has its own region
    const int32_t* table;
    int64_t table_stride;
    int32_t n_pages;
    // SQuat-style key coder: per unit U [head_dim][squat_r8] then W
    // [head_dim][squat_r8] fp32 at off_squat + u * 2 * head_dim * squat_r8 * 4
    size_t off_squat;
    int32_t squat_r8;
};

// Paged blocks: the table entry of batch row b's key block j, read through
// the scalar cache (the table is constant during a launch).
__device__ inline int32_t table_entry(const CacheGeom& g, int64_t b, int64_t j) {
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    return ((const_i32)g.table)[b * g.table_stride + j];
}

// Byte offset of KV head h's record in page p, the entry clamped into the pool.
__device__ inline size_t page_offset(const CacheGeom& g, int32_t p, int64_t h) {
    p = p < 0 ? 0 : (p >= g.n_pages ? g.n_pages - 1 : p);
    return g.off_blocks + ((size_t)p * g.n_kv_heads + (size_t)h) * g.block_bytes;
}

// Byte offset, from the cache memory's start, of unit u's key block j.
__device__ inline size_t record_offset(const CacheGeom& g, int64_t u, int64_t j) {
    if (g.table) return page_offset(g, table_entry(g, u / g.n_kv_heads, j), u % g.n_kv_heads);
    return g.off_blocks + (size_t)u * g.unit_stride + (size_t)j * g.block_bytes;
}

// Sequences of one batch may hold different numbers of tokens. A launch over
// such a batch carries one entry per batch row in a row table, passed with
// the kernel arguments (no device copy per call); n = 0 marks a batch whose
// rows all agree, and then the uniform fields of the arguments apply. Token
// counts of one sequence fit in 32 bits (its blocks fit in 4 GiB).
constexpr int kMaxRaggedRows = 128;

// Quantize key blocks [j0, j1) of every unit. Token t of a block comes from
// the ring when t < ring_end, else from input row t - ring_end of k / v
// ([units][ntok][d] fp16). With a row table, row b's units take
// [rows.j0[b], rows.j1[b]) and rows.ring_end[b], and j1 - j0 is the largest
// block count of a row (the grid).
struct QuantRows {
    int32_t n;
    int32_t j0[kMaxRaggedRows], j1[kMaxRaggedRows], ring_end[kMaxRaggedRows];
};
// With ring_wgs > 0 (rows that agree, and no quantized token read from the
// ring), the same launch also copies tokens [ring_t0, ring_t1) of every unit
// from input rows (t - ring_in_t0) into the ring: ring_wgs more work-groups
// per unit after the blocks' (x >= j1 - j0), 8 tokens each.
struct QuantArgs {
    CacheGeom g;
    int64_t j0, j1;
    int64_t ring_end;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ntok;
    int64_t ring_t0, ring_t1, ring_in_t0;
    int32_t ring_wgs;
    QuantRows rows;
};

// Copy tokens [t0, t1) of every unit from input rows (t - in_t0) into the ring.
// With a row table, row b's units copy [rows.t0[b], rows.t1[b]) from input
// rows (t - rows.in_t0[b]), and t1 - t0 is the largest count of a row.
struct RingRows {
    int32_t n;
    int32_t t0[kMaxRaggedRows], t1[kMaxRaggedRows], in_t0[kMaxRaggedRows];
};
struct RingArgs {
    CacheGeom g;
    int64_t t0, t1, in_t0;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ntok;
    RingRows rows;
};

struct AttendRows {
    int32_t n;
    int32_t n_tokens[kMaxRaggedRows], n_quant[kMaxRaggedRows], t_new[kMaxRaggedRows];
    int32_t order[kMaxRaggedRows];  // batch rows in dispatch order: costliest first
};

// Decode attention. Work-group (split s, unit u, query chunk z) covers the
// unit's key blocks [floor(s*C/n), floor((s+1)*C/n)) clipped to n_blocks,
// where C = n_blocks + (residual chunk cost) * (residual chunks) and
// n = n_split; the last split also takes the residual. qg query heads per
// work-group, nwaves waves per work-group.
struct AttendArgs {
    CacheGeom g;
    const uint16_t* q;
    int32_t q_bf16;
    float* out;
    int64_t n_tokens, n_quant, n_blocks;
    int32_t n_split;
    int32_t qg, nwaves;
    float scale_log2;  // log2(e) / sqrt(d)
    // A token appended by this call (t_new >= 0), not yet in the ring: its rows
    // are k_new / v_new + unit * d. One wave of the work-group that owns a
    // unit's residual writes them to their ring slot for later calls; this
    // call reads the token from those input rows, not from the ring.
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t t_new;
    // With a row table, row b holds rows.n_tokens[b] tokens, rows.n_quant[b]
    // of them quantized, and rows.t_new[b] (or -1) is its appended token;
    // n_blocks is then the largest row's block count, n_split the split count
    // of the costliest row (cost_max, in unit_cost terms), and row b takes
    // row_split_count(its cost, cost_max, n_split) splits.
    AttendRows rows;
    int64_t cost_max;
};

// The counters of batch row b for one attention launch, and its split count.
struct RowCounts {
    int64_t n_tokens, n_quant, n_blocks, t_new, n_split;
};
// The kernels are built twice: RAGGED for launches with a row table, and
// without it for batches whose rows agree, which then read only the uniform
// fields (no row-table read on the way to their first loads).

// The unit of grid row y: with a row table, the rows go out costliest first
// (their work-groups are dispatched in grid order), else unit y.
template <bool RAGGED>
__host__ __device__ inline int64_t dispatch_unit(const AttendArgs& a, int64_t y) {
    if constexpr (!RAGGED) return y;
    const int64_t hkv = a.g.n_kv_heads;
    return (int64_t)a.rows.order[y / hkv] * hkv + y % hkv;
}

template <bool RAGGED>
__host__ __device__ inline RowCounts row_counts(const AttendArgs& a, int64_t b) {
    RowCounts c;
    if constexpr (RAGGED) {
        c.n_tokens = a.rows.n_tokens[b];
        c.n_quant = a.rows.n_quant[b];
        c.t_new = a.rows.t_new[b];
        c.n_blocks = c.n_quant / 32;  // 32 tokens per key block
        c.n_split = row_split_count(unit_cost(c.n_blocks, c.n_tokens - c.n_quant), a.cost_max, a.n_split);
    } else {
        c.n_tokens = a.n_tokens;
        c.n_quant = a.n_quant;
        c.t_new = a.t_new;
        c.n_blocks = a.n_blocks;
        c.n_split = a.n_split;
    }
    return c;
}

// Largest query-subspace rank of the SQuat-style key coder.
constexpr int kSquatMaxRank = 32;

// Builds every unit's update coefficients from n_q past queries per query
// head (q: [B][Hq][n_q][head_dim] fp16 or bf16), rank-`rank` subspace, lambda.
struct SquatBuildArgs {
    CacheGeom g;
    const uint16_t* q;
    int32_t q_bf16;
    int64_t n_q;
    int32_t rank;
    float lambda;
};

// The library's static split-partial scratch on the current device
// (kivi_attend_decode_noalloc): its device address, looked up once per device.
hipError_t static_scratch(void** ptr);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_ring_write(const RingArgs& a, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
// SQuat-style key coder (head_dim 64 or 128): the coefficients (one work-group
// per unit), and the key codes of the blocks a QuantArgs launch just quantized
// (after it, before the ring write of the same call).
hipError_t launch_squat_build(const SquatBuildArgs& a, hipStream_t s);
hipError_t launch_squat_codes(const QuantArgs& a, hipStream_t s);

}  // namespace kivi
