// launch.hpp -- arguments of the gfx950 kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kivi {

// Geometry shared by every kernel of one cache.
struct CacheGeom {
    uint8_t* base;            // start of the cache memory
    size_t off_blocks, unit_stride, block_bytes;
    size_t rec_kcode, rec_vcode, rec_ksz, rec_vsz;
    size_t off_ring, ring_unit_stride;
    int64_t ring_slots;
    size_t off_partial, partial_stride;  // partial_stride in bytes
    int32_t max_splits;
    int32_t batch, n_kv_heads, n_q_heads, head_dim, bits;
};

// Quantize key blocks [j0, j1) of every unit. Token t of a block comes from
// the ring when t < ring_end, else from input row t - ring_end of k / v
// ([units][ntok][d] fp16).
struct QuantArgs {
    CacheGeom g;
    int64_t j0, j1;
    int64_t ring_end;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ntok;
};

// Copy tokens [t0, t1) of every unit from input rows (t - in_t0) into the ring.
struct RingArgs {
    CacheGeom g;
    int64_t t0, t1, in_t0;
    const uint16_t* k;
    const uint16_t* v;
    int64_t ntok;
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
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_ring_write(const RingArgs& a, hipStream_t s);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace kivi
