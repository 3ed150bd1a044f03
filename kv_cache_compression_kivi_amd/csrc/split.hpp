// split.hpp -- how decode attention divides one unit's tokens among
// work-groups (splits) and among the waves of a work-group. Shared by the
// kernel and the host-side tests, so both use one definition.
//
// Work items are the unit's key blocks (G = 32 quantized tokens each) and its
// residual chunks (up to 32 fp16 tokens each). A residual chunk moves about
// four times the bytes of a 2-bit block (16 KB against 4 KB at d = 128), so
// items are balanced by cost, and the residual goes to the last split.
#pragma once

#include <cstdint>

#ifdef __HIPCC__
#define KIVI_HD __host__ __device__
#else
#define KIVI_HD
#endif

namespace kivi {

// Cost of one residual chunk, in key blocks of the given bit width.
KIVI_HD inline int64_t residual_chunk_cost(int bits) { return bits == 2 ? 4 : 3; }

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

// A work-group of nw waves holds nbw key blocks and rc residual chunks;
// residual chunk k goes to wave k mod nw. Wave w takes key blocks
// [wave_start(w), wave_start(w + 1)), so that every wave carries about the
// same cost. Non-decreasing in w, wave_start(0) = 0, wave_start(nw) = nbw.
KIVI_HD inline int64_t wave_start(int64_t nbw, int64_t rc, int64_t cost, int64_t nw, int64_t w) {
    if (w >= nw) return nbw;
    const int64_t total = nbw + cost * rc;
    int64_t best = 0;
    for (int64_t v = 1; v <= w; ++v) {
        const int64_t r = rc % nw;
        const int64_t chunks_before = (rc / nw) * v + (r < v ? r : v);  // chunks held by waves [0, v)
        const int64_t f = v * total / nw - cost * chunks_before;
        if (f > best) best = f;
    }
    return best < nbw ? best : nbw;
}

}  // namespace kivi
