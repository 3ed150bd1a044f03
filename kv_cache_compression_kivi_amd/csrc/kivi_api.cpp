// kivi_api.cpp -- the C ABI of include/kivi.h: validation, host counters and
// kernel launches on the caller's stream. See kivi.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kivi.h"
#include "launch.hpp"
#include "planner.hpp"

static_assert(kivi::kMaxRaggedRows == KIVI_MAX_RAGGED_BATCH, "a row table holds the rows of one launch");
// the row tables ride in the kernel arguments, whose block is at most 4 KiB
static_assert(sizeof(kivi::QuantArgs) <= 4096 && sizeof(kivi::RingArgs) <= 4096 && sizeof(kivi::AttendArgs) <= 4096,
              "kernel arguments fit the 4 KiB argument block");

struct kivi_cache {
    kivi_config cfg;
    kivi_layout L;
    uint8_t* mem;
    size_t bytes;
    // per batch row (sequence): tokens held, and how many of them are quantized
    std::vector<int64_t> nt, nq;
    // paged blocks: the caller's device block table [batch][table_stride]
    const int32_t* table;
    int64_t table_stride;
    int32_t forced_splits;
    // compute units of the device current at create time (the split plans fill them)
    int32_t cus;
    // SQuat-style key coder: coefficients built (kivi_squat_build)
    bool squat_ready;
    bool poisoned;
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int device_fail(kivi_cache* c, const char* what, hipError_t e) {
    c->poisoned = true;
    return fail(KIVI_E_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

kivi::CacheGeom geom(const kivi_cache* c) {
    kivi::CacheGeom g;
    g.base = c->mem;
    g.off_blocks = c->L.off_blocks;
    g.unit_stride = c->L.unit_stride;
    g.block_bytes = c->L.block_bytes;
    g.rec_kcode = c->L.rec_kcode;
    g.rec_vcode = c->L.rec_vcode;
    g.rec_ksz = c->L.rec_ksz;
    g.rec_vsz = c->L.rec_vsz;
    g.off_ring = c->L.off_ring;
    g.ring_unit_stride = c->L.ring_unit_stride;
    g.ring_slots = c->L.ring_slots;
    g.partial = c->mem + c->L.off_partial;
    g.partial_stride = c->L.partial_stride;
    g.partial_splits = c->L.max_splits;
    g.batch = c->cfg.batch;
    g.n_kv_heads = c->cfg.n_kv_heads;
    g.n_q_heads = c->cfg.n_q_heads;
    g.head_dim = c->cfg.head_dim;
    g.bits = c->cfg.bits;
    g.table = c->cfg.n_pages > 0 ? c->table : nullptr;
    g.table_stride = c->table_stride;
    g.n_pages = c->cfg.n_pages;
    g.off_squat = c->L.off_squat;
    g.squat_r8 = c->L.squat_r8;
    return g;
}

bool paged(const kivi_cache* c) { return c->cfg.n_pages > 0; }

// Rows [r0, r0 + n) of the cache as a batch of their own: every per-unit
// region (key blocks unless paged, ring, split partials, SQuat coefficients)
// and the block table start at row r0. Launches that carry a row table cover
// at most kMaxRaggedRows rows, so larger batches run as several of them.
kivi::CacheGeom chunk_geom(const kivi_cache* c, int r0, int n) {
    kivi::CacheGeom g = geom(c);
    const size_t u0 = (size_t)r0 * (size_t)c->cfg.n_kv_heads;
    if (!paged(c)) g.off_blocks += u0 * g.unit_stride;
    g.off_ring += u0 * g.ring_unit_stride;
    g.partial += (size_t)r0 * (size_t)c->cfg.n_q_heads * (size_t)g.partial_splits * g.partial_stride;
    g.off_squat += u0 * 2 * (size_t)g.head_dim * (size_t)g.squat_r8 * sizeof(float);
    if (g.table) g.table += (size_t)r0 * (size_t)g.table_stride;
    g.batch = n;
    return g;
}

// Input rows of units [r0 Hkv, ...): `per_unit` elements of 16 bits per unit.
const void* rows_from(const void* p, int r0, int64_t units_per_row, int64_t per_unit) {
    return p ? static_cast<const void*>(static_cast<const uint16_t*>(p) + (size_t)r0 * units_per_row * per_unit)
             : nullptr;
}

// A paged cache's calls need the block table.
int check_table(const kivi_cache* c) {
    if (paged(c) && !c->table) return fail(KIVI_E_INVAL, "paged cache without a block table (kivi_set_block_table)");
    return KIVI_OK;
}

int check_handle(const kivi_cache* c) {
    if (!c) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (c->poisoned) return fail(KIVI_E_STATE, "cache saw an earlier device failure; reset it");
    return check_table(c);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// True when every entry of x equals the first.
bool all_same(const std::vector<int64_t>& x) {
    for (int64_t e : x)
        if (e != x[0]) return false;
    return true;
}

bool rows_agree(const kivi_cache* c) { return all_same(c->nt) && all_same(c->nq); }

int64_t max_of(const std::vector<int64_t>& x) {
    int64_t m = x[0];
    for (int64_t e : x) m = e > m ? e : m;
    return m;
}


// Per-row work of one append or flush: quantize key blocks [j0, j1) with
// tokens below ring_end read from the ring (the rest from input rows t -
// ring_end), then copy tokens [t0, t1) into the ring from input rows t - in_t0.
struct RowWork {
    std::vector<int64_t> j0, j1, ring_end, t0, t1, in_t0;
    explicit RowWork(int n) : j0(n), j1(n), ring_end(n), t0(n), t1(n), in_t0(n) {}
};

// Whether the rows' ranges differ, so that the launches need row tables.
bool work_ragged(const RowWork& w) {
    return !(all_same(w.j0) && all_same(w.j1) && all_same(w.ring_end) && all_same(w.t0) && all_same(w.t1) &&
             all_same(w.in_t0));
}

// The launches of one append or flush over rows [r0, r0 + n) (ntok input
// rows per unit in k and v, which start at row 0), with row tables when
// `ragged`. The quantization goes first: its ring reads must see the slots
// before this call's writes.
int launch_work_rows(kivi_cache* c, const RowWork& w, int r0, int n, bool ragged, const void* k, const void* v,
                     int64_t ntok, hipStream_t s) {
    const int64_t hkv = c->cfg.n_kv_heads, per_unit = ntok * c->cfg.head_dim;
    int64_t nblk = 0, ntk = 0;
    for (int b = r0; b < r0 + n; ++b) {
        nblk = w.j1[b] - w.j0[b] > nblk ? w.j1[b] - w.j0[b] : nblk;
        ntk = w.t1[b] - w.t0[b] > ntk ? w.t1[b] - w.t0[b] : ntk;
    }
    const kivi::CacheGeom g = chunk_geom(c, r0, n);
    const auto* kr = static_cast<const uint16_t*>(rows_from(k, r0, hkv, per_unit));
    const auto* vr = static_cast<const uint16_t*>(rows_from(v, r0, hkv, per_unit));
    // Rows that agree, and no quantized token read from the ring (a prefill
    // into an empty residual, say): the ring copy joins the quantize launch,
    // as nothing the launch (or the key coder after it) reads is a ring slot
    // the copy writes.
    const bool fuse_ring = !ragged && nblk > 0 && ntk > 0 && w.ring_end[r0] <= w.j0[r0] * c->cfg.k_block;
    if (nblk > 0) {
        kivi::QuantArgs a;
        a.g = g;
        a.k = kr;
        a.v = vr;
        a.ntok = ntok;
        a.ring_t0 = fuse_ring ? w.t0[r0] : 0;
        a.ring_t1 = fuse_ring ? w.t1[r0] : 0;
        a.ring_in_t0 = fuse_ring ? w.in_t0[r0] : 0;
        a.ring_wgs = fuse_ring ? (int32_t)((w.t1[r0] - w.t0[r0] + 7) / 8) : 0;
        a.rows.n = 0;
        if (ragged) {
            a.j0 = 0;
            a.j1 = nblk;
            a.ring_end = 0;
            a.rows.n = n;
            for (int b = 0; b < n; ++b) {
                a.rows.j0[b] = (int32_t)w.j0[r0 + b];
                a.rows.j1[b] = (int32_t)w.j1[r0 + b];
                a.rows.ring_end[b] = (int32_t)w.ring_end[r0 + b];
            }
        } else {
            a.j0 = w.j0[r0];
            a.j1 = w.j1[r0];
            a.ring_end = w.ring_end[r0];
        }
        hipError_t e = kivi::launch_quantize(a, s);
        if (e != hipSuccess) return device_fail(c, "quantize launch", e);
        // SQuat-style key codes over the blocks just quantized (before the
        // ring write below: they read ring slots it may overwrite)
        if (c->cfg.squat_rank > 0 && c->squat_ready) {
            e = kivi::launch_squat_codes(a, s);
            if (e != hipSuccess) return device_fail(c, "squat codes launch", e);
        }
    }
    if (ntk > 0 && !fuse_ring) {
        kivi::RingArgs a;
        a.g = g;
        a.k = kr;
        a.v = vr;
        a.ntok = ntok;
        a.rows.n = 0;
        if (ragged) {
            a.t0 = 0;
            a.t1 = ntk;
            a.in_t0 = 0;
            a.rows.n = n;
            for (int b = 0; b < n; ++b) {
                a.rows.t0[b] = (int32_t)w.t0[r0 + b];
                a.rows.t1[b] = (int32_t)(w.t1[r0 + b] > w.t0[r0 + b] ? w.t1[r0 + b] : w.t0[r0 + b]);
                a.rows.in_t0[b] = (int32_t)w.in_t0[r0 + b];
            }
        } else {
            a.t0 = w.t0[r0];
            a.t1 = w.t1[r0];
            a.in_t0 = w.in_t0[r0];
        }
        hipError_t e = kivi::launch_ring_write(a, s);
        if (e != hipSuccess) return device_fail(c, "ring write launch", e);
    }
    return KIVI_OK;
}

// The launches of one append or flush: one set over the whole batch when the
// rows' work agrees, else one per kMaxRaggedRows rows, each with row tables
// (different units, so their order does not matter).
int launch_work(kivi_cache* c, const RowWork& w, const void* k, const void* v, int64_t ntok, hipStream_t s) {
    const int B = c->cfg.batch;
    if (!work_ragged(w)) return launch_work_rows(c, w, 0, B, false, k, v, ntok, s);
    for (int r0 = 0; r0 < B; r0 += kivi::kMaxRaggedRows) {
        const int n = B - r0 < kivi::kMaxRaggedRows ? B - r0 : kivi::kMaxRaggedRows;
        const int rc = launch_work_rows(c, w, r0, n, true, k, v, ntok, s);
        if (rc != KIVI_OK) return rc;
    }
    return KIVI_OK;
}

// Appends ntok[b] tokens to row b: the per-row work and the counters after.
RowWork plan_rows(const kivi_cache* c, const int32_t* ntok, std::vector<int64_t>& nt1, std::vector<int64_t>& nq1) {
    const int B = c->cfg.batch;
    const int64_t G = c->cfg.k_block, R = c->cfg.residual;
    RowWork w(B);
    for (int b = 0; b < B; ++b) {
        const kivi::AppendPlan p = kivi::plan_append(c->nt[b], c->nq[b], ntok[b], R, G);
        w.j0[b] = p.nq0 / G;
        w.j1[b] = p.nq1 / G;
        w.ring_end[b] = p.nt0;
        w.t0[b] = p.ring_t0;
        w.t1[b] = p.nt1 > p.ring_t0 ? p.nt1 : p.ring_t0;
        w.in_t0[b] = p.nt0;
        nt1[b] = p.nt1;
        nq1[b] = p.nq1;
    }
    return w;
}

int validate_kv(const void* k, const void* v) {
    if (!k || !v) return fail(KIVI_E_INVAL, "k and v must be device pointers");
    if (!aligned16(k) || !aligned16(v)) return fail(KIVI_E_INVAL, "k and v must be 16-byte aligned");
    return KIVI_OK;
}

int validate_q(const void* q, int32_t q_dtype, const float* out) {
    if (!q || !out) return fail(KIVI_E_INVAL, "q and out must be device pointers");
    if (!aligned16(q) || !aligned16(out)) return fail(KIVI_E_INVAL, "q and out must be 16-byte aligned");
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_BF16) return fail(KIVI_E_INVAL, "q_dtype must be KIVI_F16 or KIVI_BF16");
    return KIVI_OK;
}

// Whether attention launches carry a row table: paged blocks, or rows that
// differ in length (then kMaxRaggedRows rows a launch).
bool attend_rows_table(const kivi_cache* c) { return paged(c) || !rows_agree(c); }

// The split plan of the launch over rows [r0, r0 + n) (the whole batch when
// no row table is needed); *cost_max receives the costliest row's cost.
// No heap allocation: a launch with a row table covers at most
// kMaxRaggedRows rows.
kivi::AttendPlan attend_plan(const kivi_cache* c, int r0, int n, int64_t* cost_max = nullptr) {
    const int32_t group = c->cfg.n_q_heads / c->cfg.n_kv_heads;
    const int64_t G = c->cfg.k_block;
    if (!attend_rows_table(c)) {
        if (cost_max) *cost_max = kivi::unit_cost(c->nq[0] / G, c->nt[0] - c->nq[0]);
        return kivi::plan_attend((int64_t)c->cfg.batch * c->cfg.n_kv_heads, group, c->cfg.head_dim, c->nq[0] / G,
                                 c->L.max_splits, c->forced_splits, c->cus);
    }
    int64_t cost[kivi::kMaxRaggedRows];
    int64_t nq_max = 0;
    for (int b = 0; b < n; ++b) {
        cost[b] = kivi::unit_cost(c->nq[r0 + b] / G, c->nt[r0 + b] - c->nq[r0 + b]);
        nq_max = c->nq[r0 + b] > nq_max ? c->nq[r0 + b] : nq_max;
    }
    int64_t cm = 1;
    kivi::AttendPlan p = kivi::plan_attend_rows(c->cfg.n_kv_heads, group, c->cfg.head_dim, n, cost, nq_max / G,
                                                c->L.max_splits, c->forced_splits, c->cus, &cm);
    if (cost_max) *cost_max = cm;
    return p;
}

// Where an attention launch writes its split partials: the cache's partial
// region (nullptr), or other device memory of `splits` slots per query head.
struct PartialBuf {
    uint8_t* base;
    int32_t splits;
};

// The attention launch over rows [r0, r0 + n) with the counters of the
// handle (q, out, k_new and v_new start at row 0). With k_new / v_new, the
// newest token of each row for which appended[b] holds (its token n_t - 1)
// was appended by this call and is not in the ring yet. No heap allocation.
int attend_call(kivi_cache* cache, int r0, int n, const void* q, int32_t q_dtype, float* out, void* stream,
                const void* k_new, const void* v_new, const char* appended, const kivi::AttendPlan& p,
                int64_t cost_max, PartialBuf pb = {nullptr, 0}) {
    const int64_t hq = cache->cfg.n_q_heads, hkv = cache->cfg.n_kv_heads, d = cache->cfg.head_dim;
    kivi::AttendArgs a;
    a.g = chunk_geom(cache, r0, n);
    if (pb.base) {
        a.g.partial = pb.base;
        a.g.partial_splits = pb.splits;
    }
    a.q = static_cast<const uint16_t*>(rows_from(q, r0, hq, d));
    a.q_bf16 = q_dtype == KIVI_BF16;
    a.out = out + (size_t)r0 * hq * d;
    a.n_split = p.n_split;
    a.qg = p.qg;
    a.nwaves = p.nwaves;
    a.scale_log2 = (float)(1.4426950408889634074 / std::sqrt((double)d));
    a.k_new = static_cast<const uint16_t*>(rows_from(k_new, r0, hkv, d));
    a.v_new = static_cast<const uint16_t*>(rows_from(v_new, r0, hkv, d));
    auto t_new = [&](int b) -> int64_t { return appended && appended[b] ? cache->nt[b] - 1 : -1; };
    a.rows.n = 0;
    a.cost_max = cost_max;
    // paged blocks are read by the kernels built with a row table
    if (!attend_rows_table(cache)) {
        // rows that agree (an appended token then lands in every row alike)
        a.n_tokens = cache->nt[0];
        a.n_quant = cache->nq[0];
        a.n_blocks = cache->nq[0] / cache->cfg.k_block;
        a.t_new = t_new(0);
    } else {
        int64_t nt_max = 0, nq_max = 0;
        int64_t cost[kivi::kMaxRaggedRows];
        a.rows.n = n;
        for (int b = 0; b < n; ++b) {
            const int gb = r0 + b;
            nt_max = cache->nt[gb] > nt_max ? cache->nt[gb] : nt_max;
            nq_max = cache->nq[gb] > nq_max ? cache->nq[gb] : nq_max;
            a.rows.n_tokens[b] = (int32_t)cache->nt[gb];
            a.rows.n_quant[b] = (int32_t)cache->nq[gb];
            a.rows.t_new[b] = (int32_t)t_new(gb);
            a.rows.order[b] = b;
            cost[b] = kivi::unit_cost(cache->nq[gb] / cache->cfg.k_block, cache->nt[gb] - cache->nq[gb]);
        }
        a.n_tokens = nt_max;
        a.n_quant = nq_max;
        a.n_blocks = nq_max / cache->cfg.k_block;
        a.t_new = -1;
        // costliest rows first: their work-groups start in the first round
        std::stable_sort(a.rows.order, a.rows.order + n, [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
    }
    (void)hipGetLastError();
    hipError_t e = kivi::launch_attend(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(cache, "attend launch", e);
    return KIVI_OK;
}

// Rows per attention launch: the whole batch, or kMaxRaggedRows with a row table.
int attend_chunk_rows(const kivi_cache* c) {
    return attend_rows_table(c) ? kivi::kMaxRaggedRows : c->cfg.batch;
}

// Bytes of split partials that the launch over n rows with plan p writes.
uint64_t partial_need(const kivi_cache* c, int n, const kivi::AttendPlan& p) {
    return (uint64_t)n * (uint64_t)c->cfg.n_q_heads * (uint64_t)p.n_split * (uint64_t)c->L.partial_stride;
}

// Every attention launch of one call, in row order. With `scratch`, each
// launch that splits writes its partials there (launches on one stream run
// in order, so each may reuse it); the caller has checked that they fit.
int attend_all(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream, const void* k_new,
               const void* v_new, const char* appended, uint8_t* scratch) {
    const int B = cache->cfg.batch, step = attend_chunk_rows(cache);
    for (int r0 = 0; r0 < B; r0 += step) {
        const int n = B - r0 < step ? B - r0 : step;
        int64_t cost_max = 1;
        const kivi::AttendPlan p = attend_plan(cache, r0, n, &cost_max);
        PartialBuf pb = {nullptr, 0};
        if (scratch && p.n_split > 1) pb = {scratch, p.n_split};
        const int rc = attend_call(cache, r0, n, q, q_dtype, out, stream, k_new, v_new, appended, p, cost_max, pb);
        if (rc != KIVI_OK) return rc;
    }
    return KIVI_OK;
}

// Checks common to the attention entry points: handle, query, output, and no empty sequence.
int check_attend(kivi_cache* cache, const void* q, int32_t q_dtype, const float* out) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if ((rc = validate_q(q, q_dtype, out)) != KIVI_OK) return rc;
    for (int b = 0; b < cache->cfg.batch; ++b)
        if (cache->nt[b] == 0)
            return fail(KIVI_E_EMPTY, rows_agree(cache) ? std::string("attention on an empty cache")
                                                        : "attention with sequence " + std::to_string(b) + " empty");
    return KIVI_OK;
}

// Compute units of the current device, or kDefaultCUs (an MI355X's 256) when
// no device answers (host-only use: the plan then only matters to the tests).
int32_t device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return kivi::kDefaultCUs;
    }
    return n;
}

int check_row(const kivi_cache* c, int32_t row) {
    if (row < 0 || row >= c->cfg.batch)
        return fail(KIVI_E_INVAL, "row " + std::to_string(row) + " outside [0, " + std::to_string(c->cfg.batch) + ")");
    return KIVI_OK;
}

}  // namespace

extern "C" {

int kivi_abi_version(void) { return KIVI_ABI_VERSION; }

const char* kivi_last_error(void) { return g_err.c_str(); }

int kivi_cache_bytes(const kivi_config* cfg, size_t* bytes) {
    std::string err;
    int rc = kivi::validate_config(cfg, err);
    if (rc != KIVI_OK) return fail(rc, err);
    if (!bytes) return fail(KIVI_E_INVAL, "bytes is NULL");
    kivi_layout L;
    kivi::compute_layout(cfg, &L);
    *bytes = L.total_bytes;
    return KIVI_OK;
}

int kivi_cache_layout(const kivi_config* cfg, kivi_layout* layout) {
    std::string err;
    int rc = kivi::validate_config(cfg, err);
    if (rc != KIVI_OK) return fail(rc, err);
    if (!layout) return fail(KIVI_E_INVAL, "layout is NULL");
    kivi::compute_layout(cfg, layout);
    return KIVI_OK;
}

int kivi_cache_create(const kivi_config* cfg, void* dev_mem, size_t bytes, kivi_cache** out) {
    std::string err;
    int rc = kivi::validate_config(cfg, err);
    if (rc != KIVI_OK) return fail(rc, err);
    if (!out) return fail(KIVI_E_INVAL, "out is NULL");
    if (!dev_mem) return fail(KIVI_E_INVAL, "dev_mem is NULL");
    if (((uintptr_t)dev_mem & (kivi::kAlign - 1)) != 0) return fail(KIVI_E_INVAL, "dev_mem must be 256-byte aligned");
    kivi_layout L;
    kivi::compute_layout(cfg, &L);
    if (bytes < L.total_bytes)
        return fail(KIVI_E_NOMEM, "cache memory too small: need " + std::to_string(L.total_bytes) + " bytes, got " +
                                      std::to_string(bytes));
    kivi_cache* c = new (std::nothrow) kivi_cache;
    if (!c) return fail(KIVI_E_NOMEM, "host allocation of the handle failed");
    c->cfg = *cfg;
    c->L = L;
    c->mem = static_cast<uint8_t*>(dev_mem);
    c->bytes = bytes;
    c->nt.assign(cfg->batch, 0);
    c->nq.assign(cfg->batch, 0);
    c->table = nullptr;
    c->table_stride = 0;
    c->forced_splits = 0;
    c->cus = device_cus();
    c->squat_ready = false;
    c->poisoned = false;
    *out = c;
    return KIVI_OK;
}

int kivi_cache_destroy(kivi_cache* cache) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    delete cache;
    return KIVI_OK;
}

int kivi_cache_reset(kivi_cache* cache) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    std::fill(cache->nt.begin(), cache->nt.end(), 0);
    std::fill(cache->nq.begin(), cache->nq.end(), 0);
    cache->poisoned = false;
    return KIVI_OK;
}

int kivi_set_block_table(kivi_cache* cache, const int32_t* table, int32_t stride) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (!paged(cache)) return fail(KIVI_E_INVAL, "the cache is not paged (n_pages = 0)");
    if (!table || ((uintptr_t)table & 3u) != 0) return fail(KIVI_E_INVAL, "table must be a 4-byte aligned device pointer");
    if (stride < cache->L.max_blocks)
        return fail(KIVI_E_INVAL, "stride " + std::to_string(stride) + " < max_blocks " +
                                      std::to_string(cache->L.max_blocks));
    cache->table = table;
    cache->table_stride = stride;
    return KIVI_OK;
}

int kivi_reset_row(kivi_cache* cache, int32_t row) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (cache->poisoned) return fail(KIVI_E_STATE, "cache saw an earlier device failure; reset it");
    int rc = check_row(cache, row);
    if (rc != KIVI_OK) return rc;
    cache->nt[row] = 0;
    cache->nq[row] = 0;
    return KIVI_OK;
}

int kivi_cache_query(const kivi_cache* cache, kivi_state* st) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (!st) return fail(KIVI_E_INVAL, "state is NULL");
    if (!rows_agree(cache)) return fail(KIVI_E_RAGGED, "the sequences differ in length; use kivi_query_row");
    st->n_tokens = cache->nt[0];
    st->n_quant = cache->nq[0];
    st->n_resid = cache->nt[0] - cache->nq[0];
    return KIVI_OK;
}

int kivi_query_row(const kivi_cache* cache, int32_t row, kivi_state* st) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (!st) return fail(KIVI_E_INVAL, "state is NULL");
    int rc = check_row(cache, row);
    if (rc != KIVI_OK) return rc;
    st->n_tokens = cache->nt[row];
    st->n_quant = cache->nq[row];
    st->n_resid = cache->nt[row] - cache->nq[row];
    return KIVI_OK;
}

int kivi_plan_append(const kivi_cache* cache, int32_t ntok, kivi_state* after) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (!after) return fail(KIVI_E_INVAL, "state is NULL");
    if (ntok < 1) return fail(KIVI_E_INVAL, "ntok must be >= 1");
    if (!rows_agree(cache)) return fail(KIVI_E_RAGGED, "the sequences differ in length");
    if (cache->nt[0] + ntok > cache->cfg.max_tokens) return fail(KIVI_E_CAPACITY, "append would exceed max_tokens");
    kivi::AppendPlan p = kivi::plan_append(cache->nt[0], cache->nq[0], ntok, cache->cfg.residual, cache->cfg.k_block);
    after->n_tokens = p.nt1;
    after->n_quant = p.nq1;
    after->n_resid = p.nt1 - p.nq1;
    return KIVI_OK;
}

int kivi_append(kivi_cache* cache, const void* k, const void* v, int32_t ntok, void* stream) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if ((rc = validate_kv(k, v)) != KIVI_OK) return rc;
    if (ntok < 1) return fail(KIVI_E_INVAL, "ntok must be >= 1");
    if (max_of(cache->nt) + ntok > cache->cfg.max_tokens)
        return fail(KIVI_E_CAPACITY, "append of " + std::to_string(ntok) + " tokens would exceed max_tokens (" +
                                         std::to_string(cache->cfg.max_tokens) + ")");
    const int B = cache->cfg.batch;
    std::vector<int32_t> n(B, ntok);
    std::vector<int64_t> nt1(B), nq1(B);
    const RowWork w = plan_rows(cache, n.data(), nt1, nq1);
    (void)hipGetLastError();
    rc = launch_work(cache, w, k, v, ntok, static_cast<hipStream_t>(stream));
    if (rc != KIVI_OK) return rc;
    cache->nt = nt1;
    cache->nq = nq1;
    return KIVI_OK;
}

int kivi_append_rows(kivi_cache* cache, const void* k, const void* v, const int32_t* ntok, int32_t max_ntok,
                     void* stream) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if ((rc = validate_kv(k, v)) != KIVI_OK) return rc;
    if (!ntok) return fail(KIVI_E_INVAL, "ntok is NULL");
    if (max_ntok < 1) return fail(KIVI_E_INVAL, "max_ntok must be >= 1");
    const int B = cache->cfg.batch;
    for (int b = 0; b < B; ++b) {
        if (ntok[b] < 0 || ntok[b] > max_ntok)
            return fail(KIVI_E_INVAL, "ntok[" + std::to_string(b) + "] = " + std::to_string(ntok[b]) +
                                          " outside [0, max_ntok]");
        if (cache->nt[b] + ntok[b] > cache->cfg.max_tokens)
            return fail(KIVI_E_CAPACITY, "append of " + std::to_string(ntok[b]) + " tokens to row " +
                                             std::to_string(b) + " would exceed max_tokens (" +
                                             std::to_string(cache->cfg.max_tokens) + ")");
    }
    std::vector<int64_t> nt1(B), nq1(B);
    const RowWork w = plan_rows(cache, ntok, nt1, nq1);
    (void)hipGetLastError();
    rc = launch_work(cache, w, k, v, max_ntok, static_cast<hipStream_t>(stream));
    if (rc != KIVI_OK) return rc;
    cache->nt = nt1;
    cache->nq = nq1;
    return KIVI_OK;
}

int kivi_flush(kivi_cache* cache, void* stream, int32_t* n_flushed) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    const int B = cache->cfg.batch;
    const int64_t G = cache->cfg.k_block;
    RowWork w(B);
    std::vector<int64_t> nq1(B);
    int64_t kmax = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t k = kivi::plan_flush(cache->nt[b], cache->nq[b], cache->cfg.residual, G);
        w.j0[b] = cache->nq[b] / G;
        w.j1[b] = (cache->nq[b] + k) / G;
        w.ring_end[b] = cache->nt[b];
        w.t0[b] = w.t1[b] = w.in_t0[b] = 0;
        nq1[b] = cache->nq[b] + k;
        kmax = k > kmax ? k : kmax;
    }
    (void)hipGetLastError();
    rc = launch_work(cache, w, nullptr, nullptr, 0, static_cast<hipStream_t>(stream));
    if (rc != KIVI_OK) return rc;
    cache->nq = nq1;
    if (n_flushed) *n_flushed = (int32_t)kmax;
    return KIVI_OK;
}

int kivi_plan_attend(const kivi_cache* cache, int32_t* n_split, int32_t* blocks_per_split) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    // the launch with the most splits, when the call runs several
    const int B = cache->cfg.batch, step = attend_chunk_rows(cache);
    kivi::AttendPlan p = attend_plan(cache, 0, B < step ? B : step);
    for (int r0 = step; r0 < B; r0 += step) {
        const kivi::AttendPlan q = attend_plan(cache, r0, B - r0 < step ? B - r0 : step);
        if (q.n_split > p.n_split) p = q;
    }
    if (n_split) *n_split = p.n_split;
    if (blocks_per_split) *blocks_per_split = p.blocks_per_split;
    return KIVI_OK;
}

int kivi_set_attend_splits(kivi_cache* cache, int32_t n_split) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (n_split < 0 || n_split > cache->L.max_splits)
        return fail(KIVI_E_INVAL, "n_split must be in [0, max_splits]");
    cache->forced_splits = n_split;
    return KIVI_OK;
}

int kivi_squat_build(kivi_cache* cache, const void* q, int32_t q_dtype, int32_t n_q, float lambda, void* stream) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if (cache->cfg.squat_rank <= 0) return fail(KIVI_E_INVAL, "the cache was made with squat_rank = 0");
    if (!q || !aligned16(q)) return fail(KIVI_E_INVAL, "q must be a 16-byte aligned device pointer");
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_BF16) return fail(KIVI_E_INVAL, "q_dtype must be KIVI_F16 or KIVI_BF16");
    if (n_q < 1) return fail(KIVI_E_INVAL, "n_q must be >= 1");
    if (!(lambda > 0.0f) || !std::isfinite(lambda)) return fail(KIVI_E_INVAL, "lambda must be a positive finite number");
    kivi::SquatBuildArgs a;
    a.g = geom(cache);
    a.q = static_cast<const uint16_t*>(q);
    a.q_bf16 = q_dtype == KIVI_BF16;
    a.n_q = n_q;
    a.rank = cache->cfg.squat_rank;
    a.lambda = lambda;
    (void)hipGetLastError();
    hipError_t e = kivi::launch_squat_build(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(cache, "squat build launch", e);
    cache->squat_ready = true;
    return KIVI_OK;
}

int kivi_attend_decode(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream) {
    int rc = check_attend(cache, q, q_dtype, out);
    if (rc != KIVI_OK) return rc;
    return attend_all(cache, q, q_dtype, out, stream, nullptr, nullptr, nullptr, nullptr);
}

int kivi_attend_decode_noalloc(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream) {
    int rc = check_attend(cache, q, q_dtype, out);
    if (rc != KIVI_OK) return rc;
    // the partials of each launch, n_split slots per query head of its rows,
    // in the library's static scratch: every launch's must fit (checked
    // before any launch)
    const int B = cache->cfg.batch, step = attend_chunk_rows(cache);
    bool splits = false;
    for (int r0 = 0; r0 < B; r0 += step) {
        const int n = B - r0 < step ? B - r0 : step;
        const kivi::AttendPlan p = attend_plan(cache, r0, n);
        if (p.n_split <= 1) continue;
        splits = true;
        const uint64_t need = partial_need(cache, n, p);
        if (need > (uint64_t)KIVI_NOALLOC_SCRATCH_BYTES)
            return fail(KIVI_E_NOMEM, "split partials of " + std::to_string(need) + " bytes (" + std::to_string(n) +
                                          " rows * n_q_heads * " + std::to_string(p.n_split) + " splits * " +
                                          std::to_string(cache->L.partial_stride) +
                                          ") exceed the static scratch of " +
                                          std::to_string((uint64_t)KIVI_NOALLOC_SCRATCH_BYTES) + " bytes");
    }
    void* ptr = nullptr;
    if (splits) {
        hipError_t e = kivi::static_scratch(&ptr);
        if (e != hipSuccess) return fail(KIVI_E_DEVICE, std::string("static scratch: ") + hipGetErrorString(e));
    }
    return attend_all(cache, q, q_dtype, out, stream, nullptr, nullptr, nullptr, static_cast<uint8_t*>(ptr));
}

int kivi_decode_step(kivi_cache* cache, const void* k, const void* v, const void* q, int32_t q_dtype, float* out,
                     void* stream, int32_t* n_flushed) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if ((rc = validate_q(q, q_dtype, out)) != KIVI_OK) return rc;
    if ((rc = validate_kv(k, v)) != KIVI_OK) return rc;
    if (max_of(cache->nt) + 1 > cache->cfg.max_tokens)
        return fail(KIVI_E_CAPACITY, "append of 1 token would exceed max_tokens (" +
                                         std::to_string(cache->cfg.max_tokens) + ")");
    // The same result as kivi_append(1) + kivi_flush (when a whole group lies
    // beyond the newest R) + kivi_attend_decode, in at most two launches: the
    // quantization of every group that leaves the residual (the new token,
    // should it be one of them, read from k and v), then the attention, which
    // also writes the new token into its ring slot.
    const int B = cache->cfg.batch;
    const int64_t G = cache->cfg.k_block, R = cache->cfg.residual;
    RowWork w(B);
    std::vector<int64_t> nt1(B), nq1(B);
    std::vector<char> appended(B);
    int64_t fmax = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t nt0 = cache->nt[b];
        const kivi::AppendPlan p = kivi::plan_append(nt0, cache->nq[b], 1, R, G);
        const int64_t n_res = p.nt1 - p.nq1;
        const int64_t nq = n_res >= R + G ? p.nq1 + kivi::plan_flush(p.nt1, p.nq1, R, G) : p.nq1;
        w.j0[b] = p.nq0 / G;
        w.j1[b] = nq / G;
        w.ring_end[b] = nt0;
        w.t0[b] = w.t1[b] = w.in_t0[b] = 0;  // the attention writes the token into the ring
        nt1[b] = p.nt1;
        nq1[b] = nq;
        appended[b] = nt0 >= nq;
        fmax = nq - p.nq1 > fmax ? nq - p.nq1 : fmax;
    }
    (void)hipGetLastError();
    rc = launch_work(cache, w, k, v, 1, static_cast<hipStream_t>(stream));
    if (rc != KIVI_OK) return rc;
    cache->nt = nt1;
    cache->nq = nq1;
    if (n_flushed) *n_flushed = (int32_t)fmax;
    return attend_all(cache, q, q_dtype, out, stream, k, v, appended.data(), nullptr);
}

}  // extern "C"
