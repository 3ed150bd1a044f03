// kivi_api.cpp -- the C ABI of include/kivi.h: validation, host counters and
// kernel launches on the caller's stream. See kivi.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "kivi.h"
#include "launch.hpp"
#include "planner.hpp"

struct kivi_cache {
    kivi_config cfg;
    kivi_layout L;
    uint8_t* mem;
    size_t bytes;
    int64_t n_tokens;
    int64_t n_quant;
    int32_t forced_splits;
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
    g.off_partial = c->L.off_partial;
    g.partial_stride = c->L.partial_stride;
    g.max_splits = c->L.max_splits;
    g.batch = c->cfg.batch;
    g.n_kv_heads = c->cfg.n_kv_heads;
    g.n_q_heads = c->cfg.n_q_heads;
    g.head_dim = c->cfg.head_dim;
    g.bits = c->cfg.bits;
    return g;
}

int check_handle(const kivi_cache* c) {
    if (!c) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (c->poisoned) return fail(KIVI_E_STATE, "cache saw an earlier device failure; reset it");
    return KIVI_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Quantize key blocks [j0, j1) of every unit; tokens below ring_end come from
// the ring, the rest from input rows of k / v (ntok rows per unit).
int quantize_blocks(kivi_cache* c, int64_t j0, int64_t j1, int64_t ring_end, const void* k, const void* v,
                    int64_t ntok, hipStream_t s) {
    if (j1 <= j0) return KIVI_OK;
    kivi::QuantArgs a;
    a.g = geom(c);
    a.j0 = j0;
    a.j1 = j1;
    a.ring_end = ring_end;
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.ntok = ntok;
    hipError_t e = kivi::launch_quantize(a, s);
    if (e != hipSuccess) return device_fail(c, "quantize launch", e);
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
    c->n_tokens = 0;
    c->n_quant = 0;
    c->forced_splits = 0;
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
    cache->n_tokens = 0;
    cache->n_quant = 0;
    cache->poisoned = false;
    return KIVI_OK;
}

int kivi_cache_query(const kivi_cache* cache, kivi_state* st) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (!st) return fail(KIVI_E_INVAL, "state is NULL");
    st->n_tokens = cache->n_tokens;
    st->n_quant = cache->n_quant;
    st->n_resid = cache->n_tokens - cache->n_quant;
    return KIVI_OK;
}

int kivi_plan_append(const kivi_cache* cache, int32_t ntok, kivi_state* after) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    if (!after) return fail(KIVI_E_INVAL, "state is NULL");
    if (ntok < 1) return fail(KIVI_E_INVAL, "ntok must be >= 1");
    if (cache->n_tokens + ntok > cache->cfg.max_tokens)
        return fail(KIVI_E_CAPACITY, "append would exceed max_tokens");
    kivi::AppendPlan p =
        kivi::plan_append(cache->n_tokens, cache->n_quant, ntok, cache->cfg.residual, cache->cfg.k_block);
    after->n_tokens = p.nt1;
    after->n_quant = p.nq1;
    after->n_resid = p.nt1 - p.nq1;
    return KIVI_OK;
}

int kivi_append(kivi_cache* cache, const void* k, const void* v, int32_t ntok, void* stream) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if (!k || !v) return fail(KIVI_E_INVAL, "k and v must be device pointers");
    if (!aligned16(k) || !aligned16(v)) return fail(KIVI_E_INVAL, "k and v must be 16-byte aligned");
    if (ntok < 1) return fail(KIVI_E_INVAL, "ntok must be >= 1");
    if (cache->n_tokens + ntok > cache->cfg.max_tokens)
        return fail(KIVI_E_CAPACITY, "append of " + std::to_string(ntok) + " tokens would exceed max_tokens (" +
                                         std::to_string(cache->cfg.max_tokens) + ")");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t G = cache->cfg.k_block;
    kivi::AppendPlan p = kivi::plan_append(cache->n_tokens, cache->n_quant, ntok, cache->cfg.residual, G);
    (void)hipGetLastError();
    // quantize first: its ring reads must see the slots before this call's writes
    rc = quantize_blocks(cache, p.nq0 / G, p.nq1 / G, p.nt0, k, v, ntok, s);
    if (rc != KIVI_OK) return rc;
    if (p.nt1 > p.ring_t0) {
        kivi::RingArgs a;
        a.g = geom(cache);
        a.t0 = p.ring_t0;
        a.t1 = p.nt1;
        a.in_t0 = p.nt0;
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.ntok = ntok;
        hipError_t e = kivi::launch_ring_write(a, s);
        if (e != hipSuccess) return device_fail(cache, "ring write launch", e);
    }
    cache->n_tokens = p.nt1;
    cache->n_quant = p.nq1;
    return KIVI_OK;
}

int kivi_flush(kivi_cache* cache, void* stream, int32_t* n_flushed) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    const int64_t G = cache->cfg.k_block;
    const int64_t k = kivi::plan_flush(cache->n_tokens, cache->n_quant, cache->cfg.residual, G);
    (void)hipGetLastError();
    if (k > 0) {
        rc = quantize_blocks(cache, cache->n_quant / G, (cache->n_quant + k) / G, cache->n_tokens, nullptr, nullptr,
                             0, static_cast<hipStream_t>(stream));
        if (rc != KIVI_OK) return rc;
        cache->n_quant += k;
    }
    if (n_flushed) *n_flushed = (int32_t)k;
    return KIVI_OK;
}

namespace {
kivi::AttendPlan attend_plan(const kivi_cache* c) {
    return kivi::plan_attend((int64_t)c->cfg.batch * c->cfg.n_kv_heads, c->cfg.n_q_heads / c->cfg.n_kv_heads,
                             c->cfg.head_dim, c->n_quant / c->cfg.k_block, c->L.max_splits, c->forced_splits);
}
}  // namespace

int kivi_plan_attend(const kivi_cache* cache, int32_t* n_split, int32_t* blocks_per_split) {
    if (!cache) return fail(KIVI_E_INVAL, "cache handle is NULL");
    kivi::AttendPlan p = attend_plan(cache);
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

namespace {
// The attention launch; (k_new, v_new, t_new) carry a token appended in the
// same step that is not in the ring yet (t_new < 0: none).
int attend_call(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream, const void* k_new,
                const void* v_new, int64_t t_new) {
    kivi::AttendPlan p = attend_plan(cache);
    kivi::AttendArgs a;
    a.g = geom(cache);
    a.q = static_cast<const uint16_t*>(q);
    a.q_bf16 = q_dtype == KIVI_BF16;
    a.out = out;
    a.n_tokens = cache->n_tokens;
    a.n_quant = cache->n_quant;
    a.n_blocks = cache->n_quant / cache->cfg.k_block;
    a.n_split = p.n_split;
    a.qg = p.qg;
    a.nwaves = p.nwaves;
    a.scale_log2 = (float)(1.4426950408889634074 / std::sqrt((double)cache->cfg.head_dim));
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.t_new = t_new;
    (void)hipGetLastError();
    hipError_t e = kivi::launch_attend(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(cache, "attend launch", e);
    return KIVI_OK;
}
}  // namespace

int kivi_attend_decode(kivi_cache* cache, const void* q, int32_t q_dtype, float* out, void* stream) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if (!q || !out) return fail(KIVI_E_INVAL, "q and out must be device pointers");
    if (!aligned16(q) || !aligned16(out)) return fail(KIVI_E_INVAL, "q and out must be 16-byte aligned");
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_BF16) return fail(KIVI_E_INVAL, "q_dtype must be KIVI_F16 or KIVI_BF16");
    if (cache->n_tokens == 0) return fail(KIVI_E_EMPTY, "attention on an empty cache");
    return attend_call(cache, q, q_dtype, out, stream, nullptr, nullptr, -1);
}

int kivi_decode_step(kivi_cache* cache, const void* k, const void* v, const void* q, int32_t q_dtype, float* out,
                     void* stream, int32_t* n_flushed) {
    int rc = check_handle(cache);
    if (rc != KIVI_OK) return rc;
    if (!q || !out) return fail(KIVI_E_INVAL, "q and out must be device pointers");
    if (!aligned16(q) || !aligned16(out)) return fail(KIVI_E_INVAL, "q and out must be 16-byte aligned");
    if (q_dtype != KIVI_F16 && q_dtype != KIVI_BF16) return fail(KIVI_E_INVAL, "q_dtype must be KIVI_F16 or KIVI_BF16");
    if (!k || !v) return fail(KIVI_E_INVAL, "k and v must be device pointers");
    if (!aligned16(k) || !aligned16(v)) return fail(KIVI_E_INVAL, "k and v must be 16-byte aligned");
    if (cache->n_tokens + 1 > cache->cfg.max_tokens)
        return fail(KIVI_E_CAPACITY, "append of 1 token would exceed max_tokens (" +
                                         std::to_string(cache->cfg.max_tokens) + ")");
    // The same result as kivi_append(1) + kivi_flush (when a whole group lies
    // beyond the newest R) + kivi_attend_decode, in at most two launches: the
    // quantization of every group that leaves the residual (the new token,
    // should it be one of them, read from k and v), then the attention, which
    // also writes the new token into its ring slot.
    const int64_t G = cache->cfg.k_block, R = cache->cfg.residual;
    const int64_t nt0 = cache->n_tokens;
    kivi::AppendPlan p = kivi::plan_append(nt0, cache->n_quant, 1, R, G);
    const int64_t n_res = p.nt1 - p.nq1;
    const int64_t nq = n_res >= R + G ? p.nq1 + kivi::plan_flush(p.nt1, p.nq1, R, G) : p.nq1;
    (void)hipGetLastError();
    if (nq > p.nq0) {
        rc = quantize_blocks(cache, p.nq0 / G, nq / G, nt0, k, v, 1, static_cast<hipStream_t>(stream));
        if (rc != KIVI_OK) return rc;
    }
    cache->n_tokens = p.nt1;
    cache->n_quant = nq;
    if (n_flushed) *n_flushed = (int32_t)(nq - p.nq1);
    return attend_call(cache, q, q_dtype, out, stream, k, v, nt0 >= nq ? nt0 : -1);
}

}  // extern "C"
