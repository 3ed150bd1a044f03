"""CPU checks of the C ABI and of the host planner (no GPU needed).

* libkivi.so loads and exports every function include/kivi.h declares;
* argument validation returns the documented error codes before anything
  would be launched;
* the layout matches its closed form;
* the host planner (planner.hpp, built here with g++ through a small shim)
  reproduces the oracle's token-by-token residual ring on call sequences.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kivi.h")


@pytest.fixture(scope="module")
def native():
    from kv_cache_compression_kivi_amd import _native
    if not os.path.exists(_native.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return _native


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kivi_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(native):
    lib = native.load_library()
    declared = _declared_functions()
    assert "kivi_attend_decode" in declared and "kivi_append" in declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(native.EXPORTED)
    assert native.kivi_abi_version() == native.ABI_VERSION == 5
    nm = subprocess.run(["nm", "-D", "--defined-only", native.library_path()], capture_output=True, text=True).stdout
    for name in declared:
        assert re.search(r"\bT " + name + r"\b", nm), name


def _cfg(native, **kw):
    base = dict(batch=2, n_kv_heads=4, n_q_heads=8, head_dim=128, bits=2, max_tokens=1000)
    base.update(kw)
    return native.make_config(**base)


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=96), "KIVI_E_UNSUPPORTED"),
    (dict(bits=3), "KIVI_E_UNSUPPORTED"),
    (dict(k_block=16), "KIVI_E_UNSUPPORTED"),
    (dict(v_group=64), "KIVI_E_UNSUPPORTED"),
    (dict(n_q_heads=6), "KIVI_E_INVAL"),
    (dict(batch=0), "KIVI_E_INVAL"),
    (dict(residual=100), "KIVI_E_INVAL"),
    (dict(max_splits=1), "KIVI_E_INVAL"),
    (dict(batch=70000, n_kv_heads=1, n_q_heads=1), "KIVI_E_INVAL"),
    (dict(squat_rank=-1), "KIVI_E_INVAL"),
    (dict(squat_rank=33), "KIVI_E_UNSUPPORTED"),
    (dict(squat_rank=4, head_dim=256), "KIVI_E_UNSUPPORTED"),
])
def test_config_validation(native, bad, status):
    with pytest.raises(native.KiviError) as e:
        native.kivi_cache_bytes(_cfg(native, **bad))
    assert e.value.status == status
    assert native.kivi_last_error()


@pytest.mark.parametrize("bits,d", [(2, 128), (4, 128), (2, 64), (4, 256)])
def test_layout_closed_form(native, bits, d):
    cfg = _cfg(native, bits=bits, head_dim=d, max_tokens=4096)
    L = native.kivi_cache_layout(cfg)
    G, W = 32, d * bits // 32
    assert (L.rec_kcode, L.rec_vcode, L.rec_ksz, L.rec_vsz) == (0, G * W * 4, 2 * G * W * 4, 2 * G * W * 4 + d * 8)
    assert L.block_bytes == 2 * G * W * 4 + d * 8 + G * (d // 32) * 8
    if d == 128:
        assert L.block_bytes == {2: 4096, 4: 6144}[bits]
    assert L.max_blocks == 128 and L.ring_slots == 160
    units = 2 * 4
    for off in (L.off_blocks, L.off_ring, L.off_partial, L.unit_stride, L.ring_unit_stride, L.total_bytes):
        assert off % 256 == 0
    assert L.off_ring >= units * L.max_blocks * L.block_bytes
    assert L.off_partial >= L.off_ring + units * 160 * 4 * d
    assert L.partial_stride == (d + 4) * 4 and L.max_splits == 256
    assert L.total_bytes >= L.off_partial + 2 * 8 * 256 * L.partial_stride
    assert native.kivi_cache_bytes(cfg) == L.total_bytes
    assert L.off_squat == L.total_bytes  # no coefficient region without the SQuat-style coder
    sq = native.kivi_cache_layout(_cfg(native, bits=bits, head_dim=d, max_tokens=4096, squat_rank=8)) \
        if d <= 128 else None
    if sq is not None:
        assert sq.off_squat % 256 == 0 and sq.off_squat >= L.total_bytes - 255
        assert sq.squat_r8 == 8 and sq.squat_unit_bytes == 2 * d * 8 * 4
        assert sq.total_bytes == sq.off_squat + -(-units * sq.squat_unit_bytes // 256) * 256


def test_squat_build_refusals(native):
    """Host-side checks of kivi_squat_build (nothing is launched)."""
    import ctypes
    lib = native.load_library()
    buf = ctypes.create_string_buffer(8 << 20)
    mem = (ctypes.addressof(buf) + 255) // 256 * 256  # a host address: only validated, never launched on
    plain = _cfg(native, max_tokens=64)
    sq = _cfg(native, max_tokens=64, squat_rank=4)
    for cfg, q, n_q, lam, want in [(plain, 256, 8, 0.1, -1), (sq, 0, 8, 0.1, -1), (sq, 257, 8, 0.1, -1),
                                   (sq, 256, 0, 0.1, -1), (sq, 256, 8, 0.0, -1), (sq, 256, 8, float("inf"), -1),
                                   (sq, 256, 8, float("nan"), -1)]:
        assert native.kivi_cache_bytes(cfg) <= (8 << 20) - 256
        h = native.kivi_cache_create(cfg, mem, (8 << 20) - 256)
        try:
            rc = lib.kivi_squat_build(ctypes.c_void_p(h), ctypes.c_void_p(q), 0, n_q, lam, None)
            assert rc == want, (rc, native.kivi_last_error())
            assert native.kivi_last_error()
        finally:
            native.kivi_cache_destroy(h)


def test_create_and_host_only_calls(native):
    cfg = _cfg(native)
    n = native.kivi_cache_bytes(cfg)
    fake = 1 << 40  # never dereferenced: create and the planning calls launch nothing
    with pytest.raises(native.KiviError) as e:
        native.kivi_cache_create(cfg, fake, n - 1)
    assert e.value.status == "KIVI_E_NOMEM"
    with pytest.raises(native.KiviError) as e:
        native.kivi_cache_create(cfg, fake + 16, n)
    assert e.value.status == "KIVI_E_INVAL"
    h = native.kivi_cache_create(cfg, fake, n)
    try:
        st = native.kivi_cache_query(h)
        assert (st.n_tokens, st.n_quant, st.n_resid) == (0, 0, 0)
        st = native.kivi_plan_append(h, 1000)
        assert (st.n_tokens, st.n_quant, st.n_resid) == (1000, 864, 136)
        with pytest.raises(native.KiviError) as e:
            native.kivi_plan_append(h, 1001)
        assert e.value.status == "KIVI_E_CAPACITY"
        # validation failures happen before any launch and leave the state alone
        with pytest.raises(native.KiviError) as e:
            native.kivi_append(h, fake, fake, 1001)
        assert e.value.status == "KIVI_E_CAPACITY"
        with pytest.raises(native.KiviError) as e:
            native.kivi_append(h, 0, fake, 1)
        assert e.value.status == "KIVI_E_INVAL"
        with pytest.raises(native.KiviError) as e:
            native.kivi_append(h, fake, fake, 0)
        assert e.value.status == "KIVI_E_INVAL"
        with pytest.raises(native.KiviError) as e:
            native.kivi_attend_decode(h, fake, 0, fake)
        assert e.value.status == "KIVI_E_EMPTY"
        with pytest.raises(native.KiviError) as e:
            native.kivi_attend_decode(h, fake, 7, fake)
        assert e.value.status == "KIVI_E_INVAL"
        assert native.kivi_flush(h) == 0  # nothing to flush: no launch
        st = native.kivi_cache_query(h)
        assert (st.n_tokens, st.n_quant) == (0, 0)
        native.kivi_set_attend_splits(h, 3)
        with pytest.raises(native.KiviError):
            native.kivi_set_attend_splits(h, 257)
    finally:
        native.kivi_cache_destroy(h)


def test_row_entry_points_host_only(native):
    """The per-sequence calls validate before anything would be launched, and
    appending nothing launches nothing."""
    cfg = _cfg(native)  # batch 2
    n = native.kivi_cache_bytes(cfg)
    fake = 1 << 40
    h = native.kivi_cache_create(cfg, fake, n)
    try:
        st = native.kivi_query_row(h, 1)
        assert (st.n_tokens, st.n_quant, st.n_resid) == (0, 0, 0)
        for row in (-1, 2):
            for call in (lambda: native.kivi_query_row(h, row), lambda: native.kivi_reset_row(h, row)):
                with pytest.raises(native.KiviError) as e:
                    call()
                assert e.value.status == "KIVI_E_INVAL"
        native.kivi_reset_row(h, 0)
        for ntok, max_ntok, status in [([1, 2], 1, "KIVI_E_INVAL"), ([-1, 0], 4, "KIVI_E_INVAL"),
                                       ([1, 1], 0, "KIVI_E_INVAL"), ([1001, 0], 1001, "KIVI_E_CAPACITY")]:
            with pytest.raises(native.KiviError) as e:
                native.kivi_append_rows(h, fake, fake, ntok, max_ntok)
            assert e.value.status == status, (ntok, max_ntok)
        with pytest.raises(native.KiviError) as e:
            native.kivi_append_rows(h, 0, fake, [1, 1], 1)
        assert e.value.status == "KIVI_E_INVAL"
        native.kivi_append_rows(h, fake, fake, [0, 0], 3)  # nothing to append: no launch
        st = native.kivi_cache_query(h)
        assert (st.n_tokens, st.n_quant, st.n_resid) == (0, 0, 0)
    finally:
        native.kivi_cache_destroy(h)


def test_ragged_batches_beyond_one_row_table(native):
    """Rows of different lengths pass their counters with the kernel
    arguments, KIVI_MAX_RAGGED_BATCH rows a launch; a larger batch (or paged
    cache) runs as several launches (their parity is a GPU test). On the CPU:
    such caches validate and take host-only row operations, and the split
    plan reports the launch with the most splits."""
    assert "#define KIVI_MAX_RAGGED_BATCH 128" in open(HEADER, encoding="utf-8").read()
    fake = 1 << 40
    for extra in (dict(), dict(n_pages=300 * 31)):
        cfg = _cfg(native, batch=300, n_kv_heads=1, n_q_heads=1, **extra)
        n = native.kivi_cache_bytes(cfg)
        h = native.kivi_cache_create(cfg, fake, n)
        try:
            native.kivi_reset_row(h, 299)
            assert native.kivi_query_row(h, 299).n_tokens == 0
            n_split, bps = native.kivi_plan_attend(h)
            assert 1 <= n_split <= native.kivi_cache_layout(cfg).max_splits and bps >= 0
        finally:
            native.kivi_cache_destroy(h)


def test_paged_layout_and_validation(native):
    """Paged blocks: the pool replaces the per-unit regions in the layout, and
    the block-table rules are enforced before anything is launched."""
    for bad, status in [(dict(n_pages=-1), "KIVI_E_INVAL")]:
        with pytest.raises(native.KiviError) as e:
            native.kivi_cache_bytes(_cfg(native, **bad))
        assert e.value.status == status
    cfg = _cfg(native, n_pages=37)  # batch 2, 4 KV heads, d 128, b 2, 1000 tokens
    L = native.kivi_cache_layout(cfg)
    assert L.n_pages == 37 and L.unit_stride == 0 and L.page_bytes == 4 * L.block_bytes == 4 * 4096
    assert L.off_ring >= 37 * L.page_bytes and L.off_ring % 256 == 0
    flat = native.kivi_cache_layout(_cfg(native))
    assert flat.n_pages == 0 and flat.page_bytes == 0
    assert L.total_bytes - L.off_ring == flat.total_bytes - flat.off_ring  # ring and partials unchanged
    n = native.kivi_cache_bytes(cfg)
    fake = 1 << 40
    h = native.kivi_cache_create(cfg, fake, n)
    try:
        with pytest.raises(native.KiviError) as e:
            native.kivi_append(h, fake, fake, 1)
        assert e.value.status == "KIVI_E_INVAL" and "block table" in native.kivi_last_error()
        for ptr, stride in [(0, 31), (fake + 2, 31), (fake, 30)]:
            with pytest.raises(native.KiviError) as e:
                native.kivi_set_block_table(h, ptr, stride)
            assert e.value.status == "KIVI_E_INVAL"
        native.kivi_set_block_table(h, fake, 31)  # max_blocks = 1000 // 32 = 31
        native.kivi_append_rows(h, fake, fake, [0, 0], 1)  # nothing to append: no launch
    finally:
        native.kivi_cache_destroy(h)
    h = native.kivi_cache_create(_cfg(native), fake, native.kivi_cache_bytes(_cfg(native)))
    try:
        with pytest.raises(native.KiviError) as e:
            native.kivi_set_block_table(h, fake, 31)
        assert e.value.status == "KIVI_E_INVAL"
    finally:
        native.kivi_cache_destroy(h)


# ---------------------------------------------------------------- host planner

SHIM = r"""
#include "planner.hpp"
#include "split.hpp"
extern "C" {
void shim_plan_append(int64_t nt, int64_t nq, int64_t ntok, int64_t R, int64_t G, int64_t* out) {
    kivi::AppendPlan p = kivi::plan_append(nt, nq, ntok, R, G);
    out[0] = p.nt1; out[1] = p.nq1; out[2] = p.ring_t0;
}
int64_t shim_plan_flush(int64_t nt, int64_t nq, int64_t R, int64_t G) { return kivi::plan_flush(nt, nq, R, G); }
void shim_plan_attend(int64_t units, int32_t group, int32_t d, int64_t nb, int32_t max_splits, int32_t forced,
                      int32_t cus, int32_t* out) {
    kivi::AttendPlan p = kivi::plan_attend(units, group, d, nb, max_splits, forced, cus);
    out[0] = p.n_split; out[1] = p.blocks_per_split; out[2] = p.qg; out[3] = p.nwaves;
}
void shim_split_range(int64_t nb, int64_t nrc, int64_t cost, int64_t n, int64_t s, int64_t* out) {
    kivi::split_range(nb, nrc, cost, n, s, &out[0], &out[1]);
}
int64_t shim_wave_blocks(int64_t nbw, int64_t nw, int64_t w) { return kivi::wave_blocks(nbw, nw, w); }
int64_t shim_residual_wave(int64_t c, int64_t nw) {
    return kivi::residual_wave(c, nw);
}
void shim_plan_rows(int64_t hkv, int32_t group, int32_t d, int64_t rows, const int64_t* cost, int64_t nb_max,
                    int32_t max_splits, int32_t forced, int32_t cus, int32_t* out, int64_t* cost_max) {
    kivi::AttendPlan p = kivi::plan_attend_rows(hkv, group, d, rows, cost, nb_max, max_splits, forced, cus, cost_max);
    out[0] = p.n_split; out[1] = p.blocks_per_split; out[2] = p.qg; out[3] = p.nwaves;
}
int64_t shim_row_split_count(int64_t c, int64_t cm, int64_t n) { return kivi::row_split_count(c, cm, n); }
int shim_gqa_row_token(int bits, int m) { return bits == 2 ? kivi::gqa_row_token<2>(m) : kivi::gqa_row_token<4>(m); }
int shim_gqa_channel(int bits, int kc, int q, int s) {
    return bits == 2 ? kivi::gqa_channel<2>(kc, q, s) : kivi::gqa_channel<4>(kc, q, s);
}
int64_t shim_unit_cost(int64_t nb, int64_t nres) { return kivi::unit_cost(nb, nres); }
int64_t shim_gqa_fold_blocks() { return kivi::kGqaFoldBlocks; }
int64_t shim_gqa_block_digit_sum_max() { return kivi::kGqaBlockDigitSumMax; }
}
"""


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    d = tmp_path_factory.mktemp("planner")
    src = d / "shim.cpp"
    src.write_text(SHIM)
    so = d / "libshim.so"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-fPIC", "-shared",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "kv_cache_compression_kivi_amd", "csrc"),
                           str(src), "-o", str(so)])
    lib = ctypes.CDLL(str(so))
    i64 = ctypes.c_int64
    lib.shim_plan_append.argtypes = [i64] * 5 + [ctypes.c_void_p]
    lib.shim_plan_flush.argtypes = [i64] * 4
    lib.shim_plan_flush.restype = i64
    i32 = ctypes.c_int32
    lib.shim_plan_attend.argtypes = [i64, i32, i32, i64, i32, i32, i32, ctypes.c_void_p]
    lib.shim_split_range.argtypes = [i64] * 5 + [ctypes.c_void_p]
    lib.shim_wave_blocks.argtypes = [i64] * 3
    lib.shim_wave_blocks.restype = i64
    lib.shim_residual_wave.argtypes = [i64] * 2
    lib.shim_residual_wave.restype = i64
    lib.shim_plan_rows.argtypes = [i64, i32, i32, i64, ctypes.c_void_p, i64, i32, i32, i32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.shim_gqa_row_token.argtypes = [ctypes.c_int] * 2
    lib.shim_gqa_channel.argtypes = [ctypes.c_int] * 4
    lib.shim_row_split_count.argtypes = [i64] * 3
    lib.shim_row_split_count.restype = i64
    lib.shim_unit_cost.argtypes = [i64] * 2
    lib.shim_unit_cost.restype = i64
    lib.shim_gqa_fold_blocks.restype = i64
    lib.shim_gqa_block_digit_sum_max.restype = i64
    return lib


def _plan_append(lib, nt, nq, ntok, R, G=32):
    out = np.zeros(3, np.int64)
    lib.shim_plan_append(nt, nq, ntok, R, G, out.ctypes.data_as(ctypes.c_void_p))
    return tuple(int(x) for x in out)


@pytest.mark.parametrize("R", [128, 0, 64])
def test_planner_matches_oracle_sequences(planner, oracle_mod, R):
    """Random append/flush sequences: the planner's closed forms give the same
    counters as the oracle's token-by-token ring after every call."""
    rng = np.random.default_rng(R + 1)
    d, G = 32, 32
    for trial in range(6):
        T = 3000
        oc = oracle_mod.OracleCache(1, 1, 1, d, 2, max_tokens=T, residual=R)
        nt, nq = 0, 0
        while nt < T - 300:
            if rng.random() < 0.3:
                k = int(planner.shim_plan_flush(nt, nq, R, G))
                assert k == oc.flush()
                nq += k
            else:
                ntok = int(rng.choice([1, 1, 1, 2, 31, 32, 33, 100, 160, 161, 250]))
                nt1, nq1, ring_t0 = _plan_append(planner, nt, nq, ntok, R)
                x = np.zeros((1, 1, ntok, d), np.float16)
                oc.append(x, x)
                assert (nt1, nq1) == oc.state(), (nt, nq, ntok)
                assert ring_t0 == max(nq1, nt)
                assert 0 <= nt1 - nq1 <= R + G
                nt, nq = nt1, nq1


def test_planner_config_states(planner):
    """Prefill append(T) + flush gives n_q = floor((T - R) / G) * G for the workloads' T."""
    for T, want in [(1024, 896), (4096, 3968), (8192, 8064), (131072, 130944)]:
        nt, nq, _ = _plan_append(planner, 0, 0, T, 128)
        nq += int(planner.shim_plan_flush(nt, nq, 128, 32))
        assert nq == want


@pytest.mark.parametrize("cus", [256, 32, 80, 304])
def test_attend_plan(planner, cus):
    out = np.zeros(4, np.int32)
    p = out.ctypes.data_as(ctypes.c_void_p)
    # (units, group, head_dim, key blocks) -> the automatic split count of the five workloads on 256 CUs
    if cus == 256:
        for args, want in [((1, 1, 128, 28), 1), ((256, 1, 128, 124), 1), ((32, 1, 128, 4092), 8),
                           ((512, 4, 128, 255), 1), ((1024, 4, 128, 124), 1)]:
            planner.shim_plan_attend(*args, 256, 0, cus, p)
            assert int(out[0]) == want, (args, out)
    for units, group, d in [(1, 1, 128), (7, 2, 64), (3, 4, 256), (2, 3, 128), (32, 1, 128)]:
        for nb in (0, 1, 31, 4092):
            for forced in (0, 1, 3, 17, 300):
                planner.shim_plan_attend(units, group, d, nb, 256, forced, cus, p)
                n, bps, qg, nw = (int(x) for x in out)
                assert 1 <= n <= 256 and group % qg == 0 and nw in (4, 8, 16)
                if forced:
                    assert n == min(forced, 256)
                else:
                    # one round of work-groups over the device's CUs (8 waves each), unless the
                    # two-blocks-per-wave floor or max_splits caps it, and never below 1
                    wgs_per_split = units * (group // qg)
                    want = -(-(cus * 8) // (wgs_per_split * nw))
                    want = max(1, min(want, nb // (2 * nw), 256))
                    assert n == want, (units, group, d, nb, cus, n, want)


def test_gqa_value_sums_fit_int32(planner):
    """The four-query kernel's int32 value digit sums: a block adds at most
    |digit| * code * tokens = 128 * (2^4 - 1) * 32 to a sum (signed-byte
    digits, 4-bit codes, 32 tokens a block), and the kernel folds the sums into
    fp32 at least every kGqaFoldBlocks blocks, so no sum can leave int32
    whatever a wave's share of blocks (a forced single split over a unit of
    millions of tokens included)."""
    per_block = 128 * ((1 << 4) - 1) * 32
    assert planner.shim_gqa_block_digit_sum_max() == per_block
    k = planner.shim_gqa_fold_blocks()
    assert 1 <= k and k * per_block < 2 ** 31
    # the largest wave share a config allows: 4 GiB of b = 2 records in one split, over 4 waves
    max_blocks_per_unit = (1 << 32) // 4096
    assert max_blocks_per_unit // 4 > k  # the bound, not the share, is what keeps the sums in range


@pytest.mark.parametrize("cost", [2, 4])
def test_split_and_wave_ranges_cover_every_block_once(planner, cost):
    """The attention kernel's division of a unit's work: every key block goes
    to exactly one wave of one split, the residual to the last split, and the
    per-wave cost (blocks plus residual chunks at their cost) within cost + 1
    of the mean."""
    buf = np.zeros(2, np.int64)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    rng = np.random.default_rng(cost)
    cases = [(124, 4, 1, 16), (4092, 4, 8, 16), (28, 4, 1, 16), (0, 5, 1, 16), (3, 5, 2, 8), (255, 5, 1, 4)]
    cases += [(int(rng.integers(0, 5000)), int(rng.integers(0, 6)), int(rng.integers(1, 40)),
               int(rng.choice([4, 8, 16]))) for _ in range(200)]
    for nb, nrc, n, nw in cases:
        seen = np.zeros(nb, np.int64)
        prev_end = 0
        for s in range(n):
            planner.shim_split_range(nb, nrc, cost, n, s, p)
            b0, b1 = int(buf[0]), int(buf[1])
            assert b0 == prev_end and b0 <= b1
            prev_end = b1
            rc = nrc if s == n - 1 else 0
            # round robin inside the work-group: wave w holds blocks b0 + w + k * nw
            counts = [int(planner.shim_wave_blocks(b1 - b0, nw, w)) for w in range(nw)]
            assert sum(counts) == b1 - b0
            for w in range(nw):
                for j in range(b0 + w, b1, nw):
                    seen[j] += 1
                assert counts[w] == len(range(b0 + w, b1, nw))
            chunks = [0] * nw
            for c in range(rc):
                wv = int(planner.shim_residual_wave(c, nw))
                assert 0 <= wv < nw
                chunks[wv] += 1
            total = (b1 - b0) + cost * rc
            loads = [counts[w] + cost * chunks[w] for w in range(nw)]
            assert max(loads) <= total / nw + cost + 1, (nb, nrc, n, nw, loads)
        assert prev_end == nb
        assert np.all(seen == 1)


def test_ragged_split_plan(planner):
    """Rows of different lengths: the costliest row takes all n splits, every
    row's splits cover its key blocks exactly once with the residual in its
    last split, no row's splits average more than cost_max / n, and n is the
    largest count whose work-groups fit one round over the CUs."""
    rng = np.random.default_rng(3)
    out = np.zeros(4, np.int32)
    cmax_buf = np.zeros(1, np.int64)
    rng_buf = np.zeros(2, np.int64)
    for trial in range(60):
        rows = int(rng.integers(1, 129))
        hkv = int(rng.choice([1, 8, 32]))
        group = int(rng.choice([1, 2, 4, 8]))
        lens = rng.integers(1, 20000, rows)
        nq = np.maximum(0, (lens - 128) // 32 * 32)
        nb, nres = nq // 32, lens - nq
        cost = np.array([planner.shim_unit_cost(int(a), int(r)) for a, r in zip(nb, nres)], np.int64)
        forced = int(rng.choice([0, 0, 0, 3, 50]))
        cus = int(rng.choice([256, 256, 32, 304]))
        planner.shim_plan_rows(hkv, group, 128, rows, cost.ctypes.data_as(ctypes.c_void_p), int(nb.max()), 256,
                               forced, cus, out.ctypes.data_as(ctypes.c_void_p),
                               cmax_buf.ctypes.data_as(ctypes.c_void_p))
        n, qg, nw = int(out[0]), int(out[2]), int(out[3])
        cmax = int(cmax_buf[0])
        assert cmax == cost.max() and 1 <= n <= 256
        if forced:
            assert n == forced
        wgs = 0
        for r in range(rows):
            nr = int(planner.shim_row_split_count(int(cost[r]), cmax, n))
            assert 1 <= nr <= n
            if cost[r] == cmax:
                assert nr == n
            assert cost[r] / nr <= cmax / n + 1e-9
            prev = 0
            for s_ in range(nr):
                planner.shim_split_range(int(nb[r]), int((nres[r] + 31) // 32), 2, nr, s_,
                                         rng_buf.ctypes.data_as(ctypes.c_void_p))
                assert int(rng_buf[0]) == prev and int(rng_buf[1]) >= prev
                prev = int(rng_buf[1])
            assert prev == nb[r]
            wgs += nr * hkv * (group // qg)
        if not forced:
            # the largest n whose work-groups fit one round of cus * 8 / nw (n = 1 if none does)
            target = cus * 8 // nw
            cap = min(256, max(1, int(nb.max()) // (2 * nw)))
            assert n == 1 or wgs <= target, (n, wgs, target)
            if n < cap:
                more = sum(int(planner.shim_row_split_count(int(c), cmax, n + 1)) for c in cost) * hkv * (group // qg)
                assert more > target, (n, more, target)


@pytest.mark.parametrize("bits", [2, 4])
def test_four_query_operand_layouts(planner, bits):
    """The four-query kernel's lane-to-data maps: a score operand's bytes over
    the four lane groups cover each 64-channel chunk once; score columns map
    onto a tile's 16 tokens one to one, so each row of 16 lanes reads every
    (token, value group) scale of a block once; and the four columns of a quad
    hold exactly the tokens of bytes 4e .. 4e + 3 of value operand q = 2 tt + c / 2
    (e = c % 2), whose byte s = 4e + k holds token 16 (q / 2) + 4k + 2 (q % 2) + e
    at b = 2 and 8q + 2k + e at b = 4."""
    for kc in range(2):
        ch = sorted(planner.shim_gqa_channel(bits, kc, q, s_) for q in range(4) for s_ in range(16))
        assert ch == list(range(64 * kc, 64 * kc + 64))
    rt = [planner.shim_gqa_row_token(bits, m) for m in range(16)]
    assert sorted(rt) == list(range(16))
    # lane n of a row reads group n % 4 of the tokens of columns 4 (n // 4) + r
    pairs = sorted((16 * tt + rt[4 * (n // 4) + r], n % 4) for n in range(16) for r in range(4) for tt in range(2))
    assert pairs == [(t, g) for t in range(32) for g in range(4)]
    for tt in range(2):
        for c in range(4):
            q, e = 2 * tt + c // 2, c % 2
            cols = {16 * tt + rt[4 * c + i] for i in range(4)}
            if bits == 2:
                want = {16 * (q // 2) + 4 * k + 2 * (q % 2) + e for k in range(4)}
            else:
                want = {8 * q + 2 * k + e for k in range(4)}
            assert cols == want, (bits, tt, c)


DIV_CHECK_MAIN = r"""
#include <cstdint>
#include <cstdio>
#include <cstring>
#include "codec_math.hpp"
int main() {
    const float ys[2] = {3.0f, 15.0f};
    unsigned long long bad = 0, n = 0;
    for (float y : ys) {
        for (uint32_t u = 0x33800000u; u <= 0x48000000u; ++u) {  // every fp32 in [2^-24, 2^17]
            float x;
            std::memcpy(&x, &u, 4);
            const float want = x / y;
            const float got = kivi::div_by_levels(x, y, 1.0f / y);
            ++n;
            if (std::memcmp(&want, &got, 4) != 0) ++bad;
        }
        const float z = kivi::div_by_levels(0.0f, y, 1.0f / y);
        ++n;
        if (z != 0.0f || std::signbit(z)) ++bad;
    }
    std::printf("%llu %llu\n", n, bad);
    return 0;
}
"""


def test_quantizer_division_is_exact(tmp_path):
    """The quantizer's scale (max - min) / (2^b - 1) without a division
    (codec_math.hpp: div_by_levels, the code the kernel runs) equals IEEE fp32
    division for every possible range: 0 and every fp32 in [2^-24, 2^17], for
    b = 2 and 4."""
    src = tmp_path / "divcheck.cpp"
    src.write_text(DIV_CHECK_MAIN)
    exe = tmp_path / "divcheck"
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-ffp-contract=off",
                           "-I", os.path.join(ROOT, "kv_cache_compression_kivi_amd", "csrc"), str(src), "-o", str(exe)])
    n, bad = (int(x) for x in subprocess.check_output([str(exe)], timeout=300).split())
    assert n == 2 * (0x48000000 - 0x33800000 + 2)
    assert bad == 0


SANITIZED_MAIN = r"""
#include <cstdio>
#include <cstdlib>
#include "planner.hpp"
#include "split.hpp"
int main() {
    // random append/flush walks under ASan/UBSan: counters stay consistent
    unsigned x = 12345;
    for (int R = 0; R <= 256; R += 32) {
        int64_t nt = 0, nq = 0;
        for (int step = 0; step < 20000; ++step) {
            x = x * 1103515245u + 12345u;
            if ((x >> 16) % 4 == 0) {
                nq += kivi::plan_flush(nt, nq, R, 32);
            } else {
                int64_t ntok = 1 + (x >> 8) % 200;
                kivi::AppendPlan p = kivi::plan_append(nt, nq, ntok, R, 32);
                if (p.nq1 % 32 || p.nt1 - p.nq1 > R + 32 || p.nt1 - p.nq1 < 0 || p.ring_t0 < p.nq1) return 1;
                nt = p.nt1; nq = p.nq1;
            }
            kivi::AttendPlan a = kivi::plan_attend(1 + (x >> 4) % 2000, 1 << ((x >> 2) % 4), 128, nq / 32, 256,
                                                   (x >> 3) % 5, 32 + (x >> 6) % 300);
            if (a.n_split < 1 || a.n_split > 256) return 2;
            int64_t b0, b1, prev = 0;
            for (int s = 0; s < a.n_split; ++s) {
                kivi::split_range(nq / 32, (nt - nq + 31) / 32, 4, a.n_split, s, &b0, &b1);
                if (b0 != prev || b1 < b0) return 4;
                prev = b1;
            }
            if (prev != nq / 32) return 5;
        }
    }
    // rows of different lengths: the row plan and each row's splits cover its blocks
    for (int trial = 0; trial < 3000; ++trial) {
        x = x * 1103515245u + 12345u;
        const int rows = 1 + (x >> 16) % 128;
        int64_t cost[128], nbs[128], nrs[128], nb_max = 0;
        for (int r = 0; r < rows; ++r) {
            x = x * 1103515245u + 12345u;
            const int64_t len = 1 + (x >> 8) % 200000;
            const int64_t nq = len >= 160 ? (len - 128) / 32 * 32 : 0;
            nbs[r] = nq / 32;
            nrs[r] = len - nq;
            cost[r] = kivi::unit_cost(nbs[r], nrs[r]);
            nb_max = nbs[r] > nb_max ? nbs[r] : nb_max;
        }
        int64_t cmax = 0;
        kivi::AttendPlan a = kivi::plan_attend_rows(1 + (x >> 4) % 32, 1 << ((x >> 2) % 4), 128, rows, cost, nb_max,
                                                    4096, (x >> 3) % 7 == 0 ? 1 + (x >> 5) % 300 : 0,
                                                    32 + (x >> 6) % 300, &cmax);
        if (a.n_split < 1 || a.n_split > 4096) return 6;
        for (int r = 0; r < rows; ++r) {
            const int64_t n = kivi::row_split_count(cost[r], cmax, a.n_split);
            if (n < 1 || n > a.n_split) return 7;
            int64_t b0, b1, prev = 0;
            for (int64_t s = 0; s < n; ++s) {
                kivi::split_range(nbs[r], (nrs[r] + 31) / 32, kivi::kResidualChunkCost, n, s, &b0, &b1);
                if (b0 != prev || b1 < b0) return 8;
                prev = b1;
            }
            if (prev != nbs[r]) return 9;
        }
    }
    kivi_config c{8, 32, 32, 128, 2, 32, 32, 128, 4096, 0, 0};
    std::string err;
    if (kivi::validate_config(&c, err) != KIVI_OK) return 3;
    kivi_layout L;
    kivi::compute_layout(&c, &L);
    std::printf("ok %zu\n", L.total_bytes);
    return 0;
}
"""


def test_planner_under_sanitizers(tmp_path):
    src = tmp_path / "main.cpp"
    src.write_text(SANITIZED_MAIN)
    exe = tmp_path / "planner_san"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "kv_cache_compression_kivi_amd", "csrc"),
                           str(src), "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
