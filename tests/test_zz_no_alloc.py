"""kivi_attend_decode_noalloc (split partials in the library's static device
scratch) against kivi_attend_decode (partials in the cache's region), through
the C ABI: the same kernels and plan, so the outputs must agree bit for bit,
and both must meet the attention bar against the oracle. Two calls in a row,
the second on a smaller cache, then a plan whose partials exceed the scratch,
which must be refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compression_kivi_amd as kv
import oracle
from kivi_inputs import KVWorkload
from kivi_testlib import assert_attention_close

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _filled(B, Hkv, Hq, d, bits, T, seed, splits):
    wl = KVWorkload(B, Hkv, d, seed=seed, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    cache.set_attend_splits(splits)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    return wl, cache, oc


def _both(cache, q):
    lib = kv.load_library()
    qd = kv.KIVI_BF16 if q.dtype == torch.bfloat16 else kv.KIVI_F16
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    got = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    rc = lib.kivi_attend_decode(ctypes.c_void_p(cache.handle), ctypes.c_void_p(q.data_ptr()), qd,
                                ctypes.c_void_p(ref.data_ptr()), s)
    assert rc == 0, kv.kivi_last_error()
    rc = lib.kivi_attend_decode_noalloc(ctypes.c_void_p(cache.handle), ctypes.c_void_p(q.data_ptr()), qd,
                                        ctypes.c_void_p(got.data_ptr()), s)
    assert rc == 0, kv.kivi_last_error()
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_attend_decode_twice():
    # first call: four query heads per KV head (matrix-core kernel), 7 splits
    print("\n[case] noalloc 1: B2 kv2 q8 d128 b2 T3000 splits 7", flush=True)
    wl, cache, oc = _filled(2, 2, 8, 128, 2, 3000, seed=41, splits=7)
    assert cache.plan_attend()[0] == 7
    q = wl.q(8, dtype=torch.bfloat16)
    ref, got = _both(cache, q.to(DEV))
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    assert_attention_close(got, oc.attend(q, q_is_bf16=True))
    # second call, smaller: one query head per KV head (vector kernel), d = 64, 3 splits
    print("[case] noalloc 2: B1 kv1 q1 d64 b4 T500 splits 3", flush=True)
    wl2, cache2, oc2 = _filled(1, 1, 1, 64, 4, 500, seed=42, splits=3)
    assert cache2.plan_attend()[0] == 3
    q2 = wl2.q(1)
    ref2, got2 = _both(cache2, q2.to(DEV))
    assert np.array_equal(ref2.view(np.uint32), got2.view(np.uint32))
    assert_attention_close(got2, oc2.attend(q2))
    # and the automatic plan (no split for this shape: no scratch used)
    cache2.set_attend_splits(0)
    ref3, got3 = _both(cache2, q2.to(DEV))
    assert np.array_equal(ref3.view(np.uint32), got3.view(np.uint32))


@pytest.mark.parametrize("Hq", [8, 2], ids=["four_query", "mha"])
def test_noalloc_on_paged_rows(Hq):
    """A paged cache whose rows differ in length (the kernels built with a row
    table; short rows see idle splits) at 5 forced splits: the allocation-free
    call bit for bit against kivi_attend_decode, and each row against an oracle
    cache of that row alone."""
    print(f"\n[case] noalloc paged rows: B3 kv2 q{Hq} d128 b2 lens 700/33/1200 splits 5", flush=True)
    B, Hkv, d, bits = 3, 2, 128, 2
    lens = [700, 33, 1200]
    T = max(lens)
    mb = T // 32 + 1
    n_pages = B * mb + 3
    table = np.random.default_rng(44).permutation(n_pages).astype(np.int32)[:B * mb].reshape(B, mb)
    wl = KVWorkload(B, Hkv, d, seed=44, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV, n_pages=n_pages)
    cache.set_block_table(torch.from_numpy(table).to(DEV))
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    cache.flush()
    cache.set_attend_splits(5)
    q = wl.q(Hq)
    ref, got = _both(cache, q.to(DEV))
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    for b in range(B):
        oc = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=T)
        oc.append(k[b:b + 1, :, :lens[b]].contiguous(), v[b:b + 1, :, :lens[b]].contiguous())
        oc.flush()
        assert_attention_close(got[b:b + 1], oc.attend(q[b:b + 1]))


def test_noalloc_beyond_one_row_table():
    """150 rows of different lengths: the call runs two launches (128 rows,
    then 22), whose split partials take the scratch in turn, in stream order.
    Bit for bit against kivi_attend_decode, twice in a row, and a sample of
    rows against oracle caches of those rows alone."""
    print("\n[case] noalloc 150 ragged rows: kv2 q8 d128 b2 splits 3", flush=True)
    B, Hkv, Hq, d, bits = 150, 2, 8, 128, 2
    rng = np.random.default_rng(45)
    lens = [int(x) for x in rng.integers(1, 300, B)]
    T = max(lens)
    wl = KVWorkload(B, Hkv, d, seed=45, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV)
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    cache.set_attend_splits(3)
    q = wl.q(Hq)
    for _ in range(2):
        ref, got = _both(cache, q.to(DEV))
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    for b in (0, 127, 128, 149):
        oc = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=T)
        oc.append(k[b:b + 1, :, :lens[b]].contiguous(), v[b:b + 1, :, :lens[b]].contiguous())
        assert_attention_close(got[b:b + 1], oc.attend(q[b:b + 1]))


def test_noalloc_refuses_partials_beyond_the_scratch():
    print("\n[case] noalloc too large: B64 kv8 q32 d128 splits 256", flush=True)
    B, Hkv, Hq, d = 64, 8, 32, 128
    wl = KVWorkload(B, Hkv, d, seed=43, device=DEV)
    k, v = wl.kv(0, 40)
    cache = kv.KiviCache(B, Hkv, Hq, d, 2, max_tokens=40, device=DEV)
    cache.append(k, v)
    cache.set_attend_splits(256)
    q = wl.q(Hq)
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device=DEV)
    lib = kv.load_library()
    rc = lib.kivi_attend_decode_noalloc(ctypes.c_void_p(cache.handle), ctypes.c_void_p(q.data_ptr()), kv.KIVI_F16,
                                        ctypes.c_void_p(out.data_ptr()), None)
    assert rc == -3, (rc, kv.kivi_last_error())  # KIVI_E_NOMEM
    assert "static scratch" in kv.kivi_last_error()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0  # nothing ran
