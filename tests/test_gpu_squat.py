"""GPU parity of the SQuat-style key coder (kivi_squat_build and the key codes
of every quantize launch on a cache with squat_rank > 0) against the oracle
(oracle/squat.py for the coefficients, or_squat_token for the codes).

* coefficients: each unit's g[c][j] = u_j . w_c from the device's U, W
  (computed in the subspace's coordinates, fp64, stored fp32) against the
  oracle's fp64 Cholesky route from the same past queries, within 1e-4 of the
  largest coefficient; and the closed form of the all-ones direction;
* codes: scales, zeros, value codes and residual rows bit-exact (they are the
  plain coder's); key codes judged by walking the oracle along them
  (kivi_testlib.squat_code_check): a key code may differ from the oracle's
  own only across a rounding boundary its quotient lies within 1e-3 of, since
  the two sides' coefficients differ in their last bits; the number of such
  codes is reported and bounded;
* attention over such a cache against the oracle's attention over its own.
Source: the SQuat explainer page (aibr.jp, "SQuat"), section 3
中核となる技術的要素.
"""

import numpy as np
import pytest
import torch

import kv_cache_compression_kivi_amd as kv
import oracle
from oracle import squat
from kivi_inputs import KVWorkload, query_history
from kivi_testlib import assert_attention_close, compare_unit, gpu_unit_blocks, squat_code_check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LAM = 0.1


def _announce(*parts):
    print("\n[case]", *parts, flush=True)


def _oracle_coefficients(qh, Hkv, rank, lam):
    """Oracle coefficients per unit from the past queries qh [B, Hq, n, d] (cpu)."""
    B, Hq, n, d = qh.shape
    group = Hq // Hkv
    q64 = qh.float().numpy().astype(np.float64)
    gs = []
    for b in range(B):
        for h in range(Hkv):
            qu = q64[b, h * group:(h + 1) * group].reshape(-1, d)
            gs.append(squat.unit_coefficients(qu, rank, lam))
    return np.stack(gs)


def _device_g(cache, unit):
    """g[c][j] = u_j . w_c (j > c, 0 elsewhere) from the device's U, W, in fp64."""
    U, W = (x.cpu().numpy().astype(np.float64) for x in cache.squat_factors(unit))
    return np.triu(W @ U.T, k=1)


def _key_codes(cache, unit, nq):
    """[nq, d] key codes of a unit's quantized tokens, unpacked from the device records."""
    c = cache.cfg
    kcode, _, ksz, _ = gpu_unit_blocks(cache, unit, nq // 32)
    words = kcode.reshape(nq, -1)
    per = 32 // c.bits
    shifts = (np.arange(c.head_dim) % per) * c.bits
    return ((words[:, np.arange(c.head_dim) // per] >> shifts) & ((1 << c.bits) - 1)).astype(np.uint8), ksz


def _check_unit(cache, oc, gu, ou, kf, g):
    """Everything but the key codes bit-exact; the key codes valid."""
    nt, nq = oc.state()
    # the plain parts: compare with the key codes of the oracle replaced by the device's
    codes, ksz = _key_codes(cache, gu, nq)
    s = np.repeat(ksz[..., 0], 32, axis=0)
    z = np.repeat(ksz[..., 1], 32, axis=0)
    n_diff, worst = squat_code_check(kf[:nq], s, z, g, cache.cfg.bits, codes)
    okc = oc.unit_quantized(ou)[0]
    compare_unit(cache, oc, gu, ou, key_codes=False)
    return n_diff, worst, int((okc != codes).sum())


@pytest.mark.parametrize("B,Hkv,Hq,d,bits,rank,T,q_dtype", [
    (2, 2, 8, 128, 2, 8, 700, torch.float16),    # four query heads per KV head
    (1, 2, 2, 64, 4, 4, 333, torch.bfloat16),    # d = 64, b = 4, bf16 past queries
    (2, 1, 4, 128, 4, 16, 300, torch.float16),
    (1, 1, 1, 128, 2, 1, 1024, torch.float16),   # one query head, rank 1
    (1, 3, 3, 128, 2, 32, 500, torch.float16),   # the largest rank
    (1, 2, 2, 64, 2, 20, 400, torch.float16),    # d = 64, rank padded to 24 columns
])
def test_squat_prefill_parity(B, Hkv, Hq, d, bits, rank, T, q_dtype):
    _announce("squat prefill", B, Hkv, Hq, d, bits, rank, T, q_dtype)
    wl = KVWorkload(B, Hkv, d, seed=40 + rank + d, device="cpu")
    k, v = wl.kv(0, T)
    qh = query_history(wl, Hq, 96, rank=rank, dtype=q_dtype)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV, squat_rank=rank)
    cache.squat_build(qh.to(DEV), LAM)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    q = wl.q(Hq)
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    gs = _oracle_coefficients(qh, Hkv, rank, LAM)
    # coefficients: the device's U, W (fp32) give g[c][j] = u_j . w_c; against the
    # oracle's fp64 Cholesky route, rounded to fp32
    for u in range(B * Hkv):
        err = np.abs(_device_g(cache, u) - gs[u]).max()
        assert err <= 1e-4 * max(np.abs(gs[u]).max(), 1e-3), (u, err)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.set_squat(gs)
    oc.append(k, v)
    oc.flush()
    total = diff = own_diff = 0
    kf = oracle.half_to_float(k).reshape(B * Hkv, T, d)
    for u in range(B * Hkv):
        n, worst, od = _check_unit(cache, oc, u, u, kf[u], gs[u])
        total += oc.state()[1] * d
        diff += n
        own_diff += od
    print(f"  key codes differing from the oracle's own: {own_diff} of {total}; after the replay {diff}", flush=True)
    assert diff <= 1e-3 * total
    assert_attention_close(out.cpu().numpy(), oc.attend(q))


@pytest.mark.parametrize("lam", [1e-2, 10.0])
def test_squat_lambda_range(lam):
    """The objective's weight lambda away from the 0.1 of the other cases: 1e-2
    (larger corrections) and 10 (codes close to the plain coder's).
    Coefficients within 1e-4 of the oracle's, key codes valid by replay,
    attention within the bar."""
    _announce("squat lambda", lam)
    B, Hkv, Hq, d, bits, rank, T = 1, 2, 8, 128, 2, 8, 400
    wl = KVWorkload(B, Hkv, d, seed=61, device="cpu")
    k, v = wl.kv(0, T)
    qh = query_history(wl, Hq, 96, rank=rank)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV, squat_rank=rank)
    cache.squat_build(qh.to(DEV), lam)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    q = wl.q(Hq)
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    gs = _oracle_coefficients(qh, Hkv, rank, lam)
    for u in range(B * Hkv):
        err = np.abs(_device_g(cache, u) - gs[u]).max()
        assert err <= 1e-4 * max(np.abs(gs[u]).max(), 1e-3), (u, err)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.set_squat(gs)
    oc.append(k, v)
    oc.flush()
    kf = oracle.half_to_float(k).reshape(B * Hkv, T, d)
    for u in range(B * Hkv):
        n, worst, od = _check_unit(cache, oc, u, u, kf[u], gs[u])
        print(f"  unit {u}: key codes differing from the oracle's own: {od}; after the replay {n}", flush=True)
        assert n <= 1e-3 * oc.state()[1] * d
    assert_attention_close(out.cpu().numpy(), oc.attend(q))


def test_squat_coefficients_closed_form():
    """Past queries all along the all-ones direction: rank-1 subspace u = 1/sqrt(d),
    and g[c][j] = -1 / (lambda d + d - 1 - c) for j > c."""
    _announce("squat closed form")
    B, Hkv, Hq, d, lam = 1, 2, 4, 128, 0.3
    coef = torch.randn(B, Hq, 40, 1) * 3
    qh = (coef * torch.ones(B, Hq, 40, d)).half().contiguous()
    cache = kv.KiviCache(B, Hkv, Hq, d, 2, max_tokens=64, device=DEV, squat_rank=1)
    cache.squat_build(qh.to(DEV), lam)
    torch.cuda.synchronize()
    c = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    want = np.where(j > c, -1.0 / (lam * d + d - 1 - c), 0.0)
    for u in range(B * Hkv):
        assert np.abs(_device_g(cache, u) - want).max() <= 1e-5 * np.abs(want).max()


def test_squat_before_build_and_decode_steps():
    """Blocks quantized before kivi_squat_build keep the plain codes (bit-exact
    against the plain oracle); after it, decode steps whose flushes quantize
    the new blocks (R = 32: a flush every 32 steps) code them with the coder;
    a ragged append (rows of different lengths) codes each row's blocks."""
    _announce("squat decode steps")
    B, Hkv, Hq, d, bits, R, rank = 2, 2, 8, 128, 2, 32, 8
    T0, steps = 100, 70
    wl = KVWorkload(B, Hkv, d, seed=77, device="cpu")
    k, v = wl.kv(0, T0)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T0 + steps + 200, residual=R, device=DEV,
                         squat_rank=rank)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    torch.cuda.synchronize()
    plain = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T0 + steps + 200, residual=R)
    plain.append(k, v)
    plain.flush()
    for u in range(B * Hkv):
        compare_unit(cache, plain, u, u)
    nq_plain = plain.state()[1]
    qh = query_history(wl, Hq, 64, rank=rank)
    cache.squat_build(qh.to(DEV), LAM)
    gs = _oracle_coefficients(qh, Hkv, rank, LAM)
    hist_k = [k]
    for i in range(steps):
        kt, vt = wl.kv(T0 + i, 1)
        q = wl.q(Hq, step=i)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), q.to(DEV))
        hist_k.append(kt)
        plain.append(kt, vt)
        nt, nq = plain.state()
        if nt - nq >= R + 32:
            plain.flush()
    # ragged: 40 more tokens to row 0, 7 to row 1, then a flush
    ka, va = wl.kv(T0 + steps, 40)
    cache.append_rows(ka.to(DEV), va.to(DEV), [40, 7])
    n_flushed = cache.flush()
    torch.cuda.synchronize()
    kall = torch.cat(hist_k, dim=2)
    for b, nadd in enumerate([40, 7]):
        rows_k = torch.cat([kall[b:b + 1], ka[b:b + 1, :, :nadd]], dim=2)
        kf = oracle.half_to_float(rows_k)[0]
        nt, nq, _ = cache.row_state(b)
        for h in range(Hkv):
            u = b * Hkv + h
            codes, ksz = _key_codes(cache, u, nq)
            s = np.repeat(ksz[..., 0], 32, axis=0)
            z = np.repeat(ksz[..., 1], 32, axis=0)
            # blocks quantized before the build: plain; after: the coder's
            assert np.array_equal(codes[:nq_plain], plain.unit_quantized(u)[0][:nq_plain])
            n, worst = squat_code_check(kf[h, nq_plain:nq], s[nq_plain:], z[nq_plain:], gs[u], bits,
                                        codes[nq_plain:])
            assert nq >= nq_plain + 64 and n <= 1e-3 * (nq - nq_plain) * d, (b, h, nq, n)


@pytest.mark.parametrize("bits", [2, 4])
def test_squat_degenerate_channels(bits):
    """Key channels that are constant within a block (s floored at 1e-8, so any
    correction saturates the code), signed zeros, fp16 subnormals, and a
    constant token, among moderate keys: every key code a valid rounding of the
    oracle's walk, the plain parts bit-exact, the attention within the bar and
    finite."""
    _announce("squat degenerate channels", bits)
    B, Hkv, Hq, d, rank, T = 1, 1, 4, 128, 8, 32 * 6 + 128 + 5
    wl = KVWorkload(B, Hkv, d, seed=77 + bits, device="cpu")
    k, v = wl.kv(0, T)
    x = k.float().numpy()
    rng = np.random.default_rng(5 + bits)
    x[..., 0] = 3.0                                         # constant channel
    x[..., 1] = 0.0
    x[..., ::2, 1] = -0.0                                   # signed zeros
    x[..., 2] = rng.integers(1, 1024, T) * 2.0 ** -24       # fp16 subnormals
    x[..., 9, :] = 1.5                                      # a constant token
    k = torch.from_numpy(x.astype(np.float16))
    qh = query_history(wl, Hq, 96, rank=rank)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV, squat_rank=rank)
    cache.squat_build(qh.to(DEV), LAM)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    q = wl.q(Hq)
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    gs = _oracle_coefficients(qh, Hkv, rank, LAM)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.set_squat(gs)
    oc.append(k, v)
    oc.flush()
    kf = oracle.half_to_float(k).reshape(B * Hkv, T, d)
    n, worst, od = _check_unit(cache, oc, 0, 0, kf[0], gs[0])
    print(f"  key codes differing from the oracle's own: {od}; after the replay {n}", flush=True)
    assert n <= 1e-3 * oc.state()[1] * d
    assert_attention_close(out.cpu().numpy(), oc.attend(q))


@pytest.mark.parametrize("Hkv,Hq,d,bits,rank,n", [
    (2, 8, 128, 2, 16, 100),   # 400 past queries a unit
    (1, 4, 64, 4, 20, 75),     # d = 64, 300 past queries
    (1, 4, 128, 2, 32, 100),   # the largest rank
])
def test_squat_flat_spectrum(Hkv, Hq, d, bits, rank, n):
    """Past queries with no low-rank structure (small integers, uniform over
    [-8, 8]): the eigenvalues of their Gram matrix fall off slowly, so 48 steps
    of subspace iteration cannot settle on the top r directions, and the build
    takes its Jacobi eigen-decomposition instead. Every query and every Gram
    entry is an exact integer in fp32, so the device's Gram matrix is the
    oracle's, and its subspace is held to the oracle's eigenvectors:
    coefficients within 1e-4, codes valid by replay, attention within the bar."""
    _announce("squat flat spectrum", Hkv, Hq, d, bits, rank, n)
    B, T = 1, 400
    group = Hq // Hkv
    gen = torch.Generator().manual_seed(70 + d + rank)
    qh = torch.randint(-8, 9, (B, Hq, n, d), generator=gen).half().contiguous()
    for h in range(Hkv):
        qu = qh[0, h * group:(h + 1) * group].reshape(-1, d).double().numpy()
        ev = np.linalg.eigvalsh(qu.T @ qu)[::-1]
        ratio = ev[rank] / ev[rank - 1]
        print(f"  KV head {h}: lambda_(r+1) / lambda_r = {ratio:.4f}", flush=True)
        # flat (the iteration's error shrinks by about ratio^2 a step) but
        # separated (the top-r subspace is well defined)
        assert 0.9 < ratio < 1.0 - 1e-6, ratio
    wl = KVWorkload(B, Hkv, d, seed=80 + d, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV, squat_rank=rank)
    cache.squat_build(qh.to(DEV), LAM)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    q = wl.q(Hq)
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    gs = _oracle_coefficients(qh, Hkv, rank, LAM)
    for u in range(B * Hkv):
        err = np.abs(_device_g(cache, u) - gs[u]).max()
        print(f"  unit {u}: coefficient error {err:.3e} (largest {np.abs(gs[u]).max():.3e})", flush=True)
        assert err <= 1e-4 * max(np.abs(gs[u]).max(), 1e-3), (u, err)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.set_squat(gs)
    oc.append(k, v)
    oc.flush()
    kf = oracle.half_to_float(k).reshape(B * Hkv, T, d)
    for u in range(B * Hkv):
        nd, worst, od = _check_unit(cache, oc, u, u, kf[u], gs[u])
        print(f"  unit {u}: key codes differing from the oracle's own: {od}; after the replay {nd}", flush=True)
        assert nd <= 1e-3 * oc.state()[1] * d
    assert_attention_close(out.cpu().numpy(), oc.attend(q))


@pytest.mark.parametrize("span", [3, 0], ids=["three_directions", "all_zero"])
def test_squat_rank_deficient_history(span):
    """Past queries that span fewer directions than the rank: three, or none
    (all zero). The subspace then holds free directions (any orthonormal
    completion of the queries' span has the same top eigenvalues), so the
    device's basis is checked for what is unique: orthonormal columns whose
    span holds every past query. Its coefficients are checked against the
    oracle's formula applied to that same basis, the key codes walked by the
    oracle with those coefficients, and the attention against the bar."""
    _announce("squat rank-deficient history", span)
    B, Hkv, Hq, d, bits, rank, T = 1, 2, 8, 128, 2, 8, 300
    group = Hq // Hkv
    gen = torch.Generator().manual_seed(11 + span)
    if span:
        # small-integer directions and weights: every query is exact in fp16, so
        # the history spans exactly `span` directions
        basis = torch.randint(-1, 2, (d, span), generator=gen).float()
        qh = (torch.randint(-4, 5, (B, Hq, 20, span), generator=gen).float() @ basis.T).half().contiguous()
    else:
        qh = torch.zeros(B, Hq, 20, d, dtype=torch.float16)
    wl = KVWorkload(B, Hkv, d, seed=90 + span, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=DEV, squat_rank=rank)
    cache.squat_build(qh.to(DEV), LAM)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    q = wl.q(Hq)
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    gs = []
    for u in range(B * Hkv):
        U = cache.squat_factors(u)[0].cpu().numpy().astype(np.float64)[:, :rank]
        assert np.abs(U.T @ U - np.eye(rank)).max() <= 1e-5, u
        if span:
            qu = qh[0, u * group:(u + 1) * group].reshape(-1, d).double().numpy()
            resid = qu - (qu @ U) @ U.T
            assert np.linalg.norm(resid) <= 1e-5 * np.linalg.norm(qu), u
        g = squat.coefficients(U, LAM).astype(np.float32)
        err = np.abs(_device_g(cache, u) - g).max()
        assert err <= 1e-4 * max(np.abs(g).max(), 1e-3), (u, err)
        gs.append(g)
    gs = np.stack(gs)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.set_squat(gs)
    oc.append(k, v)
    oc.flush()
    kf = oracle.half_to_float(k).reshape(B * Hkv, T, d)
    for u in range(B * Hkv):
        n, worst, od = _check_unit(cache, oc, u, u, kf[u], gs[u])
        print(f"  unit {u}: key codes differing from the oracle's own: {od}; after the replay {n}", flush=True)
        assert n <= 1e-3 * oc.state()[1] * d
    assert_attention_close(out.cpu().numpy(), oc.attend(q))


def test_squat_paged_rows():
    """The SQuat-style coder on a paged cache whose rows differ in length: the
    coefficients built first, a ragged prefill whose blocks land on scrambled
    pages, then decode steps whose flushes (R = 32) code new blocks on further
    pages. Each row against an oracle cache of that row alone with the oracle's
    own coefficients: key codes valid by replay, the plain parts bit-exact,
    attention within the bar at several steps."""
    _announce("squat paged rows")
    B, Hkv, Hq, d, bits, rank, R = 3, 2, 8, 128, 2, 8, 32
    lens = [300, 77, 520]
    steps = 40
    T = max(lens)
    max_tokens = T + steps + 40
    mb = max_tokens // 32
    n_pages = B * mb + 5
    rng = np.random.default_rng(9)
    table = rng.permutation(n_pages).astype(np.int32)[:B * mb].reshape(B, mb)
    wl = KVWorkload(B, Hkv, d, seed=123, device="cpu")
    k, v = wl.kv(0, T)
    qh = query_history(wl, Hq, 96, rank=rank)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV, n_pages=n_pages,
                         squat_rank=rank)
    cache.set_block_table(torch.from_numpy(table).to(DEV))
    cache.squat_build(qh.to(DEV), LAM)
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    gs = _oracle_coefficients(qh, Hkv, rank, LAM)
    ocs = []
    for b in range(B):
        oc = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R)
        oc.set_squat(gs[b * Hkv:(b + 1) * Hkv])
        oc.append(k[b:b + 1, :, :lens[b]].contiguous(), v[b:b + 1, :, :lens[b]].contiguous())
        ocs.append(oc)
    new_k = []
    for i in range(steps):
        kt, vt = wl.kv(T + i, 1)
        q = wl.q(Hq, step=i + 1)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), q.to(DEV))
        new_k.append(kt)
        for b, oc in enumerate(ocs):
            oc.append(kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
            nt, nq = oc.state()
            if nt - nq >= R + 32:
                oc.flush()
        if i % 13 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            for b, oc in enumerate(ocs):
                assert cache.row_state(b)[:2] == oc.state(), (b, cache.row_state(b), oc.state())
                assert_attention_close(out[b:b + 1].cpu().numpy(), oc.attend(q[b:b + 1]))
    torch.cuda.synchronize()
    kn = torch.cat(new_k, dim=2)
    total = diff = 0
    for b, oc in enumerate(ocs):
        for h in range(Hkv):
            kf = oracle.half_to_float(torch.cat([k[b, h, :lens[b]], kn[b, h]], dim=0).contiguous())
            n, worst, od = _check_unit(cache, oc, b * Hkv + h, h, kf, gs[b * Hkv + h])
            total += oc.state()[1] * d
            diff += n
    print(f"  key codes differing after the replay: {diff} of {total}", flush=True)
    assert diff <= 1e-3 * total
