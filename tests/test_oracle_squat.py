"""Pins of the SQuat-style key coder's oracle (oracle/squat.py for the
subspace and update coefficients, or_squat_token in oracle/kivi_oracle.c for
the codes), against what the mathematics fixes:

* the coefficients in a closed form: for the one-dimensional subspace of the
  all-ones direction, (u u^T + lambda I) restricted to the n = d - c elements
  not yet fixed inverts in closed form, and the optimal step of element j > c
  per unit error of element c is -1 / (lambda d + n - 1);
* each step against a direct solve of the constrained minimum: after fixing
  elements 0..c, the free elements must minimise ||U^T e||^2 + lambda ||e||^2,
  i.e. e_F = -H_FF^-1 H_FQ e_Q, solved here with numpy.linalg.solve;
* the subspace from queries that lie exactly in a known span;
* special cases that reduce to the plain KIVI coder (empty subspace);
* the point of the method: the error's component in the query subspace is far
  smaller than plain rounding's, and inner products with queries from that
  subspace are better preserved;
* the replay used to judge another implementation's codes agrees with the walk.
Source: the SQuat explainer page (aibr.jp, "SQuat"), section 3 中核となる技術的要素.
"""

import numpy as np
import pytest

import oracle
from oracle import squat


@pytest.mark.parametrize("d,lam", [(8, 0.3), (64, 0.1), (128, 0.01), (128, 1.0)])
def test_coefficients_closed_form_all_ones_direction(d, lam):
    u = np.ones((d, 1)) / np.sqrt(d)
    g = squat.coefficients(u, lam)
    c = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    want = np.where(j > c, -1.0 / (lam * d + d - 1 - c), 0.0)
    assert np.abs(g - want).max() < 1e-12


@pytest.mark.parametrize("d,r,lam", [(6, 2, 0.05), (16, 3, 0.2), (32, 8, 0.01)])
def test_each_step_is_the_constrained_minimum(d, r, lam):
    """fp64 walk with the oracle's coefficients and arbitrary fixed values:
    after every step the free elements equal the direct minimiser."""
    rng = np.random.default_rng(d + r)
    u, _ = np.linalg.qr(rng.standard_normal((d, r)))
    g = squat.coefficients(u, lam)
    h = u @ u.T + lam * np.eye(d)
    k = rng.standard_normal(d)
    x = k.copy()
    for c in range(d):
        fixed = np.round(x[c] * 2.0) / 2.0  # any quantizer: a grid of step 1/2
        delta = x[c] - fixed
        x[c] = fixed
        x[c + 1:] -= delta * g[c, c + 1:]
        e = k - x  # error so far (free elements included)
        q, f = np.arange(c + 1), np.arange(c + 1, d)
        if f.size:
            e_f = -np.linalg.solve(h[np.ix_(f, f)], h[np.ix_(f, q)] @ e[q])
            assert np.abs(e[f] - e_f).max() < 1e-9, c


@pytest.mark.parametrize("r", [1, 4, 8])
def test_subspace_of_queries_in_a_known_span(r):
    rng = np.random.default_rng(r)
    d, n = 64, 500
    a = rng.standard_normal((d, r))
    q = (a @ rng.standard_normal((r, n))).T
    u = squat.subspace(q, r)
    assert np.abs(u.T @ u - np.eye(r)).max() < 1e-10
    p_want = a @ np.linalg.solve(a.T @ a, a.T)
    assert np.abs(u @ u.T - p_want).max() < 1e-9


def _block(rng, d=128, G=32, bits=2):
    """A key block (fp16 values, channel spreads as the synthetic keys have
    them) and its KIVI per-channel statistics from the oracle's group quantizer."""
    sigma = np.exp(rng.standard_normal(d))
    k16 = (rng.standard_normal((G, d)) * sigma).astype(np.float16)
    kf = oracle.half_to_float(k16)
    s = np.empty(d, np.float32)
    z = np.empty(d, np.float32)
    kivi = np.empty((G, d), np.uint8)
    for c in range(d):
        codes, s[c], z[c] = oracle.quant_group(kf[:, c], bits)
        kivi[:, c] = codes
    return kf, s, z, kivi


@pytest.mark.parametrize("bits", [2, 4])
def test_empty_subspace_is_plain_kivi(bits):
    rng = np.random.default_rng(bits)
    kf, s, z, kivi = _block(rng, bits=bits)
    g = squat.unit_coefficients(np.zeros((10, 128)), 0, 0.1)
    assert not g.any()
    for t in range(kf.shape[0]):
        assert np.array_equal(oracle.squat_token(kf[t], s, z, g, bits), kivi[t])


@pytest.mark.parametrize("bits,ratio", [(2, 0.75), (4, 0.5)])
def test_error_in_the_query_subspace_shrinks(bits, ratio):
    """At lambda = 0.1 the subspace component of the error drops to about
    0.62 (b = 2) and 0.39 (b = 4) of plain rounding's on this block: at two
    bits the clamp to [0, 3] absorbs much of the correction. A wrong sign or
    index in the update would raise it instead."""
    rng = np.random.default_rng(10 + bits)
    d, r = 128, 8
    kf, s, z, kivi = _block(rng, bits=bits)
    a = rng.standard_normal((d, r)) * np.linspace(3, 1, r)
    qs = (a @ rng.standard_normal((r, 2000))).T + 0.05 * rng.standard_normal((2000, d))
    u = squat.subspace(qs, r)
    g = squat.coefficients(u, 0.1).astype(np.float32)
    deq = lambda codes: s.astype(np.float64) * codes + z.astype(np.float64)
    sq = np.stack([oracle.squat_token(kf[t], s, z, g, bits) for t in range(kf.shape[0])])
    assert ((sq >= 0) & (sq < (1 << bits))).all()
    e_kivi = kf - deq(kivi)
    e_squat = kf - deq(sq)
    sub_kivi = np.linalg.norm(e_kivi @ u)
    sub_squat = np.linalg.norm(e_squat @ u)
    assert sub_squat < ratio * sub_kivi, (sub_squat, sub_kivi)
    # inner products with fresh queries from the same distribution
    qn = (a @ rng.standard_normal((r, 200))).T
    assert np.abs(qn @ e_squat.T).mean() < (ratio + 0.05) * np.abs(qn @ e_kivi.T).mean()


def test_cache_uses_the_token_coder():
    """A cache with coefficients set codes every key of a quantized block as
    or_squat_token does with that block's statistics; values are untouched."""
    rng = np.random.default_rng(5)
    B, Hkv, d, T, bits = 1, 2, 64, 160, 2
    k = (rng.standard_normal((B, Hkv, T, d)) * 2).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    gs = np.stack([squat.unit_coefficients(rng.standard_normal((50, d)), 4, 0.1) for _ in range(B * Hkv)])
    plain = oracle.OracleCache(B, Hkv, Hkv, d, bits, max_tokens=T, residual=32)
    sq = oracle.OracleCache(B, Hkv, Hkv, d, bits, max_tokens=T, residual=32)
    sq.set_squat(gs)
    for c in (plain, sq):
        c.append(k, v)
        c.flush()
    for u in range(B * Hkv):
        pk, ps, pz, pv, pvs, pvz = plain.unit_quantized(u)
        qk, qs_, qz, qv, qvs, qvz = sq.unit_quantized(u)
        assert np.array_equal(ps, qs_) and np.array_equal(pz, qz)
        assert np.array_equal(pv, qv) and np.array_equal(pvs, qvs) and np.array_equal(pvz, qvz)
        kf = oracle.half_to_float(k[0, u])
        for t in range(qk.shape[0]):
            want = oracle.squat_token(kf[t], qs_[t // 32], qz[t // 32], gs[u], bits)
            assert np.array_equal(qk[t], want)
        assert not np.array_equal(pk, qk)  # the coefficients did change codes


def test_replay_along_its_own_codes():
    rng = np.random.default_rng(9)
    kf, s, z, _ = _block(rng, d=64)
    g = squat.unit_coefficients(rng.standard_normal((100, 64)), 6, 0.1)
    for t in range(8):
        codes = oracle.squat_token(kf[t], s, z, g, 2)
        own, q = oracle.squat_replay(kf[t], s, z, g, 2, codes)
        assert np.array_equal(own, codes)
        assert np.array_equal(np.clip(np.rint(q), 0, 3).astype(np.uint8), own)


def _walk64(k, s, z, g, bits):
    """The walk in fp64 (independent of the C oracle): codes by rounding half
    to even of (x - z) / s, clamped."""
    x = np.asarray(k, np.float64).copy()
    codes = np.zeros(x.size, np.int64)
    for c in range(x.size):
        codes[c] = min(max(np.rint((x[c] - z[c]) / s[c]), 0), (1 << bits) - 1)
        delta = x[c] - (float(s[c]) * codes[c] + float(z[c]))
        x[c + 1:] -= delta * g[c, c + 1:].astype(np.float64)
    return codes


@pytest.mark.parametrize("bits", [2, 4])
def test_c_walk_against_an_fp64_walk(bits):
    """The C oracle's fp32 walk and an fp64 walk written here agree except where
    fp32 rounding tips a code across a boundary (rare, and then by one)."""
    rng = np.random.default_rng(20 + bits)
    kf, s, z, _ = _block(rng, bits=bits)
    g = squat.unit_coefficients(rng.standard_normal((300, 128)) * np.linspace(4, 0.2, 128), 8, 0.1)
    diff = 0
    for t in range(kf.shape[0]):
        a = oracle.squat_token(kf[t], s, z, g, bits).astype(np.int64)
        b = _walk64(kf[t], s, z, g, bits)
        assert np.abs(a - b).max() <= 1
        diff += int((a != b).sum())
    assert diff <= 0.01 * kf.size


def test_code_check_accepts_the_oracle_and_catches_planted_codes():
    from kivi_testlib import squat_code_check
    rng = np.random.default_rng(31)
    kf, s, z, _ = _block(rng, d=64)
    g = squat.unit_coefficients(rng.standard_normal((200, 64)), 4, 0.1)
    codes = np.stack([oracle.squat_token(kf[t], s, z, g, 2) for t in range(kf.shape[0])])
    S, Z = np.tile(s, (kf.shape[0], 1)), np.tile(z, (kf.shape[0], 1))
    assert squat_code_check(kf, S, Z, g, 2, codes) == (0, 0.0)
    # one code moved to a neighbour far from its rounding boundary: rejected
    for _ in range(20):
        t, c = int(rng.integers(kf.shape[0])), int(rng.integers(64))
        own, q = oracle.squat_replay(kf[t], s, z, g, 2, codes[t])
        if abs(q[c] - np.rint(q[c])) < 0.3 and 0 < own[c] < 3:
            bad = codes.copy()
            bad[t, c] = own[c] + (1 if q[c] > own[c] else -1)
            with pytest.raises(AssertionError):
                squat_code_check(kf, S, Z, g, 2, bad)
            break
    else:
        pytest.fail("no element far from a boundary found")
