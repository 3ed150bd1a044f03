"""Pins of the oracle's residual-ring bookkeeping.

Source: KIVI explainer page ("ICML 2024論文解説: KIVI — チューニング不要のKVキャッシュ
2bit非対称量子化"), section 残差バッファ（Residual Buffer） (the newest r tokens stay
fp16) and section Per-Token量子化（Value Cache） (a group of g tokens is quantized
once it has accumulated). Reading: a ring of C = R + G fp16 slots; a token that
arrives at a full ring first flushes the oldest G tokens; an explicit flush
quantizes floor((n_res - R) / G) * G tokens.

The oracle simulates this token by token; the tests check it against closed
forms derived separately on paper:
  after append(T) from empty:   n_q = ceil((T - C) / G) * G  for T > C, else 0
  after append(T) then flush:   n_q = floor((T - R) / G) * G for T >= R, else 0
"""

import numpy as np
import pytest


def _closed_append(T, R, G):
    C = R + G
    return 0 if T <= C else -(-(T - C) // G) * G


def _closed_prefill(T, R, G):
    return 0 if T < R else ((T - R) // G) * G


def _kv(rng, B, H, T, d):
    k = rng.normal(size=(B, H, T, d)).astype(np.float16)
    v = rng.normal(size=(B, H, T, d)).astype(np.float16)
    return k, v


@pytest.mark.parametrize("R", [128, 0, 32])
def test_bulk_append_and_flush_closed_forms(oracle_mod, R):
    G, d = 32, 32
    rng = np.random.default_rng(R)
    for T in [1, 31, 32, 127, 128, 129, 159, 160, 161, 191, 192, 193, 1000, 1024]:
        oc = oracle_mod.OracleCache(1, 1, 1, d, 2, max_tokens=1024, residual=R)
        k, v = _kv(rng, 1, 1, T, d)
        oc.append(k, v)
        nt, nq = oc.state()
        assert nt == T and nq == _closed_append(T, R, G), (T, nq)
        oc.flush()
        nt, nq = oc.state()
        assert nq == _closed_prefill(T, R, G), (T, nq)
        assert R <= nt - nq < R + G or (T < R and nq == 0)


def test_chunked_append_equals_bulk(oracle_mod):
    """Bytes of the quantized part depend only on the tokens: appending the
    same tokens in different chunkings, with flushes in between, gives the
    same codes wherever both have quantized."""
    G, R, d, T = 32, 128, 64, 700
    rng = np.random.default_rng(5)
    k, v = _kv(rng, 2, 2, T, d)
    a = oracle_mod.OracleCache(2, 2, 2, d, 2, max_tokens=T)
    a.append(k, v)
    a.flush()
    b = oracle_mod.OracleCache(2, 2, 2, d, 2, max_tokens=T)
    pos = 0
    for n in [1, 5, 64, 200, 3, 160, 267]:
        b.append(np.ascontiguousarray(k[:, :, pos:pos + n]), np.ascontiguousarray(v[:, :, pos:pos + n]))
        if n % 2:
            b.flush()
        pos += n
    assert pos == T
    b.flush()
    assert a.state() == b.state()
    for u in range(4):
        for x, y in zip(a.unit_quantized(u), b.unit_quantized(u)):
            assert np.array_equal(x, y)
        for x, y in zip(a.unit_residual(u), b.unit_residual(u)):
            assert np.array_equal(x, y)


def test_streaming_schedule(oracle_mod):
    """Prefill then one token per step with a flush every G steps (the GQA
    streaming workload, scaled down): n_res cycles R..R+G-1 before each flush."""
    G, R, d = 32, 128, 32
    T0 = 1024
    rng = np.random.default_rng(9)
    oc = oracle_mod.OracleCache(1, 1, 1, d, 2, max_tokens=T0 + 100)
    k, v = _kv(rng, 1, 1, T0, d)
    oc.append(k, v)
    oc.flush()
    assert oc.state() == (T0, _closed_prefill(T0, R, G))
    for i in range(1, 100):
        k, v = _kv(rng, 1, 1, 1, d)
        oc.append(k, v)
        if i % G == 0:
            assert oc.flush() == G
        nt, nq = oc.state()
        assert nt == T0 + i
        assert nq == _closed_prefill(T0, R, G) + G * (i // G)
        assert nt - nq == R + (i % G)


def test_capacity(oracle_mod):
    oc = oracle_mod.OracleCache(1, 1, 1, 32, 2, max_tokens=40)
    k, v = _kv(np.random.default_rng(0), 1, 1, 41, 32)
    with pytest.raises(ValueError):
        oc.append(k, v)
    assert oc.state() == (0, 0)


def test_residual_is_newest_tokens(oracle_mod):
    G, R, d, T = 32, 128, 32, 300
    rng = np.random.default_rng(2)
    k, v = _kv(rng, 1, 1, T, d)
    oc = oracle_mod.OracleCache(1, 1, 1, d, 2, max_tokens=T)
    oc.append(k, v)
    nt, nq = oc.state()
    kr, vr = oc.unit_residual(0)
    assert np.array_equal(kr, k[0, 0, nq:].view(np.uint16))
    assert np.array_equal(vr, v[0, 0, nq:].view(np.uint16))
