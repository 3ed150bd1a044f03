"""Pins of the oracle's decode attention.

Source: KIVI explainer page ("ICML 2024論文解説: KIVI — チューニング不要のKVキャッシュ
2bit非対称量子化"), section 残差バッファ（Residual Buffer）: one softmax of
q . [D(K_quant); K_res]^T / sqrt(d_k) over all tokens, times [D(V_quant); V_res];
section 量子化アルゴリズム: D(x) = s * x + z.

Pins (none re-types the oracle's formula):
  * lossless case: when every group holds only values on its own grid
    {z + k s} with s a power of two and both ends present, the codec loses
    nothing, so the method reduces to textbook softmax attention over the fp16
    inputs, computed here with scipy's softmax;
  * q = 0: every score is equal, so the output is the plain mean of V;
  * a single token: the output is that token's value row;
  * GQA: query head i reads KV head i // (Hq / Hkv), checked through the
    lossless case with distinct KV heads.
"""

import numpy as np
import pytest
from scipy.special import softmax


def _lossless_kv(rng, B, H, T, d, G=32, vg=32, bits=2):
    """Values on per-group grids {z + k * s}, k in [0, 2^b - 1], both ends present.
    Keys: grid per (channel, G-token block). Values: grid per (token, vg channels)."""
    L = 2 ** bits - 1
    k = np.empty((B, H, T, d), np.float32)
    v = np.empty((B, H, T, d), np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(0, T, G):
                n = min(G, T - j)
                s = 2.0 ** rng.integers(-4, 2, size=d)
                z = np.round(rng.normal(0, 4, size=d) * 16) / 16
                codes = rng.integers(0, L + 1, size=(n, d))
                if n >= 2:
                    codes[0, :] = 0
                    codes[1, :] = L
                k[b, h, j:j + n] = z[None, :] + codes * s[None, :]
            for t in range(T):
                for g in range(d // vg):
                    s = 2.0 ** rng.integers(-4, 2)
                    z = np.round(rng.normal(0, 2) * 16) / 16
                    codes = rng.integers(0, L + 1, size=vg)
                    codes[0], codes[1] = 0, L
                    v[b, h, t, g * vg:(g + 1) * vg] = z + codes * s
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    assert np.array_equal(k16.astype(np.float32), k) and np.array_equal(v16.astype(np.float32), v)
    return k16, v16


def _textbook(q, k, v, Hq, Hkv):
    B, _, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for i in range(Hq):
            h = i // (Hq // Hkv)
            K = k[b, h].astype(np.float64)
            V = v[b, h].astype(np.float64)
            p = softmax(K @ q[b, i].astype(np.float64) / np.sqrt(d))
            out[b, i] = p @ V
    return out


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("T", [1, 100, 160, 161, 300, 517])
def test_lossless_equals_textbook(oracle_mod, bits, T):
    B, Hkv, Hq, d = 2, 2, 4, 64
    rng = np.random.default_rng(T * 10 + bits)
    k, v = _lossless_kv(rng, B, Hkv, T, d, bits=bits)
    q = rng.normal(size=(B, Hq, d)).astype(np.float16)
    oc = oracle_mod.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    nt, nq = oc.state()
    assert nt == T
    got = oc.attend(q)
    want = _textbook(q, k, v, Hq, Hkv)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_lossless_gqa_mapping_matters(oracle_mod):
    """A query head attached to the wrong KV head gives a visibly different answer."""
    B, Hkv, Hq, d, T = 1, 2, 4, 32, 200
    rng = np.random.default_rng(1)
    k, v = _lossless_kv(rng, B, Hkv, T, d)
    q = rng.normal(size=(B, Hq, d)).astype(np.float16)
    oc = oracle_mod.OracleCache(B, Hkv, Hq, d, 2, max_tokens=T)
    oc.append(k, v)
    got = oc.attend(q)
    wrong = np.zeros_like(got)
    for i in range(Hq):
        h = i % Hkv
        p = softmax(k[0, h].astype(np.float64) @ q[0, i].astype(np.float64) / np.sqrt(d))
        wrong[0, i] = p @ v[0, h].astype(np.float64)
    assert np.abs(got - wrong).max() > 1e-3
    np.testing.assert_allclose(got, _textbook(q, k, v, Hq, Hkv), rtol=1e-10, atol=1e-10)


def test_zero_query_gives_mean_value(oracle_mod):
    B, H, d, T = 1, 1, 64, 400
    rng = np.random.default_rng(4)
    k, v = _lossless_kv(rng, B, H, T, d)
    oc = oracle_mod.OracleCache(B, H, H, d, 2, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    got = oc.attend(np.zeros((B, H, d), np.float16))
    np.testing.assert_allclose(got[0, 0], v[0, 0].astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value(oracle_mod):
    rng = np.random.default_rng(6)
    k = rng.normal(size=(1, 1, 1, 128)).astype(np.float16)
    v = rng.normal(size=(1, 1, 1, 128)).astype(np.float16)
    oc = oracle_mod.OracleCache(1, 1, 1, 128, 2, max_tokens=4)
    oc.append(k, v)
    got = oc.attend(rng.normal(size=(1, 1, 128)).astype(np.float16))
    assert np.array_equal(got[0, 0], v[0, 0, 0].astype(np.float64))


def test_bf16_query(oracle_mod):
    import torch
    B, H, d, T = 1, 1, 32, 64
    rng = np.random.default_rng(8)
    k, v = _lossless_kv(rng, B, H, T, d)
    qf = torch.randn(B, H, d, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    oc = oracle_mod.OracleCache(B, H, H, d, 2, max_tokens=T)
    oc.append(k, v)
    got = oc.attend(qf, q_is_bf16=True)
    want = _textbook(qf.float().numpy(), k, v, H, H)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_empty_cache_raises(oracle_mod):
    oc = oracle_mod.OracleCache(1, 1, 1, 32, 2, max_tokens=4)
    with pytest.raises(ValueError):
        oc.attend(np.zeros((1, 1, 32), np.float16))
