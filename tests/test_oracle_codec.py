"""Pins of the oracle's codec against what the KIVI page and arithmetic fix.

Source: KIVI explainer page ("ICML 2024論文解説: KIVI — チューニング不要のKVキャッシュ
2bit非対称量子化"), section 量子化アルゴリズム (Q, D, s, z), section アルゴリズム
(scale floor, round-then-clamp), section 実装のポイント (bit-packed codes).

None of these tests re-types the oracle's formula: they check hand-worked
values, a library conversion, invariants, and brute-force nearest-level search
in exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden


def _f32(hexbits):
    return np.array([int(hexbits, 16)], np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("row", read_golden("codec_cases.txt"), ids=lambda r: r[0])
def test_hand_worked_groups(oracle_mod, row):
    name, bits, xs, s_hex, z_hex, codes = row
    x = np.array([float(v) for v in xs.split()], np.float32)
    if name == "signed_zero":
        x = np.array([-0.0, 0.0, -0.0], np.float32)
    got_c, got_s, got_z = oracle_mod.quant_group(x, int(bits))
    assert list(got_c) == [int(c) for c in codes.split()]
    assert np.float32(got_s).view(np.uint32) == int(s_hex, 16), hex(np.float32(got_s).view(np.uint32))
    assert np.float32(got_z).view(np.uint32) == int(z_hex, 16), hex(np.float32(got_z).view(np.uint32))


def test_half_conversion_all_patterns(oracle_mod):
    """The oracle's binary16 decoder against numpy's, on all 65536 bit patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.half_to_float(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_conversion(oracle_mod):
    import torch
    vals = torch.tensor([0.0, -0.0, 1.0, -2.5, 3.140625, 1e-30, 6.5e4, -1.7e38], dtype=torch.bfloat16)
    for v in vals:
        b = int(v.view(torch.int16).item()) & 0xFFFF
        assert oracle_mod.bf16_to_float(b) == float(v.float())


@pytest.mark.parametrize("row", [r for r in read_golden("pack_rows.txt") if ";" not in r[2]], ids=lambda r: r[0])
def test_pack_hand_built_rows(oracle_mod, row):
    name, bits, codes, words = row
    codes = np.array([int(c) for c in codes.split()], np.uint8)
    want = np.array([int(w, 16) for w in words.split()], np.uint32)
    got = oracle_mod.pack_row(codes, int(bits))
    assert np.array_equal(got, want), [hex(w) for w in got]
    assert np.array_equal(oracle_mod.unpack_row(got, codes.size, int(bits)), codes)


@pytest.mark.parametrize("row", [r for r in read_golden("pack_rows.txt") if ";" in r[2]], ids=lambda r: r[0])
def test_pack_hand_built_multirow(oracle_mod, row):
    """or_pack_rows on hand-built rows: each row's words, row after row."""
    name, bits, codes, words = row
    codes = np.array([[int(c) for c in r.split()] for r in codes.split(";")], np.uint8)
    want = np.array([int(w, 16) for w in words.split()], np.uint32).reshape(codes.shape[0], -1)
    got = oracle_mod.pack_rows(codes, int(bits))
    assert np.array_equal(got, want), [[hex(w) for w in r] for r in got]


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_roundtrip_random(oracle_mod, bits):
    rng = np.random.default_rng(7)
    for d in (32, 64, 128):
        codes = rng.integers(0, 2 ** bits, d).astype(np.uint8)
        words = oracle_mod.pack_row(codes, bits)
        assert words.size == d * bits // 32
        assert np.array_equal(oracle_mod.unpack_row(words, d, bits), codes)


def _random_groups(rng, n_groups, n):
    """fp16-representable groups with varied spreads, outliers and repeats."""
    out = []
    for i in range(n_groups):
        scale = float(np.exp(rng.normal(0, 2)))
        x = rng.normal(0, scale, n)
        if i % 5 == 0:
            x[rng.integers(0, n)] *= 30.0
        if i % 7 == 0:
            x[: n // 2] = x[0]
        out.append(x.astype(np.float16).astype(np.float32))
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_invariants(oracle_mod, bits):
    """codes in range; min -> 0; max -> 2^b-1 when s is not floored; and the
    dequantization error |x - (s*code + z)| stays within s/2 (checked in fp64,
    with slack for the fp32 rounding of the quotient)."""
    qmax = 2 ** bits - 1
    rng = np.random.default_rng(11)
    for x in _random_groups(rng, 400, 32):
        codes, s, z = oracle_mod.quant_group(x, bits)
        assert codes.max() <= qmax
        assert codes[np.argmin(x)] == 0
        assert z == x.min()
        if x.max() > x.min():
            assert s > 0
            assert codes[np.argmax(x)] == qmax
        err = np.abs(x.astype(np.float64) - (np.float64(s) * codes + np.float64(z)))
        assert np.all(err <= np.float64(s) * (0.5 + 2.0 ** -18) + 1e-30)


@pytest.mark.parametrize("bits", [2, 4])
def test_brute_force_nearest_level(oracle_mod, bits):
    """Exact rational search: the chosen code is the nearest level z + k*s
    (k clamped to [0, 2^b-1]); elements whose exact quotient sits within 1e-5
    of a midpoint are left to the fp32 rounding and only range-checked.
    s and z themselves are checked exactly: z = min, s = fl(fl(max - min) / qmax)."""
    qmax = 2 ** bits - 1
    rng = np.random.default_rng(3 + bits)
    for x in _random_groups(rng, 150, 32):
        codes, s, z = oracle_mod.quant_group(x, bits)
        mn, mx = Fraction(float(x.min())), Fraction(float(x.max()))
        assert Fraction(float(z)) == mn
        rng_exact = mx - mn
        if rng_exact == 0:
            assert np.float32(s) == np.float32(1e-8)
            assert np.all(codes == 0)
            continue
        # fl32(max - min) then fl32(/ qmax): check s is the nearest fp32 to that quotient
        diff32 = np.float32(np.float32(x.max()) - np.float32(x.min()))
        exact_q = Fraction(float(diff32)) / qmax
        cand = np.float32(float(exact_q))
        nbrs = [np.nextafter(cand, np.float32(-np.inf)), cand, np.nextafter(cand, np.float32(np.inf))]
        best = min(nbrs, key=lambda c: abs(Fraction(float(c)) - exact_q))
        assert np.float32(s) == best
        S, Z = Fraction(float(s)), Fraction(float(z))
        for xi, ci in zip(x, codes):
            t = (Fraction(float(xi)) - Z) / S
            k = int(t + Fraction(1, 2)) if t >= 0 else 0
            k = max(0, min(qmax, k))
            frac = t - int(t) if t >= 0 else t
            near_mid = abs(frac - Fraction(1, 2)) < Fraction(1, 100000)
            if near_mid:
                assert ci in (int(t), int(t) + 1) or ci == qmax
            else:
                assert ci == k, (float(t), ci, k)


def test_key_axis_is_per_channel(oracle_mod):
    """Keys: statistics per channel over the G tokens of a block (section
    Per-Channel量子化). With every channel constant over the block's tokens,
    each channel's range is 0: s takes the floor, z is the channel's value, and
    all codes are 0. A per-token reading would give nonzero codes."""
    d, G = 32, 32
    oc = oracle_mod.OracleCache(1, 1, 1, d, 2, max_tokens=2 * G, residual=0)
    k = np.tile(np.arange(d, dtype=np.float16)[None, :], (G, 1))[None, None]
    v = np.tile(np.arange(G, dtype=np.float16)[:, None], (1, d))[None, None]
    oc.append(k, v)
    oc.flush()
    kc, ks, kz, vc, vs, vz = oc.unit_quantized(0)
    assert kc.shape == (G, d) and np.all(kc == 0)
    assert np.all(ks == np.float32(1e-8)) and np.array_equal(kz[0], np.arange(d, dtype=np.float32))
    # values: every token constant over its channel group -> per-token floor, z = token value
    assert np.all(vc == 0)
    assert np.all(vs == np.float32(1e-8)) and np.array_equal(vz[:, 0], np.arange(G, dtype=np.float32))


def test_key_ramp_over_tokens(oracle_mod):
    """K[t, c] = t mod 4 for every channel: per channel the block spans {0..3},
    so s = 1, z = 0 and the code of token t is t mod 4. V[t, c] = c mod 4:
    per token each 32-channel group spans {0..3}: s = 1, z = 0, code = c mod 4."""
    d, G = 64, 32
    oc = oracle_mod.OracleCache(1, 1, 1, d, 2, max_tokens=G, residual=0)
    t = np.arange(G)[:, None]
    c = np.arange(d)[None, :]
    k = np.broadcast_to(t % 4, (G, d)).astype(np.float16)[None, None]
    v = np.broadcast_to(c % 4, (G, d)).astype(np.float16)[None, None]
    oc.append(np.ascontiguousarray(k), np.ascontiguousarray(v))
    assert oc.flush() == G
    kc, ks, kz, vc, vs, vz = oc.unit_quantized(0)
    assert np.array_equal(kc, np.broadcast_to(t % 4, (G, d)))
    assert np.all(ks == 1) and np.all(kz == 0)
    assert np.array_equal(vc, np.broadcast_to(c % 4, (G, d)))
    assert vs.shape == (G, 2) and np.all(vs == 1) and np.all(vz == 0)
