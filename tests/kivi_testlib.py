"""Helpers of the GPU parity tests: read a cache's device memory back through
the layout the C ABI reports (kivi_cache_layout), and compare it with the
oracle. Nothing here computes any of the method's arithmetic."""

from __future__ import annotations

import numpy as np

import oracle

# Attention tolerances (fp32 GPU path vs fp64 oracle): max |diff| over all
# outputs and ||diff||_2 / ||ref||_2 over the whole output tensor.
ATOL_MAX = 2e-3
REL_L2 = 1e-3


def gpu_unit_blocks(cache, unit: int, n_blocks: int):
    """(kcode [nb,G,W] u32 token-major, vcode [nb,d,b] u32 channel-major, ksz [nb,d,2] f32,
    vsz [nb,G,d/32,2] f32), read through the layout the C ABI reports."""
    L, c = cache.layout, cache.cfg
    G, d, W = c.k_block, c.head_dim, c.head_dim * c.bits // 32
    if c.n_pages > 0:
        # paged: block j of unit u = b * Hkv + h lives in page table[b][j], record h of the page
        b, h = divmod(unit, c.n_kv_heads)
        pages = cache.block_table[b, :n_blocks].cpu().numpy()
        mem = cache.memory
        raw = np.stack([mem[L.off_blocks + (int(p) * c.n_kv_heads + h) * L.block_bytes:][:L.block_bytes].cpu().numpy()
                        for p in pages]) if n_blocks else np.zeros((0, L.block_bytes), np.uint8)
    else:
        start = L.off_blocks + unit * L.unit_stride
        raw = cache.memory[start:start + n_blocks * L.block_bytes].cpu().numpy().reshape(n_blocks, L.block_bytes)
    kcode = raw[:, L.rec_kcode:L.rec_kcode + G * W * 4].copy().view(np.uint32).reshape(n_blocks, G, W)
    vcode = raw[:, L.rec_vcode:L.rec_vcode + G * W * 4].copy().view(np.uint32).reshape(n_blocks, d, c.bits)
    ksz = raw[:, L.rec_ksz:L.rec_ksz + d * 8].copy().view(np.float32).reshape(n_blocks, d, 2)
    ng = d // c.v_group
    vsz = raw[:, L.rec_vsz:L.rec_vsz + G * ng * 8].copy().view(np.float32).reshape(n_blocks, G, ng, 2)
    return kcode, vcode, ksz, vsz


def gpu_unit_residual(cache, unit: int, n_quant: int, n_tokens: int):
    """fp16 bit patterns (kres [n_res,d], vres [n_res,d]) of tokens [n_quant, n_tokens), in token order."""
    L, c = cache.layout, cache.cfg
    d = c.head_dim
    start = L.off_ring + unit * L.ring_unit_stride
    ring = cache.memory[start:start + L.ring_slots * 4 * d].cpu().numpy().copy().view(np.uint16)
    ring = ring.reshape(L.ring_slots, 2, d)
    slots = np.arange(n_quant, n_tokens) % L.ring_slots
    return ring[slots, 0], ring[slots, 1]


def compare_unit(cache, oc: "oracle.OracleCache", gpu_unit: int, or_unit: int, key_codes: bool = True):
    """Bit-exact comparison of one unit's quantized blocks and residual (the
    key codes left out with key_codes=False: the SQuat-style coder's are
    judged by squat_code_check instead)."""
    nt, nq = oc.state()
    c = cache.cfg
    st = cache.row_state(gpu_unit // c.n_kv_heads)
    assert (st[0], st[1]) == (nt, nq), (st, (nt, nq))
    G, bits = c.k_block, c.bits
    nb = nq // G
    kc, ks, kz, vc, vs, vz = oc.unit_quantized(or_unit)
    if nb:
        gk, gv, gksz, gvsz = gpu_unit_blocks(cache, gpu_unit, nb)
        # keys: one packed row per token; values: one packed row of the block's 32 tokens per channel
        want_k = oracle.pack_rows(kc, bits).reshape(nb, G, -1)
        vcb = np.ascontiguousarray(vc.reshape(nb, G, -1).transpose(0, 2, 1))  # [nb, d, G]
        want_v = oracle.pack_rows(vcb.reshape(-1, G), bits).reshape(nb, c.head_dim, -1)
        bad = np.argwhere(gk != want_k)
        assert not key_codes or bad.size == 0, f"key codes differ at {bad[:5].tolist()}"
        bad = np.argwhere(gv != want_v)
        assert bad.size == 0, f"value codes differ at {bad[:5].tolist()}"
        assert np.array_equal(gksz[..., 0].view(np.uint32), ks.view(np.uint32)), "key scales differ"
        assert np.array_equal(gksz[..., 1].view(np.uint32), kz.view(np.uint32)), "key zeros differ"
        ng = c.head_dim // c.v_group
        assert np.array_equal(gvsz[..., 0].reshape(nq, ng).view(np.uint32), vs.view(np.uint32)), "value scales differ"
        assert np.array_equal(gvsz[..., 1].reshape(nq, ng).view(np.uint32), vz.view(np.uint32)), "value zeros differ"
    kr, vr = oc.unit_residual(or_unit)
    gkr, gvr = gpu_unit_residual(cache, gpu_unit, nq, nt)
    assert np.array_equal(gkr, kr), "residual keys differ"
    assert np.array_equal(gvr, vr), "residual values differ"


def attention_error(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = got - want
    max_abs = float(np.abs(diff).max())
    rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300))
    return max_abs, rel_l2


def assert_attention_close(got, want):
    max_abs, rel_l2 = attention_error(got, want)
    assert max_abs <= ATOL_MAX and rel_l2 <= REL_L2, f"max_abs {max_abs:.3e} rel_l2 {rel_l2:.3e}"
    return max_abs, rel_l2


def squat_code_check(kf, s, z, g, bits, codes, tau=1e-3):
    """Judges SQuat-style key codes from another implementation against the
    oracle's walk. kf [T, d] fp32 keys, s, z [T, d] their blocks' per-channel
    statistics (row t: token t's block), g [d, d] fp32 update coefficients,
    codes [T, d]. The oracle walks each key along the given codes; a given code
    that differs from the oracle's own decision there must be the neighbour
    across a rounding boundary that the oracle's quotient lies within tau of
    (in code units): the two implementations' coefficients differ in their last
    bits, so either side of such a boundary is a correct rounding.
    Returns (number of codes that differ, largest boundary distance among them);
    raises AssertionError on a code that is not a valid rounding."""
    n_diff, worst = 0, 0.0
    for t in range(kf.shape[0]):
        own, q = oracle.squat_replay(kf[t], s[t], z[t], g, bits, codes[t])
        bad = np.nonzero(own != codes[t])[0]
        for c in bad:
            lo = min(int(own[c]), int(codes[t][c]))
            assert abs(int(own[c]) - int(codes[t][c])) == 1, (t, c, own[c], codes[t][c], q[c])
            dist = abs(q[c] - (lo + 0.5))
            assert dist <= tau, (t, c, own[c], codes[t][c], q[c])
            worst = max(worst, dist)
        n_diff += bad.size
    return n_diff, worst
