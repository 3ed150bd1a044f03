"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Packed codes, scales, zeros and residual rows must be bit-exact; decode
attention (fp32) must be within max-abs 2e-3 and rel-L2 1e-3 of the fp64
oracle. Inputs come from kivi_inputs (seeded; channel-outlier keys, sink-token
values). At the five workloads' full sizes the GPU runs the whole batch and the
oracle recomputes sampled (batch row, KV head) units from the same tensors.
"""

import numpy as np
import pytest
import torch

import kv_cache_compression_kivi_amd as kv
import oracle
from kivi_inputs import CONFIGS, KVWorkload, page_order, row_lengths
from kivi_testlib import assert_attention_close, compare_unit

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _announce(*parts):
    print("\n[case]", *parts, flush=True)


def _unit_oracle(k_cpu, v_cpu, b, h, group, d, bits, max_tokens, residual=128):
    oc = oracle.OracleCache(1, 1, group, d, bits, max_tokens=max_tokens, residual=residual)
    oc.append(k_cpu[b:b + 1, h:h + 1].contiguous(), v_cpu[b:b + 1, h:h + 1].contiguous())
    return oc


def _unit_rows(q_cpu, b, h, group):
    return q_cpu[b:b + 1, h * group:(h + 1) * group].contiguous()


SHAPES = [
    # B, Hkv, Hq, d, bits, T
    (1, 1, 1, 128, 2, 1024),
    (2, 3, 6, 128, 4, 700),
    (1, 2, 2, 64, 2, 333),
    (1, 1, 2, 256, 4, 200),
    (2, 2, 8, 128, 2, 161),
    (1, 1, 1, 128, 2, 1),
    (3, 2, 2, 128, 2, 100),
    (1, 2, 4, 256, 2, 517),
    (2, 1, 3, 64, 4, 1000),
    # four query heads per KV head at d = 128 (the matrix-core kernel with staged blocks):
    (1, 2, 8, 128, 4, 700),    # b = 4, ragged tail
    (1, 1, 4, 128, 2, 2000),   # many blocks per wave: the slot ring wraps
    (2, 1, 4, 128, 4, 330),    # fewer blocks than a wave's slots
    (1, 2, 16, 128, 2, 900),   # group of 8: two work-groups of four query heads per KV head
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_kv%d_q%d_d%d_b%d_T%d" % s)
@pytest.mark.parametrize("q_dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
def test_prefill_parity(shape, q_dtype):
    B, Hkv, Hq, d, bits, T = shape
    _announce("prefill", shape, q_dtype)
    wl = KVWorkload(B, Hkv, d, seed=sum(shape) + (q_dtype == torch.bfloat16))
    k, v = wl.kv(0, T)
    q = wl.q(Hq, dtype=q_dtype)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T + 7)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T + 7)
    oc.append(k, v)
    oc.flush()
    for u in range(B * Hkv):
        compare_unit(cache, oc, u, u)
    ref = oc.attend(q, q_is_bf16=q_dtype == torch.bfloat16)
    assert_attention_close(out.cpu().numpy(), ref)


@pytest.mark.parametrize("bits", [2, 4])
def test_chunked_appends_and_flushes(bits):
    """Arbitrary chunking, implicit and explicit flushes: same bytes as the oracle."""
    B, Hkv, Hq, d = 2, 2, 4, 128
    _announce("chunked", bits)
    T = 1500
    wl = KVWorkload(B, Hkv, d, seed=77 + bits)
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    rng = np.random.default_rng(bits)
    pos = 0
    step = 0
    while pos < T:
        n = int(min(T - pos, rng.choice([1, 1, 2, 7, 31, 32, 33, 64, 159, 160, 161, 300])))
        kk = k[:, :, pos:pos + n].contiguous()
        vv = v[:, :, pos:pos + n].contiguous()
        cache.append(kk.to(DEV), vv.to(DEV))
        oc.append(kk, vv)
        pos += n
        if rng.random() < 0.4:
            assert cache.flush() == oc.flush()
        step += 1
        if step % 5 == 0:
            q = wl.q(Hq, step=step)
            out = cache.attend(q.to(DEV))
            torch.cuda.synchronize()
            assert_attention_close(out.cpu().numpy(), oc.attend(q))
    torch.cuda.synchronize()
    for u in range(B * Hkv):
        compare_unit(cache, oc, u, u)


@pytest.mark.parametrize("Hq,bits", [(8, 2), (16, 2), (16, 4)], ids=["group2_b2", "group4_b2", "group4_b4"])
def test_split_invariance_and_determinism(Hq, bits):
    B, Hkv, d, T = 2, 4, 128, 4096
    _announce("splits", Hq, bits)
    wl = KVWorkload(B, Hkv, d, seed=5)
    k, v = wl.kv(0, T)
    q = wl.q(Hq).to(DEV)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    outs = {}
    for n in [0, 1, 2, 5, 31, 124, 200]:
        cache.set_attend_splits(n)
        n_split, bps = cache.plan_attend()
        a = cache.attend(q).cpu().numpy()
        b = cache.attend(q).cpu().numpy()
        assert np.array_equal(a, b), "attention is not bitwise deterministic"
        outs[(n, n_split, bps)] = a
    ref = list(outs.values())[0]
    # The four-query kernel takes its value weights' digits against a running
    # power-of-two bound, up to 2^2 above a block's own bound, so the split
    # count (which blocks a wave sees) moves a weight's rounding by up to
    # 2^-20 of its bound; the vector kernel's fp32 sums differ only in order.
    tol = 5e-5 if Hq // Hkv == 4 else 1e-5
    for key, a in outs.items():
        rel = np.abs(a - ref).max() / np.abs(ref).max()
        assert rel < tol, (key, rel)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    assert_attention_close(ref, oc.attend(q.cpu()))


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_ties_and_near_ties(bits):
    """Groups whose range is 2^b - 1 (so s = 1, z = 0) with values on half
    integers: (x - z) / s is exactly k + 0.5 and must round to even. Mixed in,
    values one fp16 step off a half integer (just on either side of a tie), and
    groups of range 1 (s = 1/(2^b - 1), not a power of two). Bit-exact against
    the oracle."""
    _announce("ties", bits)
    qmax = (1 << bits) - 1
    G, d, T = 32, 128, 32 * 6 + 128
    rng = np.random.default_rng(bits)
    halves = np.arange(qmax) + 0.5                      # every tie k + 0.5
    eps = np.float16(2.0 ** -10)                          # an fp16 step near 1..2
    pool = np.concatenate([halves, halves + eps, halves - eps, np.arange(qmax + 1)])
    x = rng.choice(pool, size=(T, d)).astype(np.float32)
    # every key channel block and every value group holds 0 and qmax: s = 1
    for j in range(T // G):
        x[j * G, :] = 0.0
        x[j * G + 1, :] = qmax
    x[:, 0::32] = 0.0
    x[:, 1::32] = qmax
    # a few channels / groups of range 1 instead
    x[:, 5] = rng.choice(np.linspace(0, 1, 17), size=T)
    k = torch.from_numpy(x.astype(np.float16)).reshape(1, 1, T, d)
    v = torch.from_numpy(np.ascontiguousarray(x[::-1]).astype(np.float16)).reshape(1, 1, T, d)
    cache = kv.KiviCache(1, 1, 1, d, bits, max_tokens=T, device=DEV)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    torch.cuda.synchronize()
    oc = oracle.OracleCache(1, 1, 1, d, bits, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    compare_unit(cache, oc, 0, 0)


@pytest.mark.parametrize("B,Hkv,Hq,d,bits,R,T0,steps,splits", [
    (2, 2, 2, 128, 2, 128, 200, 70, 0),   # MHA, flushes at the steps that complete a group past R
    (1, 2, 8, 128, 4, 32, 40, 40, 0),     # GQA (matrix-core kernel), small residual
    (2, 1, 1, 64, 2, 0, 5, 40, 0),        # no residual: a flush takes the new token itself
    (1, 1, 4, 256, 2, 64, 100, 35, 0),    # d = 256, GQA on the vector path
    # forced split counts: the new token is written by the last split, the
    # splits are merged by the combine kernel, and some splits hold no block
    (2, 2, 2, 128, 2, 128, 600, 40, 3),   # MHA, 3 splits
    (1, 2, 8, 128, 4, 32, 300, 40, 17),   # GQA matrix cores, 17 splits (more than the blocks of early steps)
    (2, 1, 2, 64, 2, 0, 500, 40, 5),      # no residual, two query heads per KV head, 5 splits
    (1, 1, 1, 256, 4, 64, 700, 35, 17),   # d = 256, 17 splits
])
def test_decode_step_parity(B, Hkv, Hq, d, bits, R, T0, steps, splits):
    """kivi_decode_step (quantize when due, then one attention launch that also
    writes the new token into the ring, then the merge when split) against the
    oracle run token by token: attention at every few steps, the whole cache
    bit-exact at the end."""
    _announce("decode_step", B, Hkv, Hq, d, bits, R, T0, steps, splits)
    wl = KVWorkload(B, Hkv, d, seed=11 + R, device="cpu")
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T0 + steps, residual=R, device=DEV)
    cache.set_attend_splits(splits)
    oc = oracle.OracleCache(B, Hkv, Hq, d, bits, max_tokens=T0 + steps, residual=R)
    k, v = wl.kv(0, T0)
    cache.append(k.to(DEV), v.to(DEV))
    oc.append(k, v)
    for i in range(steps):
        kt, vt = wl.kv(T0 + i, 1)
        q = wl.q(Hq, step=i)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), q.to(DEV))
        oc.append(kt, vt)
        nt, nq = oc.state()
        if nt - nq >= R + 32:
            assert oc.flush() == cache.last_flushed
        else:
            assert cache.last_flushed == 0
        assert cache.state()[:2] == oc.state()
        if i % 7 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            assert_attention_close(out.cpu().numpy(), oc.attend(q))
    torch.cuda.synchronize()
    for u in range(B * Hkv):
        compare_unit(cache, oc, u, u)


def test_errors_on_device():
    _announce("errors")
    cache = kv.KiviCache(1, 1, 1, 128, 2, max_tokens=64)
    q = torch.zeros(1, 1, 128, dtype=torch.float16, device=DEV)
    with pytest.raises(kv.KiviError) as e:
        cache.attend(q)
    assert e.value.status == "KIVI_E_EMPTY"
    k = torch.randn(1, 1, 64, 128, device=DEV).half()
    cache.append(k, k)
    with pytest.raises(kv.KiviError) as e:
        cache.append(k[:, :, :1].contiguous(), k[:, :, :1].contiguous())
    assert e.value.status == "KIVI_E_CAPACITY"
    assert cache.state() == (64, 0, 64)
    out = cache.attend(q)
    torch.cuda.synchronize()
    # q = 0: uniform weights, the output is the mean of the (residual) values
    np.testing.assert_allclose(out[0, 0].cpu().numpy(), k[0, 0].float().mean(0).cpu().numpy(), rtol=1e-5, atol=1e-5)
    cache.reset()
    assert cache.state() == (0, 0, 0)


# ------------------------------------------------------------------ full sizes

def _full_prefill(cfg, bits=None, layer=0):
    B, Hkv, Hq, d, T = cfg["batch"], cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    bits = bits if bits is not None else cfg["bits"]
    wl = KVWorkload(B, Hkv, d, seed=cfg["seed"], layer=layer, device=DEV)
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T + cfg.get("decode_steps", 0))
    cache.append(k, v)
    cache.flush()
    return wl, cache, k, v


@pytest.mark.parametrize("name,units", [("tiny", [0]), ("llama2_7b_layer", [0, 77, 255]),
                                        ("long_context", [0, 31])])
def test_workload_full_size(name, units):
    cfg = CONFIGS[name]
    _announce("full", name)
    wl, cache, k, v = _full_prefill(cfg)
    q_dtype = torch.float16
    q = wl.q(cfg["n_q_heads"], dtype=q_dtype)
    out = cache.attend(q)
    torch.cuda.synchronize()
    Hkv, Hq, d, T = cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    group = Hq // Hkv
    n_split, bps = cache.plan_attend()
    print(f"  splits {n_split} blocks/split {bps}", flush=True)
    for u in units:
        b, h = divmod(u, Hkv)
        kc = k[b:b + 1, h:h + 1].cpu()
        vc = v[b:b + 1, h:h + 1].cpu()
        oc = oracle.OracleCache(1, 1, group, d, cfg["bits"], max_tokens=T)
        oc.append(kc, vc)
        oc.flush()
        compare_unit(cache, oc, u, 0)
        ref = oc.attend(_unit_rows(q.cpu(), b, h, group))
        got = out[b:b + 1, h * group:(h + 1) * group].cpu().numpy()
        assert_attention_close(got, ref)


def test_gqa_streaming_full_size():
    """The GQA streaming workload at full size through kivi_decode_step, the
    call the benchmark times: prefill, then 256 steps of (append one token,
    flush when a group lies beyond the newest 128, attend) in one call each.
    Sampled units against their oracle caches at several steps, bytes at the
    end."""
    cfg = CONFIGS["gqa_streaming"]
    _announce("gqa_streaming")
    B, Hkv, Hq, d, T0, bits = (cfg[x] for x in ("batch", "n_kv_heads", "n_q_heads", "head_dim", "T", "bits"))
    steps = cfg["decode_steps"]
    group = Hq // Hkv
    wl, cache, k, v = _full_prefill(cfg)
    units = [0, 301, 511]
    ocs = {}
    for u in units:
        b, h = divmod(u, Hkv)
        oc = oracle.OracleCache(1, 1, group, d, bits, max_tokens=T0 + steps)
        oc.append(k[b:b + 1, h:h + 1].cpu(), v[b:b + 1, h:h + 1].cpu())
        oc.flush()
        ocs[u] = oc
    del k, v
    check_at = {1, 31, 32, 33, steps}
    for i in range(1, steps + 1):
        kt, vt = wl.kv(T0 + i - 1, 1)
        q = wl.q(Hq, step=i)
        out = cache.decode_step(kt, vt, q)
        flushed = 0
        for u in units:
            b, h = divmod(u, Hkv)
            ocs[u].append(kt[b:b + 1, h:h + 1].cpu(), vt[b:b + 1, h:h + 1].cpu())
            nt, nq = ocs[u].state()
            if nt - nq >= 128 + 32:
                flushed = ocs[u].flush()
        assert cache.last_flushed == flushed
        if i in check_at:
            torch.cuda.synchronize()
            print(f"  step {i} state {cache.state()}", flush=True)
            for u in units:
                b, h = divmod(u, Hkv)
                ref = ocs[u].attend(_unit_rows(q.cpu(), b, h, group))
                got = out[b:b + 1, h * group:(h + 1) * group].cpu().numpy()
                assert_attention_close(got, ref)
    torch.cuda.synchronize()
    for u in units:
        compare_unit(cache, ocs[u], u, 0)


@pytest.mark.parametrize("paged", [False, True], ids=["regions", "paged"])
def test_serving_batch_full_size(paged):
    """The serving-batch workloads at full size, built as the benchmark builds
    them (64 rows at their seeded lengths; paged: every row's pages in the
    seeded random order), then 40 steps through kivi_decode_step, whose flushes
    fall on different steps per row. The longest, the shortest and a middling
    row, KV heads 0 and 7, against their oracle caches at several steps; their
    bytes at the end."""
    cfg = CONFIGS["gqa_paged" if paged else "gqa_ragged"]
    _announce("serving batch", "paged" if paged else "regions")
    B, Hkv, Hq, d, T, bits = (cfg[x] for x in ("batch", "n_kv_heads", "n_q_heads", "head_dim", "T", "bits"))
    group = Hq // Hkv
    steps = 40
    lens = row_lengths(B, cfg["ragged"][0], cfg["ragged"][1], cfg["seed"])
    max_tokens = T + steps + 64
    wl = KVWorkload(B, Hkv, d, seed=cfg["seed"], device=DEV)
    k, v = wl.kv(0, T)
    if paged:
        mb = max_tokens // 32
        cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, device=DEV, n_pages=B * mb)
        cache.set_block_table(page_order(B * mb, cfg["seed"]).reshape(B, mb).to(DEV))
    else:
        cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, device=DEV)
    cache.append_rows(k, v, lens)
    cache.flush()
    order = sorted(range(B), key=lambda r: lens[r])
    rows = [order[-1], order[0], order[B // 2]]
    units = [(r, h) for r in rows for h in (0, Hkv - 1)]
    ocs = {}
    for r, h in units:
        oc = oracle.OracleCache(1, 1, group, d, bits, max_tokens=max_tokens)
        oc.append(k[r:r + 1, h:h + 1, :lens[r]].cpu(), v[r:r + 1, h:h + 1, :lens[r]].cpu())
        nt, nq = oc.state()
        if nt - nq >= 128 + 32:
            oc.flush()
        ocs[(r, h)] = oc
    del k, v
    for i in range(1, steps + 1):
        kt, vt = wl.kv(T + i - 1, 1)
        q = wl.q(Hq, step=i)
        out = cache.decode_step(kt, vt, q)
        for r, h in units:
            ocs[(r, h)].append(kt[r:r + 1, h:h + 1].cpu(), vt[r:r + 1, h:h + 1].cpu())
            nt, nq = ocs[(r, h)].state()
            if nt - nq >= 128 + 32:
                ocs[(r, h)].flush()
        if i in (1, 17, 33, steps):
            torch.cuda.synchronize()
            for r, h in units:
                assert cache.row_state(r)[:2] == ocs[(r, h)].state(), (r, cache.row_state(r), ocs[(r, h)].state())
                ref = ocs[(r, h)].attend(_unit_rows(q.cpu(), r, h, group))
                got = out[r:r + 1, h * group:(h + 1) * group].cpu().numpy()
                assert_attention_close(got, ref)
    torch.cuda.synchronize()
    for r, h in units:
        compare_unit(cache, ocs[(r, h)], r * Hkv + h, 0)


@pytest.mark.parametrize("layer", [0, 31])
def test_full_stack_layer(layer):
    cfg = CONFIGS["full_stack"]
    bits = cfg["layer_bits"][layer]
    _announce("full_stack layer", layer, "bits", bits)
    B, Hkv, Hq, d, T = cfg["batch"], cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    group = Hq // Hkv
    steps = 33  # the 32nd decode step flushes a group
    wl, cache, k, v = _full_prefill(dict(cfg, decode_steps=steps), bits=bits, layer=layer)
    q = wl.q(Hq, dtype=torch.bfloat16)
    out = cache.attend(q)
    torch.cuda.synchronize()
    ocs = {}
    for u in [5, 1023]:
        b, h = divmod(u, Hkv)
        oc = oracle.OracleCache(1, 1, group, d, bits, max_tokens=T + steps)
        oc.append(k[b:b + 1, h:h + 1].cpu(), v[b:b + 1, h:h + 1].cpu())
        oc.flush()
        compare_unit(cache, oc, u, 0)
        ref = oc.attend(_unit_rows(q.cpu(), b, h, group), q_is_bf16=True)
        got = out[b:b + 1, h * group:(h + 1) * group].cpu().numpy()
        assert_attention_close(got, ref)
        ocs[u] = oc
    del k, v
    # then the benchmark's decode steps (kivi_decode_step), across a flush
    for i in range(1, steps + 1):
        kt, vt = wl.kv(T + i - 1, 1)
        qi = wl.q(Hq, step=i, dtype=torch.bfloat16)
        out = cache.decode_step(kt, vt, qi)
        for u, oc in ocs.items():
            b, h = divmod(u, Hkv)
            oc.append(kt[b:b + 1, h:h + 1].cpu(), vt[b:b + 1, h:h + 1].cpu())
            nt, nq = oc.state()
            if nt - nq >= 128 + 32:
                assert oc.flush() == cache.last_flushed == 32
        if i in (1, 32, steps):
            torch.cuda.synchronize()
            for u, oc in ocs.items():
                b, h = divmod(u, Hkv)
                ref = oc.attend(_unit_rows(qi.cpu(), b, h, group), q_is_bf16=True)
                got = out[b:b + 1, h * group:(h + 1) * group].cpu().numpy()
                assert_attention_close(got, ref)
    torch.cuda.synchronize()
    for u, oc in ocs.items():
        compare_unit(cache, oc, u, 0)


# ------------------------------------------------------- sequences of different lengths

def _row_oracles(k, v, lens, Hq, bits, max_tokens, R):
    """One batch-of-one oracle cache per row, holding that row's own tokens."""
    B, Hkv, _, d = k.shape
    ocs = []
    for b in range(B):
        oc = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R)
        if lens[b]:
            oc.append(k[b:b + 1, :, :lens[b]].contiguous(), v[b:b + 1, :, :lens[b]].contiguous())
        ocs.append(oc)
    return ocs


def _check_rows(cache, ocs, out, q, q_bf16=False):
    Hkv = cache.cfg.n_kv_heads
    for b, oc in enumerate(ocs):
        assert cache.row_state(b)[:2] == oc.state(), (b, cache.row_state(b), oc.state())
        assert_attention_close(out[b:b + 1].cpu().numpy(), oc.attend(q[b:b + 1], q_is_bf16=q_bf16))


def _check_bytes(cache, ocs):
    Hkv = cache.cfg.n_kv_heads
    for b, oc in enumerate(ocs):
        for h in range(Hkv):
            compare_unit(cache, oc, b * Hkv + h, h)


@pytest.mark.parametrize("B,Hkv,Hq,d,bits,R,lens", [
    (5, 2, 2, 128, 2, 128, [1, 33, 160, 161, 700]),   # MHA vector kernel, pairs of blocks
    (4, 2, 8, 128, 4, 128, [700, 5, 192, 2000]),      # four query heads per KV head (matrix cores), b = 4
    (3, 1, 4, 128, 2, 32, [64, 1000, 31]),            # four-query kernel at b = 2, small residual
    (3, 2, 4, 64, 2, 64, [300, 1, 97]),               # d = 64, two query heads per KV head
    (2, 1, 2, 256, 4, 128, [129, 517]),               # d = 256
    (3, 2, 16, 128, 2, 32, [400, 2, 1100]),           # eight query heads per KV head: two chunks on one XCD
    (2, 1, 4, 256, 2, 64, [300, 45]),                 # four query heads on the vector kernel (d = 256)
])
def test_ragged_rows_parity(B, Hkv, Hq, d, bits, R, lens):
    """Sequences of different lengths in one batch (the per-row entry points):
    a ragged prefill (kivi_append_rows), attention at several forced split
    counts (short rows see empty splits), decode steps whose flushes fall on
    different steps per row, a row emptied and refilled with a new sequence,
    and a uniform append and flush on the ragged batch. Each row against an
    oracle cache of that row alone: attention within the bar, bytes exact."""
    _announce("ragged", B, Hkv, Hq, d, bits, R, lens)
    steps = 40
    T = max(lens)
    max_tokens = T + steps + 80
    wl = KVWorkload(B, Hkv, d, seed=sum(lens) + d + bits, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV)
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    ocs = _row_oracles(k, v, lens, Hq, bits, max_tokens, R)
    q = wl.q(Hq, step=0)
    for n in (0, 1, 3, 17):
        cache.set_attend_splits(n)
        out = cache.attend(q.to(DEV))
        torch.cuda.synchronize()
        _check_rows(cache, ocs, out, q)
    cache.set_attend_splits(0)
    _check_bytes(cache, ocs)
    assert cache.flush() == max(oc.flush() for oc in ocs)
    for i in range(steps):
        if i == 15:
            # row 1 ends; a new sequence of 70 tokens takes its place
            cache.reset_row(1)
            kn, vn = wl.kv(5000, 70)
            ntok = [0] * B
            ntok[1] = 70
            cache.append_rows(kn.to(DEV), vn.to(DEV), ntok)
            ocs[1] = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R)
            ocs[1].append(kn[1:2].contiguous(), vn[1:2].contiguous())
        kt, vt = wl.kv(T + i, 1)
        qi = wl.q(Hq, step=i + 1, dtype=torch.bfloat16 if i % 2 else torch.float16)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), qi.to(DEV))
        flushed = 0
        for b, oc in enumerate(ocs):
            oc.append(kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
            nt, nq = oc.state()
            if nt - nq >= R + 32:
                flushed = max(flushed, oc.flush())
        assert cache.last_flushed == flushed
        if i % 6 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            _check_rows(cache, ocs, out, qi, q_bf16=qi.dtype == torch.bfloat16)
    # the same number of tokens appended to every row of the ragged batch, then a flush
    ka, va = wl.kv(9000, 45)
    cache.append(ka.to(DEV), va.to(DEV))
    for b, oc in enumerate(ocs):
        oc.append(ka[b:b + 1].contiguous(), va[b:b + 1].contiguous())
    assert cache.flush() == max(oc.flush() for oc in ocs)
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    _check_rows(cache, ocs, out, q)
    _check_bytes(cache, ocs)
    with pytest.raises(kv.KiviError) as e:
        cache.state()
    assert e.value.status == "KIVI_E_RAGGED"
    # an emptied row makes attention fail before any launch
    cache.reset_row(0)
    with pytest.raises(kv.KiviError) as e:
        cache.attend(q.to(DEV))
    assert e.value.status == "KIVI_E_EMPTY"


@pytest.mark.parametrize("B,Hkv,Hq,d,bits,R,lens", [
    (4, 2, 2, 128, 2, 128, [700, 33, 161, 1]),        # MHA vector kernel
    (3, 2, 8, 128, 4, 128, [450, 2000, 5]),           # four query heads per KV head (matrix cores)
    (3, 2, 4, 64, 2, 32, [97, 640, 300]),             # d = 64, two query heads per KV head
    (2, 1, 4, 256, 4, 64, [45, 300]),                 # d = 256, four query heads on the vector kernel
])
def test_paged_blocks_parity(B, Hkv, Hq, d, bits, R, lens):
    """Paged blocks: every (row, block) maps through a caller-owned block table
    to a page of a shared pool, in scrambled order with spare pages. A ragged
    prefill, attention at several split counts, decode steps whose flushes
    write new pages, and a row emptied and refilled on other pages (some freed
    by itself, some spare). Each row against an oracle cache of that row alone;
    the bytes are read back page by page through the table."""
    _announce("paged", B, Hkv, Hq, d, bits, R, lens)
    steps = 40
    T = max(lens)
    max_tokens = T + steps + 80
    max_blocks = max_tokens // 32
    stride = max_blocks + 3
    n_pages = B * max_blocks + 9
    rng = np.random.default_rng(sum(lens) + bits)
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((B, stride), -1, np.int32)   # -1 in unused entries: the kernels never need them
    table[:, :max_blocks] = perm[:B * max_blocks].reshape(B, max_blocks)
    spare = list(perm[B * max_blocks:])
    wl = KVWorkload(B, Hkv, d, seed=sum(lens) + 3 * d, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV, n_pages=n_pages)
    assert cache.layout.unit_stride == 0 and cache.layout.page_bytes == Hkv * cache.layout.block_bytes
    tab = torch.from_numpy(table).to(DEV)
    cache.set_block_table(tab)
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    ocs = _row_oracles(k, v, lens, Hq, bits, max_tokens, R)
    q = wl.q(Hq, step=0)
    for n in (0, 1, 3, 17):
        cache.set_attend_splits(n)
        out = cache.attend(q.to(DEV))
        torch.cuda.synchronize()
        _check_rows(cache, ocs, out, q)
    cache.set_attend_splits(0)
    _check_bytes(cache, ocs)
    for i in range(steps):
        if i == 15:
            # row 1 ends; its new sequence takes half of its old pages (reversed) and the spare ones
            cache.reset_row(1)
            old = list(table[1, :max_blocks])
            new = (old[::-2] + spare + old[-2::-2])[:max_blocks]
            spare = [p for p in old + spare if p not in set(new)]
            table[1, :max_blocks] = np.array(new, np.int32)
            tab.copy_(torch.from_numpy(table).to(DEV))
            kn, vn = wl.kv(5000, 99)
            ntok = [0] * B
            ntok[1] = 99
            cache.append_rows(kn.to(DEV), vn.to(DEV), ntok)
            ocs[1] = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R)
            ocs[1].append(kn[1:2].contiguous(), vn[1:2].contiguous())
        kt, vt = wl.kv(T + i, 1)
        qi = wl.q(Hq, step=i + 1)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), qi.to(DEV))
        for b, oc in enumerate(ocs):
            oc.append(kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
            nt, nq = oc.state()
            if nt - nq >= R + 32:
                oc.flush()
        if i % 6 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            _check_rows(cache, ocs, out, qi)
    torch.cuda.synchronize()
    _check_bytes(cache, ocs)
    # a paged cache refuses work without a table; a contiguous one refuses a table
    plain = kv.KiviCache(1, 1, 1, d, bits, max_tokens=64, device=DEV)
    with pytest.raises(kv.KiviError) as e:
        plain.set_block_table(tab[:1].contiguous())
    assert e.value.status == "KIVI_E_INVAL"
    fresh = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV, n_pages=n_pages)
    with pytest.raises(kv.KiviError) as e:
        fresh.append_rows(k.to(DEV), v.to(DEV), lens)
    assert e.value.status == "KIVI_E_INVAL"


@pytest.mark.parametrize("B,bits,t_max,paged", [(40, 2, 700, False), (128, 4, 300, False), (40, 2, 500, True),
                                                 (300, 2, 200, False), (200, 4, 160, True)],
                         ids=["40rows_b2", "128rows_b4", "40rows_b2_paged", "300rows_b2", "200rows_b4_paged"])
def test_large_ragged_batch_parity(B, bits, t_max, paged):
    """Serving batches with many rows of different lengths on the four-query
    kernel: 40 rows, 128 (one full row table), and 300 and 200 (paged), which
    run as several launches of at most 128 rows; 8 KV heads, 320 to 2400
    units, more work-groups than one round over the CUs. Attention at splits
    0, 1 and 3 with bf16 queries, then decode steps whose appended tokens the
    work-groups write to the ring. Every row against an oracle cache of that
    row alone, bytes exact at the end."""
    Hkv, Hq, d, R = 8, 32, 128, 128
    rng = np.random.default_rng(B + bits)
    lens = [int(x) for x in rng.integers(1, t_max + 1, B)]
    _announce("large ragged batch", B, bits, t_max, "paged" if paged else "regions")
    steps = 10
    T = max(lens)
    max_tokens = T + steps + 40
    wl = KVWorkload(B, Hkv, d, seed=B * 7 + bits, device="cpu")
    k, v = wl.kv(0, T)
    if paged:
        max_blocks = max_tokens // 32
        n_pages = B * max_blocks
        perm = rng.permutation(n_pages).astype(np.int32)
        cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV, n_pages=n_pages)
        cache.set_block_table(torch.from_numpy(perm.reshape(B, max_blocks)).to(DEV))
    else:
        cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV)
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    ocs = _row_oracles(k, v, lens, Hq, bits, max_tokens, R)
    q = wl.q(Hq, step=0, dtype=torch.bfloat16)
    for n in (0, 1, 3):
        cache.set_attend_splits(n)
        out = cache.attend(q.to(DEV))
        torch.cuda.synchronize()
        _check_rows(cache, ocs, out, q, q_bf16=True)
    cache.set_attend_splits(0)
    for i in range(steps):
        kt, vt = wl.kv(T + i, 1)
        qi = wl.q(Hq, step=i + 1)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), qi.to(DEV))
        for b, oc in enumerate(ocs):
            oc.append(kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
            nt, nq = oc.state()
            if nt - nq >= R + 32:
                oc.flush()
        if i % 3 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            _check_rows(cache, ocs, out, qi)
    torch.cuda.synchronize()
    _check_bytes(cache, ocs)


def test_mha_batch_beyond_one_row_table():
    """The MHA vector kernel and the quantizer on 140 rows of different
    lengths (launches of 128 and 12 rows), d = 64, b = 4, R = 32 so that the
    decode steps' flushes fall on different steps per row and in both
    launches: a ragged prefill (some rows empty), then 8 decode steps at
    splits 0 and 3 alternately. Every row against an oracle cache of that row
    alone after every step, bytes exact at the end."""
    B, Hkv, Hq, d, bits, R, steps = 140, 2, 2, 64, 4, 32, 8
    rng = np.random.default_rng(140)
    lens = [int(x) for x in rng.integers(0, 200, B)]
    lens[0], lens[127], lens[128] = 199, 0, 64  # the launches' first and last rows
    _announce("mha beyond one row table", B, Hkv, Hq, d, bits, R)
    T = max(lens)
    max_tokens = T + steps + 8
    wl = KVWorkload(B, Hkv, d, seed=140, device="cpu")
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R, device=DEV)
    cache.append_rows(k.to(DEV), v.to(DEV), lens)
    ocs = _row_oracles(k, v, lens, Hq, bits, max_tokens, R)
    # attention needs a token in every row: the first decode step brings one to the empty rows
    for i in range(steps):
        kt, vt = wl.kv(T + i, 1)
        qi = wl.q(Hq, step=i)
        cache.set_attend_splits(3 if i % 2 else 0)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), qi.to(DEV))
        for b, oc in enumerate(ocs):
            oc.append(kt[b:b + 1].contiguous(), vt[b:b + 1].contiguous())
            nt, nq = oc.state()
            if nt - nq >= R + 32:
                oc.flush()
        torch.cuda.synchronize()
        _check_rows(cache, ocs, out, qi)
    _check_bytes(cache, ocs)


@pytest.mark.parametrize("paged", [False, True], ids=["regions", "paged"])
@pytest.mark.parametrize("Hq,d,bits,R", [(2, 64, 4, 0), (8, 128, 2, 32), (4, 128, 4, 128)])
def test_row_operations_random_walk(paged, Hq, d, bits, R):
    """A seeded random sequence of per-row operations on a batch of 5 sequences:
    ragged appends of 0-70 tokens a row, uniform appends, flushes, decode
    steps, rows emptied (and, paged, moved onto other pages), attention at a
    random forced split count. After every attention each row matches an
    oracle cache of that row alone; at the end every unit's bytes match."""
    _announce("random walk", paged, Hq, d, bits, R)
    B, Hkv = 5, 2
    max_tokens = 700
    mb = max_tokens // 32
    rng = np.random.default_rng(1000 * bits + d + R + paged)
    wl = KVWorkload(B, Hkv, d, seed=int(rng.integers(1 << 30)), device="cpu")
    kw = dict(max_tokens=max_tokens, residual=R, device=DEV)
    if paged:
        n_pages = B * mb + 11
        kw["n_pages"] = n_pages
        free = list(rng.permutation(n_pages).astype(np.int32))
        table = np.zeros((B, mb), np.int32)
        for b in range(B):
            table[b] = [free.pop() for _ in range(mb)]
        tab = torch.from_numpy(table).to(DEV)
    cache = kv.KiviCache(B, Hkv, Hq, d, bits, **kw)
    if paged:
        cache.set_block_table(tab)
    ocs = [oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R) for _ in range(B)]
    pos = 0
    for step in range(60):
        op = rng.choice(["rows", "rows", "uniform", "flush", "decode", "decode", "reset", "attend"])
        lens = [oc.state()[0] for oc in ocs]
        if op == "rows":
            ntok = [int(x) if lens[b] + x <= max_tokens - 40 else 0 for b, x in enumerate(rng.integers(0, 71, B))]
            k, v = wl.kv(pos, max(ntok) or 1)
            pos += 71
            cache.append_rows(k.to(DEV), v.to(DEV), ntok)
            for b in range(B):
                if ntok[b]:
                    ocs[b].append(k[b:b + 1, :, :ntok[b]].contiguous(), v[b:b + 1, :, :ntok[b]].contiguous())
        elif op == "uniform" and max(lens) + 9 <= max_tokens - 40:
            k, v = wl.kv(pos, 9)
            pos += 9
            cache.append(k.to(DEV), v.to(DEV))
            for b in range(B):
                ocs[b].append(k[b:b + 1].contiguous(), v[b:b + 1].contiguous())
        elif op == "flush":
            assert cache.flush() == max(oc.flush() for oc in ocs)
        elif op == "decode" and max(lens) + 1 <= max_tokens - 40:
            k, v = wl.kv(pos, 1)
            pos += 1
            q = wl.q(Hq, step=step)
            out = cache.decode_step(k.to(DEV), v.to(DEV), q.to(DEV))
            for b in range(B):
                ocs[b].append(k[b:b + 1].contiguous(), v[b:b + 1].contiguous())
                nt, nq = ocs[b].state()
                if nt - nq >= R + 32:
                    ocs[b].flush()
            torch.cuda.synchronize()
            _check_rows(cache, ocs, out, q)
        elif op == "reset":
            b = int(rng.integers(B))
            cache.reset_row(b)
            ocs[b] = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=max_tokens, residual=R)
            if paged:  # the row's pages go back to the pool; it takes others
                free = list(table[b]) + free
                rng.shuffle(free)
                table[b] = [free.pop() for _ in range(mb)]
                tab.copy_(torch.from_numpy(table).to(DEV))
        elif op == "attend" and min(lens) > 0:
            cache.set_attend_splits(int(rng.choice([0, 1, 2, 5, 13])))
            q = wl.q(Hq, step=step, dtype=torch.bfloat16)
            out = cache.attend(q.to(DEV))
            torch.cuda.synchronize()
            _check_rows(cache, ocs, out, q, q_bf16=True)
            cache.set_attend_splits(0)
        for b in range(B):
            assert cache.row_state(b)[:2] == ocs[b].state(), (step, op, b)
    torch.cuda.synchronize()
    _check_bytes(cache, ocs)


@pytest.mark.parametrize("Hq,bits", [(1, 2), (2, 4), (4, 2)], ids=["mha", "group2", "group4"])
def test_unwritten_ring_slots_never_reach_the_output(Hq, bits):
    """Cache memory filled with NaN bit patterns before use: decode steps from an
    empty cache read partial residual chunks whose unused token lanes point at
    ring slots this call has not written yet. Their weight is zero, and so must
    be their contribution: outputs stay finite and match the oracle."""
    _announce("unwritten slots", Hq, bits)
    B, Hkv, d, steps = 2, 2, 128, 40
    wl = KVWorkload(B, Hkv, d, seed=77 + Hq, device="cpu")
    cfg = kv._native.make_config(B, Hkv, Hkv * Hq, d, bits, steps)
    mem = torch.full((kv.kivi_cache_bytes(cfg),), 0xFF, dtype=torch.uint8, device=DEV)  # fp16 0xFFFF is a NaN
    cache = kv.KiviCache(B, Hkv, Hkv * Hq, d, bits, max_tokens=steps, device=DEV, memory=mem)
    oc = oracle.OracleCache(B, Hkv, Hkv * Hq, d, bits, max_tokens=steps)
    for i in range(steps):
        kt, vt = wl.kv(i, 1)
        q = wl.q(Hkv * Hq, step=i)
        out = cache.decode_step(kt.to(DEV), vt.to(DEV), q.to(DEV))
        oc.append(kt, vt)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all(), i
        assert_attention_close(got, oc.attend(q))


@pytest.mark.parametrize("bits", [2, 4])
def test_degenerate_and_extreme_groups(bits):
    """Key channels and value groups that are constant (s floored at 1e-8), all
    zero with mixed signs of zero, at the fp16 extremes (+-65504, one range
    spanning both), made of fp16 subnormals, holding a single outlier, or offset
    from zero by more than, about or less than 32 of their scales (the fast
    code path's limit).
    Codes, scales, zeros and residual rows bit-exact against the oracle; the
    attention (a zero query, so every weight is equal and the outputs stay near
    the values' means) within the bar where the values are moderate."""
    _announce("degenerate", bits)
    d, T = 128, 32 * 5 + 128 + 7
    rng = np.random.default_rng(99 + bits)
    x = rng.standard_normal((T, d)).astype(np.float32)
    x[:, 0] = 3.0                                          # constant channel
    x[:, 1] = 0.0
    x[::2, 1] = -0.0                                       # signed zeros
    x[:, 2] = rng.choice([65504.0, -65504.0], size=T)      # the whole fp16 range
    x[:, 3] = 65504.0
    x[:, 4] = rng.integers(1, 1024, T) * 2.0 ** -24        # fp16 subnormals
    x[:, 5] = 0.0
    x[::37, 5] = 1000.0                                    # a lone outlier per block
    x[:, 6] = 1000.0 + rng.standard_normal(T) * 0.5        # offset far beyond the range: the division path
    x[:, 7] = 40.0 + rng.integers(0, 4, T)                 # z / s = 40 at b = 2, beyond the fast path's 32
    x[:, 8] = 30.0 + rng.integers(0, 4, T)                 # z / s = 30 at b = 2, inside it
    x[:, 9] = -32.0 + rng.integers(0, 4, T)                # z / s = -32, on its edge
    x[7, :] = 2.5                                          # a constant token (value groups)
    x[11, 32:64] = -65504.0
    x[13, 64:96] = 500.0 + rng.standard_normal(32)         # a value group far from zero
    k = torch.from_numpy(x.astype(np.float16)).reshape(1, 1, T, d)
    v = torch.from_numpy(np.ascontiguousarray(x[::-1]).astype(np.float16)).reshape(1, 1, T, d)
    cache = kv.KiviCache(1, 1, 1, d, bits, max_tokens=T, device=DEV)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    torch.cuda.synchronize()
    oc = oracle.OracleCache(1, 1, 1, d, bits, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    compare_unit(cache, oc, 0, 0)
    # attention over moderate values: zero the extreme value channels for this part
    vm = v.clone()
    vm[..., 2:4] = 0
    vm[..., 6] = 0
    vm[0, 0, T - 1 - 11, 32:64] = 0
    vm[0, 0, T - 1 - 13, 64:96] = 0
    cm = kv.KiviCache(1, 1, 1, d, bits, max_tokens=T, device=DEV)
    cm.append(k.to(DEV), vm.to(DEV))
    om = oracle.OracleCache(1, 1, 1, d, bits, max_tokens=T)
    om.append(k, vm)
    q = torch.zeros(1, 1, d, dtype=torch.float16)
    out = cm.attend(q.to(DEV))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert_attention_close(got, om.attend(q))


@pytest.mark.parametrize("Hq", [1, 4], ids=["mha", "group4"])
def test_maximum_split_count(Hq):
    """The largest split count a config allows (max_splits = 4096), forced on a
    cache of 4100 key blocks: about one block per split, most splits without a
    residual, the merge over 4096 partials per query head."""
    _announce("max splits", Hq)
    T = 32 * 4100 + 50
    wl = KVWorkload(1, 1, 128, seed=4096 + Hq, device="cpu")
    k, v = wl.kv(0, T)
    q = wl.q(Hq)
    cache = kv.KiviCache(1, 1, Hq, 128, 2, max_tokens=T, max_splits=4096, device=DEV)
    cache.append(k.to(DEV), v.to(DEV))
    cache.flush()
    cache.set_attend_splits(4096)
    assert cache.plan_attend()[0] == 4096
    out = cache.attend(q.to(DEV))
    torch.cuda.synchronize()
    oc = oracle.OracleCache(1, 1, Hq, 128, 2, max_tokens=T)
    oc.append(k, v)
    oc.flush()
    assert_attention_close(out.cpu().numpy(), oc.attend(q))


def test_largest_unit_count():
    """The largest number of units a cache allows (batch * n_kv_heads = 65504 of
    at most 65535): the launch grids' unit dimension at its limit. Sampled units
    (first, middle, last) against the oracle, bytes and attention."""
    B, Hkv, Hq, d, T = 2047, 32, 32, 128, 200
    _announce("largest unit count", B * Hkv)
    wl = KVWorkload(B, Hkv, d, seed=65504, device=DEV)
    k, v = wl.kv(0, T)
    cache = kv.KiviCache(B, Hkv, Hq, d, 2, max_tokens=T, device=DEV)
    cache.append(k, v)
    cache.flush()
    q = wl.q(Hq)
    out = cache.attend(q)
    torch.cuda.synchronize()
    for u in (0, 33333, B * Hkv - 1):
        b, h = divmod(u, Hkv)
        oc = oracle.OracleCache(1, 1, 1, d, 2, max_tokens=T)
        oc.append(k[b:b + 1, h:h + 1].cpu(), v[b:b + 1, h:h + 1].cpu())
        oc.flush()
        compare_unit(cache, oc, u, 0)
        assert_attention_close(out[b:b + 1, h:h + 1].cpu().numpy(), oc.attend(q[b:b + 1, h:h + 1].cpu()))
