"""Benchmark of the KIVI cache hot path on one MI355X.

Metric: decode-attention effective HBM GB/s (and % of the 8 TB/s peak), plus
quantize-append tokens/s.

A timed step is one decode step of the whole path over one batch: append one
token per sequence (residual ring), flush when a whole 32-token group lies
beyond the newest 128 (quantize-and-pack keys per channel, values per token),
and the fused split-K decode attention over the packed cache and the fp16
residual. `value` is the algorithmic bytes of those steps (attention reads of
codes, scales, zeros and residual rows, query in, output out; the append and
flush bytes) divided by the wall time of the K timed steps. Inputs are
resident in HBM before the timed region starts.

The 256 MB Infinity Cache would hold a whole llama2_7b_layer cache (147 MB),
so steps rotate over independent caches whose total exceeds 1 GiB.

Also measured in the same run:
  * the attention kernel alone (one launch per kivi_attend_decode), timed with
    HIP events on the stream it runs on, for the roofline entry;
  * prefill quantize-append (append(T) + flush into an empty cache): tokens/s;
  * single-token append latency (ring write) and one 32-token flush: latency
    and GB/s;
  * the CPU oracle on a bounded sample of the same workload (cpu_baseline).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "decode-attention effective HBM GB/s (% of peak) + quantize-append tokens/s"


# ---------------------------------------------------------------- byte accounting

def bytes_per_quant_token(d, bits, G=32, vg=32):
    """Key codes + value codes + key (s, z) share + value (s, z), per token per KV head."""
    return 2 * d * bits // 8 + 8 * d // G + 8 * d // vg


def attend_bytes(units, rows, d, bits, n_quant, n_resid):
    """Algorithmic bytes of one decode attention: the packed part, the fp16
    residual (key + value rows), each query head's fp16 query and fp32 output."""
    return units * (n_quant * bytes_per_quant_token(d, bits) + n_resid * 4 * d) + rows * (2 * d + 4 * d)


def append_bytes(units, d, ntok):
    """fp16 key + value rows read and written into the ring."""
    return units * ntok * 4 * d * 2


def flush_bytes(units, d, bits, ntok):
    """fp16 rows read from the ring, packed codes + statistics written."""
    return units * ntok * (4 * d + bytes_per_quant_token(d, bits))


def prefill_bytes(units, d, bits, T, n_quant):
    """append(T) + flush into an empty cache: fp16 input read once; the packed
    part and the residual written."""
    return units * (T * 4 * d + n_quant * bytes_per_quant_token(d, bits) + (T - n_quant) * 4 * d)


def row_groups(c):
    """A cache's rows grouped by their counters: [(n_tokens, n_quant, n_resid, rows)]."""
    from collections import Counter
    cnt = Counter(c.row_state(b) for b in range(c.cfg.batch))
    return [(nt, nq, nr, w) for (nt, nq, nr), w in sorted(cnt.items())]


def cache_attend_bytes(c):
    """Algorithmic bytes of one decode attention over the cache's current rows."""
    Hkv, Hq, d, bits = c.cfg.n_kv_heads, c.cfg.n_q_heads, c.cfg.head_dim, c.cfg.bits
    return sum(attend_bytes(Hkv * w, Hq * w, d, bits, nq, nr) for _, nq, nr, w in row_groups(c))


# ---------------------------------------------------------------- helpers

ATTEND_SOURCES = ("attend.hip", "attend_gqa.hip", "attend_common.hpp", "split.hpp", "launch.hpp", "planner.hpp")


def _kernel_source_hash():
    """Hash of the sources the attention kernels are built from, without their
    // comments and blank lines: a counter summary taken before any code in
    them changed no longer describes the kernel."""
    h = hashlib.sha256()
    for name in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_compression_kivi_amd", "csrc", name), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode("utf-8") + b"\n")
    return h.hexdigest()[:16]


def _traffic_from_profile(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when there is none or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != _kernel_source_hash():
        return None
    return float(t.group(1))


def _cpu_baseline(cfg, seconds=8.0):
    """The oracle as it is, on the host cores: prefill-quantize and attention
    over one batch row (all KV heads) of the workload, attention repeated until
    about `seconds` have passed. Reported in the same units as the GPU line."""
    import torch

    import oracle
    from kivi_inputs import KVWorkload

    Hkv, Hq, d, T, bits = cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"], cfg.get("bits", 2)
    wl = KVWorkload(1, Hkv, d, seed=cfg["seed"], device="cpu")
    k, v = wl.kv(0, T)
    q = wl.q(Hq)
    oc = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=T)
    t0 = time.perf_counter()
    oc.append(k, v)
    oc.flush()
    t_prefill = time.perf_counter() - t0
    nt, nq = oc.state()
    nbytes = attend_bytes(Hkv, Hq, d, bits, nq, nt - nq)
    n = 0
    t0 = time.perf_counter()
    while True:
        oc.attend(q)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    del torch
    return {
        "value": round(nbytes * n / el / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"1 batch row x {Hkv} KV heads x {T} tokens of the workload; attention repeated {n} times "
                  f"in {el:.1f} s; prefill-quantize of the same sample {Hkv * T / t_prefill:.0f} tokens/s",
        "quantize_append_tokens_per_s": round(Hkv * T / t_prefill, 1),
    }


def _time_attend(kv, lib, caches, handles, qp, qd, outp, stream, sp, units, rows, d, q0, out, n_att=None):
    """The attention launches alone: n_att back-to-back kivi_attend_decode
    calls over the rotating caches, bracketed by one pair of HIP events on the
    stream they run on. Returns (ms per call, algorithmic bytes per call, n)."""
    import torch

    n_caches = len(caches)
    if n_att is None:
        n_att = max(2 * n_caches, min(200, 20 * n_caches))
    per_cache = [cache_attend_bytes(c) for c in caches]
    att_bytes = sum(per_cache[i % n_caches] for i in range(n_att))
    for i in range(min(n_caches, 8)):  # warm the launch path
        caches[i].attend(q0, out=out)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n_att):
        rc = lib.kivi_attend_decode(handles[i % n_caches], qp[i % len(qp)], qd, outp, sp)
        if rc != 0:
            raise kv.KiviError(rc, kv.kivi_last_error())
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n_att, att_bytes / n_att, n_att


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama2_7b_layer",
                    choices=["tiny", "llama2_7b_layer", "long_context", "gqa_streaming", "full_stack",
                             "gqa_ragged", "gqa_paged"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--profile", action="store_true",
                    help="for hardware-counter runs: the decode steps and attention launches of the default "
                         "run, then a plain 256 MiB device copy (the counters' calibration); no prefill "
                         "timing, no CPU baseline, no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the KV cache units are independent per (batch row, KV head), "
              "so a multi-GPU run would shard them with no communication; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_compression_kivi_amd as kv
    from kivi_inputs import CONFIGS, KVWorkload, page_order, row_lengths

    kv.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = dict(CONFIGS[args.workload])
    B, Hkv, Hq, d, T = cfg["batch"], cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    units, rows = B * Hkv, B * Hq
    layers = cfg.get("layers", 1)
    layer_bits = cfg.get("layer_bits", [cfg.get("bits", 2)] * layers)
    q_dtype = torch.bfloat16 if cfg.get("q_dtype") == "bf16" else torch.float16
    total_steps = args.warmup + args.steps
    # a serving batch: each sequence at its own seeded length (appended with kivi_append_rows)
    lens = row_lengths(B, cfg["ragged"][0], cfg["ragged"][1], cfg["seed"]) if cfg.get("ragged") else [T] * B

    # one cache per layer; rotate over copies when a step's working set would sit in the Infinity Cache
    per_step_bytes = sum(attend_bytes(Hkv, Hq, d, b, max(0, (t - 128) // 32 * 32), t - max(0, (t - 128) // 32 * 32))
                         for b in layer_bits for t in lens)
    n_rot = 1 if per_step_bytes >= (1 << 30) else min(16, int(-(-(1 << 30) // per_step_bytes)))
    n_caches = n_rot * layers
    max_tokens = T + -(-total_steps // n_rot) + 64
    print(f"[bench] workload {args.workload}: {layers} layer(s) x {n_rot} rotation(s), "
          f"{per_step_bytes / 1e6:.1f} MB per step", file=sys.stderr, flush=True)

    caches = []
    prefill_inputs = {}
    for r in range(n_rot):
        for layer in range(layers):
            bits = layer_bits[layer]
            wl = KVWorkload(B, Hkv, d, seed=cfg["seed"], layer=layer + 1000 * r, device=dev)
            k, v = wl.kv(0, T)
            if cfg.get("paged"):
                # a pool page for every block a row can hold, the table taking them in a seeded random order
                mb = max_tokens // 32
                c = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, device=dev, n_pages=B * mb)
                c.set_block_table(page_order(B * mb, cfg["seed"] + 1000 * len(caches)).reshape(B, mb).to(dev))
            else:
                c = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, device=dev)
            if cfg.get("ragged"):
                c.append_rows(k, v, lens)
            else:
                c.append(k, v)
            c.flush()
            caches.append(c)
            if r == 0 and layer in (0, layers - 1):
                prefill_inputs[layer] = (k, v)
            del k, v
    torch.cuda.synchronize()

    # decode inputs, resident before timing: a pool of new tokens and queries
    wl0 = KVWorkload(B, Hkv, d, seed=cfg["seed"], device=dev)
    pool = 32
    new_kv = [wl0.kv(T + i, 1) for i in range(pool)]
    queries = [wl0.q(Hq, step=i, dtype=q_dtype) for i in range(pool)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    s_ptr = stream.cuda_stream

    lib = kv.load_library()
    import ctypes
    qd = kv.KIVI_BF16 if q_dtype == torch.bfloat16 else kv.KIVI_F16
    nfl = ctypes.c_int32()
    kvp = [(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr())) for a, b in new_kv]
    qp = [ctypes.c_void_p(x.data_ptr()) for x in queries]
    outp = ctypes.c_void_p(out.data_ptr())
    sp = ctypes.c_void_p(s_ptr)
    handles = [ctypes.c_void_p(c.handle) for c in caches]

    def run_step(i):
        r = i % n_rot
        for layer in range(layers):
            kp, vp = kvp[i % pool]
            rc = lib.kivi_decode_step(handles[r * layers + layer], kp, vp, qp[i % pool], qd, outp, sp,
                                      ctypes.byref(nfl))
            if rc != 0:
                raise kv.KiviError(rc, kv.kivi_last_error())

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    # the bytes of each step follow from the host counters alone: replay the
    # counter arithmetic before timing (checked against the caches afterwards)
    bytes_total = 0
    sim_state = [row_groups(c) for c in caches]
    for i in range(args.warmup, total_steps):
        r = i % n_rot
        for layer in range(layers):
            ci = r * layers + layer
            groups = []
            for nt, nq, nr, w in sim_state[ci]:
                nt, nr = nt + 1, nr + 1
                b = append_bytes(Hkv * w, d, 1)
                if nr >= 128 + 32:
                    b += flush_bytes(Hkv * w, d, layer_bits[layer], 32)
                    nq, nr = nq + 32, nr - 32
                b += attend_bytes(Hkv * w, Hq * w, d, layer_bits[layer], nq, nr)
                bytes_total += b
                groups.append((nt, nq, nr, w))
            sim_state[ci] = groups
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total_steps):
        run_step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ci, c in enumerate(caches):
        assert row_groups(c) == sorted(sim_state[ci]), (row_groups(c), sim_state[ci])
    ms_per_step = wall / args.steps * 1e3
    value = bytes_total / wall / 1e9

    att_avg_ms, att_bytes_avg, n_att = _time_attend(kv, lib, caches, handles, qp, qd, outp, stream, sp, units, rows, d,
                                                    queries[0], out)
    att_gbs = att_bytes_avg / (att_avg_ms * 1e-3) / 1e9
    if args.profile:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # known traffic: 256 MiB read + 256 MiB written per copy
        torch.cuda.synchronize()
        print(f"[bench] profile: the last {n_att} attention calls carry {att_bytes_avg:.0f} algorithmic bytes "
              f"each ({att_avg_ms * 1e3:.2f} us); then 3 copies of {256 << 20} bytes", file=sys.stderr, flush=True)
        return

    # prefill quantize-append: append(T) + flush into an empty cache
    n_pf = min(len(caches), max(4, n_rot))
    pf_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_pf)]
    pf_bytes = 0
    for i in range(n_pf):
        c = caches[i]
        layer = i % layers
        k, v = prefill_inputs.get(layer, prefill_inputs[0])
        c.reset()
        pf_ev[i][0].record(stream)
        if cfg.get("ragged"):
            c.append_rows(k, v, lens)
        else:
            c.append(k, v)
        c.flush()
        pf_ev[i][1].record(stream)
        pf_bytes += sum(prefill_bytes(Hkv * w, d, c.cfg.bits, nt, nq) for nt, nq, _, w in row_groups(c))
    torch.cuda.synchronize()
    pf_ms = sum(a.elapsed_time(b) for a, b in pf_ev)
    pf_tok_s = n_pf * Hkv * sum(lens) / (pf_ms * 1e-3)
    pf_gbs = pf_bytes / (pf_ms * 1e-3) / 1e9

    # single-token appends (ring writes only) and one 32-token flush, on the
    # caches just prefilled: n_res = R there, so 32 appends fit before the ring
    # is full and the flush then quantizes exactly one group (rows at one length only)
    ap_us = fl_us = fl_gbs = None
    if not cfg.get("ragged"):
        ap_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_pf)]
        n_ap = 32
        for i in range(n_pf):
            h = handles[i]
            assert caches[i].state()[2] == 128
            ap_ev[i][0].record(stream)
            for t in range(n_ap):
                kp, vp = kvp[t % pool]
                rc = lib.kivi_append(h, kp, vp, 1, sp)
                if rc != 0:
                    raise kv.KiviError(rc, kv.kivi_last_error())
            ap_ev[i][1].record(stream)
            rc = lib.kivi_flush(h, sp, ctypes.byref(nfl))
            if rc != 0:
                raise kv.KiviError(rc, kv.kivi_last_error())
            ap_ev[i][2].record(stream)
            assert nfl.value == 32, nfl.value
        torch.cuda.synchronize()
        ap_us = sum(e[0].elapsed_time(e[1]) for e in ap_ev) * 1e3 / (n_pf * n_ap)
        fl_us = sum(e[1].elapsed_time(e[2]) for e in ap_ev) * 1e3 / n_pf
        fl_gbs = sum(flush_bytes(units, d, caches[i].cfg.bits, 32) for i in range(n_pf)) / n_pf / (fl_us * 1e-6) / 1e9

    traffic = _traffic_from_profile(args.workload)
    plan = caches[0].plan_attend()
    gqa4 = (Hq // Hkv) % 4 == 0 and d == 128
    attend_kernel_name = ("kivi_attend_decode = " + ("attend_gqa_kernel (four query heads, int8 matrix cores)"
                                                     if gqa4 else "attend_kernel") +
                          (" + combine_kernel (merge of %d splits)" % plan[0] if plan[0] > 1 else ", one split"))
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "n_kv_heads": Hkv, "n_q_heads": Hq, "head_dim": d,
                   "tokens": T if not cfg.get("ragged") else {"per_row": "uniform over [%d, %d]" % tuple(cfg["ragged"]),
                                                              "min": min(lens), "max": max(lens),
                                                              "mean": round(sum(lens) / B, 1)},
                   "bits": layer_bits if layers > 1 else layer_bits[0], "layers": layers,
                   "k_block": 32, "v_group": 32, "residual": 128, "q_dtype": str(q_dtype).replace("torch.", ""),
                   "step": "append 1 token + flush when due + decode attention, per layer",
                   "blocks": "paged (pool pages in random order)" if cfg.get("paged") else "one region per unit",
                   "rotating_caches": n_rot},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "quantize_append_tokens_per_s": round(pf_tok_s, 1),
        "quantize_append_gbs": round(pf_gbs, 2),
        "append_1_token_us": round(ap_us, 3) if ap_us else None,
        "append_1_token_tokens_per_s": round(units / (ap_us * 1e-6), 1) if ap_us else None,
        "flush_32_tokens_us": round(fl_us, 3) if fl_us else None,
        "flush_32_tokens_gbs": round(fl_gbs, 2) if fl_gbs else None,
        "roofline": {
            "bound": "hbm",
            "kernel": attend_kernel_name,
            "achieved": round(att_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(att_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(att_bytes_avg),
            "avg_launch_us": round(att_avg_ms * 1e3, 3),
            "timed_launches": n_att,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        try:
            line["cpu_baseline"] = _cpu_baseline(cfg, seconds=args.cpu_seconds)
        except Exception as e:  # the GPU line stands on its own
            line["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
