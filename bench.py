"""Benchmark of the KIVI cache hot path on one MI355X.

Metric: decode-attention effective HBM GB/s (and % of the 8 TB/s peak), plus
quantize-append tokens/s.

Default workload: the full-stack decode step (32 layers x batch 128 x 8 KV
heads / 32 query heads x head_dim 128 x 4096 cached tokens, layers 0-15 at
b = 2 and 16-31 at b = 4, bf16 queries), the largest configuration that fits
one GPU; --workload picks another. Its line also carries the
Llama-2-7B-shaped layer's figures (key llama2_7b_layer: the same benchmark
of that workload, run as a child process after the full stack's).

A timed step is one decode step of the whole path over one batch: append one
token per sequence (residual ring), flush when a whole 32-token group lies
beyond the newest 128 (quantize-and-pack keys per channel, values per token),
and the fused split-K decode attention over the packed cache and the fp16
residual. `value` is the algorithmic bytes of those steps (attention reads of
codes, scales, zeros and residual rows, query in, output out; the append and
flush bytes) divided by the wall time of the K timed steps. Inputs are
resident in HBM before the timed region starts. Before the W warm-up steps,
about 50 ms of attention launches over the same caches run back to back, so
that the timed steps see the clocks' steady state rather than the power
manager's start-up transient.

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

# prefill sweeps timed back to back (each cache's median counts)
PF_REPS = 5
# back-to-back attention launches before the warm-up steps (seconds of GPU time)
SETTLE_S = 0.05
SETTLE_MAX_LAUNCHES = 4000
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


def _traffic_from_profile(workload, bits=None):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (of the b-bit layers' launches when `bits` is given), or None when
    there is none or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    key = "hbm_bytes_per_launch" + (f"_b{bits}" if bits is not None else "")
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != _kernel_source_hash():
        return None
    return float(t.group(1))


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_baseline(cfg, seconds=8.0):
    """The oracle as it is, on the host cores: prefill-quantize and attention
    over one batch row (all KV heads) of one layer of the workload, attention
    repeated until about `seconds` have passed, once on every thread and once
    on a single thread. The sample's byte and token rates stand for the whole
    workload's: every (batch row, KV head) unit costs the oracle the same, so
    bytes, tokens and time all scale by the same unit count. Reported in the
    GPU line's units."""
    import numpy as np

    import oracle
    from kivi_inputs import KVWorkload

    Hkv, Hq, d, T = cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    bits = cfg.get("bits", cfg.get("layer_bits", [2])[0])
    q_bf16 = cfg.get("q_dtype") == "bf16"
    import torch
    wl = KVWorkload(1, Hkv, d, seed=cfg["seed"], device="cpu")
    k, v = wl.kv(0, T)
    q = wl.q(Hq, dtype=torch.bfloat16 if q_bf16 else torch.float16)
    n_all = oracle.num_threads()

    gs = None
    if cfg.get("squat_rank"):
        # the SQuat-style coder: the oracle's coefficients from the sample's past queries (set-up, not timed)
        from oracle import squat
        from kivi_inputs import query_history
        qh = query_history(wl, Hq, cfg["squat_queries"], rank=cfg["squat_rank"]).float().numpy()
        group = Hq // Hkv
        gs = np.stack([squat.unit_coefficients(qh[0, h * group:(h + 1) * group].reshape(-1, d),
                                               cfg["squat_rank"], cfg["squat_lambda"]) for h in range(Hkv)])

    def run(threads, secs):
        oracle.set_num_threads(threads)
        oc = oracle.OracleCache(1, Hkv, Hq, d, bits, max_tokens=T)
        if gs is not None:
            oc.set_squat(gs)
        t0 = time.perf_counter()
        oc.append(k, v)
        oc.flush()
        t_prefill = time.perf_counter() - t0
        nt, nq = oc.state()
        nbytes = attend_bytes(Hkv, Hq, d, bits, nq, nt - nq)
        n = 0
        t0 = time.perf_counter()
        while True:
            oc.attend(q, q_is_bf16=q_bf16)
            n += 1
            el = time.perf_counter() - t0
            if el >= secs:
                break
        return nbytes * n / el / 1e9, T / t_prefill, n, el

    try:
        gbs, tok_s, n, el = run(n_all, seconds)
        gbs1, tok_s1, n1, el1 = run(1, seconds / 2)
    finally:
        oracle.set_num_threads(n_all)
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": n_all,
        "kind": "oracle",
        "sample": f"1 batch row x {Hkv} KV heads x {T} tokens of one b={bits} layer of the workload "
                  f"(rates stand for the whole workload: units cost the oracle alike, so bytes, tokens and "
                  f"time scale together); attention repeated {n} times in {el:.1f} s on {n_all} threads and "
                  f"{n1} times in {el1:.1f} s on 1 thread",
        "cpu_model": _cpu_model(),
        "single_thread_gbs": round(gbs1, 4),
        "quantize_append_tokens_per_s": round(tok_s, 1),
        "quantize_append_tokens_per_s_single_thread": round(tok_s1, 1),
    }


def _attend_kernel_name(c):
    """The kernel a cache's kivi_attend_decode launches, and its merge."""
    cfg = c.cfg
    n_split = c.plan_attend()[0]
    gqa4 = (cfg.n_q_heads // cfg.n_kv_heads) % 4 == 0 and cfg.head_dim == 128
    name = "attend_gqa_kernel (four query heads, int8 matrix cores)" if gqa4 else "attend_kernel"
    return name + (" + combine_kernel (merge of %d splits)" % n_split if n_split > 1 else ", one split")


def _arith_dtype(caches):
    """The arithmetic the attention path computes in."""
    c = caches[0].cfg
    if (c.n_q_heads // c.n_kv_heads) % 4 == 0 and c.head_dim == 128:
        return ("i8 x i8 -> i32 (codes against 3 signed-byte digits of 23-bit fixed-point folded queries "
                "and weights) + f32 softmax and sums")
    return "f32 (fp16 code halves in fp32 FMAs)"


def _time_attend(kv, lib, caches, idx, qp, qd, outp, sp, out, rounds):
    """Back-to-back kivi_attend_decode launches over the caches `idx` (in
    order, `rounds` times), bracketed by one pair of HIP events on the stream
    they run on. The settle launches (about 50 ms) and as many untimed
    launches as timed ones (at least 16) go first, enqueued right before the
    timed ones with no host wait between: after the host's pause the launches
    run slower for some 15-20 ms (measured on MI355X: the full stack's kernels
    took up to 20% longer per launch over the first four rounds of its 32
    caches), and the timed launches should see the steady state the decode
    steps run in. Returns (us per launch, algorithmic bytes per launch, n)."""
    import ctypes

    import torch

    handles = [ctypes.c_void_p(caches[i].handle) for i in idx]
    per = [cache_attend_bytes(caches[i]) for i in idx]
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = rounds * len(idx)
    _settle(kv, lib, [caches[i] for i in idx], qp, qd, outp, sp)
    warm = max(n, 16)
    for w in range(warm):
        rc = lib.kivi_attend_decode(handles[w % len(idx)], qp[w % len(qp)], qd, outp, sp)
        if rc != 0:
            raise kv.KiviError(rc, kv.kivi_last_error())
    ev0.record(stream)
    for r in range(rounds):
        for k, h in enumerate(handles):
            rc = lib.kivi_attend_decode(h, qp[(r * len(idx) + k) % len(qp)], qd, outp, sp)
            if rc != 0:
                raise kv.KiviError(rc, kv.kivi_last_error())
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / n, sum(per) / len(per), n


def _side_workload(name, warmup):
    """The benchmark of another workload, run as a child process (its own
    caches; the parent's stay allocated but idle): the fields of its JSON line
    that sit beside the main workload's, or the child's exit status."""
    import subprocess

    cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--no-cpu-baseline",
           "--warmup", str(warmup)]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
    got = [x for x in p.stdout.splitlines() if x.startswith("{")]
    if p.returncode != 0 or not got:
        print(f"[bench] {name}: child run failed (exit {p.returncode})", file=sys.stderr, flush=True)
        return {"workload": name, "error": f"exit {p.returncode}"}
    d = json.loads(got[-1])
    r = d["roofline"]
    return {"workload": name, "config": d["config"], "value": d["value"], "unit": d["unit"],
            "pct_of_peak": d["pct_of_peak"], "ms_per_step": d["ms_per_step"], "steps": d["steps"],
            "warmup": d["warmup"], "dtype": d["dtype"],
            "roofline": {k: r[k] for k in ("kernel", "achieved", "frac", "avg_launch_us",
                                           "algorithmic_bytes_per_launch", "timed_launches", "traffic")},
            "quantize_append_tokens_per_s": d["quantize_append_tokens_per_s"],
            "quantize_append_gbs": d["quantize_append_gbs"],
            "quantize_append_pct_of_peak": d["quantize_append_pct_of_peak"]}


def _settle(kv, lib, caches, qp, qd, outp, sp):
    """kivi_attend_decode over the caches in turn, back to back, for about
    SETTLE_S of GPU time at 6 TB/s of algorithmic bytes (at most
    SETTLE_MAX_LAUNCHES launches), with no host wait: the clocks then sit in
    their steady state for what follows on the stream."""
    import ctypes

    handles = [ctypes.c_void_p(c.handle) for c in caches]
    per = [cache_attend_bytes(c) for c in caches]
    n = min(SETTLE_MAX_LAUNCHES, max(len(caches), int(SETTLE_S * 6e12 * len(per) / sum(per))))
    for w in range(n):
        rc = lib.kivi_attend_decode(handles[w % len(handles)], qp[w % len(qp)], qd, outp, sp)
        if rc != 0:
            raise kv.KiviError(rc, kv.kivi_last_error())
    print(f"[bench] settle: {n} attention launches over {len(caches)} cache(s)", file=sys.stderr, flush=True)


def _time_attend_single(kv, lib, caches, idx, qp, qd, outp, sp):
    """Each launch between its own pair of HIP events, the host waiting for
    it before the next: us per launch (no overlap with a neighbour)."""
    import ctypes

    import torch

    stream = torch.cuda.current_stream()
    ts = []
    for k, i in enumerate(idx):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.kivi_attend_decode(ctypes.c_void_p(caches[i].handle), qp[k % len(qp)], qd, outp, sp)
        if rc != 0:
            raise kv.KiviError(rc, kv.kivi_last_error())
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return sum(ts) / len(ts)


def _stream_probe(dev, nbytes=256 << 20):
    """The box's plain streaming rates on `nbytes` buffers (torch's copy and
    sum kernels, HIP events, best of 5): copy GB/s counts the bytes read plus
    written, sum GB/s the bytes read. Context for the attention roofline."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    best_copy = best_sum = float("inf")
    for _ in range(5):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        best_copy = min(best_copy, ev[0].elapsed_time(ev[1]))
        ev[0].record()
        torch.sum(src, dim=0, out=acc)
        ev[1].record()
        torch.cuda.synchronize()
        best_sum = min(best_sum, ev[0].elapsed_time(ev[1]))
    del src, dst
    return {"bytes": nbytes, "copy_gbs": round(2 * nbytes / (best_copy * 1e-3) / 1e9, 1),
            "sum_read_gbs": round(nbytes / (best_sum * 1e-3) / 1e9, 1), "how": "torch copy_ / sum, best of 5"}


PEAK_FP32_TFLOPS = 157.3


def _squat_measure(kv, cfg, dev, caches, prefill_inputs, reps=8):
    """The SQuat-style key coder on the workload's first layer: the build of
    the coefficients (HIP events), and the prefill (append(T) + flush into an
    empty cache) with the coder against the same prefill on a cache without
    it; the difference is the code kernel's time (the launches are otherwise
    the same). Its algorithmic work, in the subspace's coordinates, is 2 r
    fused multiply-adds per element (the correction it receives and the update
    it makes), 2 flops each, against the fp32 vector peak; it also reads the
    fp16 key rows again and writes the key codes."""
    import torch

    import kv_cache_compression_kivi_amd as kvm
    from kivi_inputs import KVWorkload, query_history

    B, Hkv, Hq, d, T = cfg["batch"], cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    bits, rank, lam, nqh = cfg.get("bits", 2), cfg["squat_rank"], cfg["squat_lambda"], cfg["squat_queries"]
    k, v = prefill_inputs[min(prefill_inputs)]
    qh = query_history(KVWorkload(B, Hkv, d, seed=cfg["seed"], device=dev), Hq, nqh, rank=rank)
    sq = kvm.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=dev, squat_rank=rank)
    plain = kvm.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    def prefill(c):
        c.reset()
        c.append(k, v)
        c.flush()

    sq.squat_build(qh, lam)  # warm
    torch.cuda.synchronize()
    build_us = min(timed(lambda: sq.squat_build(qh, lam)) for _ in range(3))
    prefill(sq)
    prefill(plain)
    t_sq, t_pl = [], []
    for _ in range(reps):
        t_sq.append(timed(lambda: prefill(sq)))
        t_pl.append(timed(lambda: prefill(plain)))
    us_sq, us_pl = sum(t_sq) / reps, sum(t_pl) / reps
    nq = sq.state()[1]
    # per quantized token per unit: the correction u_c . a and the update a += delta w_c, r FMAs
    # each, for each of the d elements (2 flops per FMA); the key row read (fp16) and the codes written
    flops = 2.0 * B * Hkv * nq * d * 2 * rank
    nbytes = B * Hkv * nq * (2 * d + d * bits // 8)
    codes_us = us_sq - us_pl
    tf = flops / (codes_us * 1e-6) / 1e12
    return {
        "rank": rank, "lambda": lam, "past_queries_per_head": nqh,
        "build_us": round(build_us, 2),
        "prefill_us": round(us_sq, 2), "prefill_plain_us": round(us_pl, 2),
        "prefill_tokens_per_s": round(B * T / (us_sq * 1e-6), 1),
        "prefill_plain_tokens_per_s": round(B * T / (us_pl * 1e-6), 1),
        "codes_us": round(codes_us, 2),
        "codes_gbs": round(nbytes / (codes_us * 1e-6) / 1e9, 1),
        "roofline": {"bound": "alu", "kernel": "squat_codes_kernel (fp32 FMAs of the element-by-element walk)",
                     "achieved": round(tf, 2), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP32_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                     "how": "prefill with the coder minus the same prefill without it, HIP events"},
    }


def _profile_prefill(workload, n):
    """n prefills of the workload's first layer into one cache, back to back,
    each timed with its own pair of HIP events (for a profile of the quantizer
    alone), after untimed ones for at least 0.5 s: measured on MI355X, a GPU
    that starts cold runs the first tens of milliseconds of prefills up to 35%
    slower than later ones."""
    import torch

    import kv_cache_compression_kivi_amd as kv
    from kivi_inputs import CONFIGS, KVWorkload

    kv.load_library()
    cfg = dict(CONFIGS[workload])
    B, Hkv, Hq, d, T = cfg["batch"], cfg["n_kv_heads"], cfg["n_q_heads"], cfg["head_dim"], cfg["T"]
    bits = cfg.get("bits", cfg.get("layer_bits", [2])[0])
    dev = torch.device("cuda:0")
    wl = KVWorkload(B, Hkv, d, seed=cfg["seed"], device=dev)
    k, v = wl.kv(0, T)
    c = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=T, device=dev, squat_rank=cfg.get("squat_rank", 0))
    if cfg.get("squat_rank"):
        from kivi_inputs import query_history
        c.squat_build(query_history(wl, Hq, cfg["squat_queries"], rank=cfg["squat_rank"]), cfg["squat_lambda"])
    stream = torch.cuda.current_stream()
    warm, t_start = 0, time.perf_counter()
    while time.perf_counter() - t_start < 0.5:
        for _ in range(8):
            c.reset()
            c.append(k, v)
            c.flush()
        warm += 8
        torch.cuda.synchronize()
    evs = []
    for _ in range(n):
        c.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        c.append(k, v)
        c.flush()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) * 1e3 for a, b in evs]
    nt, nq, _ = c.state()
    nb = prefill_bytes(B * Hkv, d, bits, nt, nq)
    avg = sum(ts) / len(ts)
    print(f"[bench] prefill profile {workload}: {warm} untimed then {n} timed prefills of B={B} x Hkv={Hkv} x T={T} "
          f"(b={bits}), back to back: {avg:.2f} us each by HIP events (min {min(ts):.2f}, max {max(ts):.2f}), {nb} "
          f"algorithmic bytes -> {nb / (avg * 1e-6) / 1e9:.1f} GB/s, {B * T / (avg * 1e-6):.4g} tokens/s (B*T)",
          file=sys.stderr, flush=True)


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default: 100 for full_stack, 200 otherwise)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="full_stack",
                    choices=["tiny", "llama2_7b_layer", "long_context", "gqa_streaming", "full_stack",
                             "gqa_ragged", "gqa_paged", "gqa_paged_256", "llama2_7b_layer_squat"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side-workload", action="store_true",
                    help="full_stack only: skip the Llama-2-7B-shaped layer's figures (a child run of "
                         "--workload llama2_7b_layer) that the line otherwise carries")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--profile-prefill", type=int, default=0, metavar="N",
                    help="for profiles of the quantizer: untimed prefills (append(T) + flush into an emptied "
                         "cache) of the workload's first layer for 0.5 s, then N timed ones back to back, each "
                         "between its own HIP events, then exit (no decode steps, no JSON line)")
    ap.add_argument("--profile", action="store_true",
                    help="for hardware-counter runs: the decode steps and attention launches of the default "
                         "run, then a plain 256 MiB device copy (the counters' calibration); no prefill "
                         "timing, no CPU baseline, no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the KV cache units are independent per (batch row, KV head), "
              "so a multi-GPU run would shard them with no communication; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = 100 if args.workload == "full_stack" else 200
    if args.profile_prefill:
        _profile_prefill(args.workload, args.profile_prefill)
        return

    import ctypes

    import torch

    import kv_cache_compression_kivi_amd as kv
    from kivi_inputs import CONFIGS, KVWorkload, page_order, query_history, row_lengths

    lib = kv.load_library()
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
    max_tokens = T + -(-total_steps // n_rot) + 64
    print(f"[bench] workload {args.workload}: {layers} layer(s) x {n_rot} rotation(s), "
          f"{per_step_bytes / 1e6:.1f} MB per step", file=sys.stderr, flush=True)

    # the layers whose prefill is timed (and whose inputs are kept): the first and last of each bit width
    pf_layers = sorted({min(i for i in range(layers) if layer_bits[i] == b) for b in set(layer_bits)} |
                       {max(i for i in range(layers) if layer_bits[i] == b) for b in set(layer_bits)})
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
                c = kv.KiviCache(B, Hkv, Hq, d, bits, max_tokens=max_tokens, device=dev,
                                 squat_rank=cfg.get("squat_rank", 0))
            if cfg.get("squat_rank"):
                # the SQuat-style coder's coefficients from the layer's past queries, before the prefill
                c.squat_build(query_history(wl, Hq, cfg["squat_queries"], rank=cfg["squat_rank"]),
                              cfg["squat_lambda"])
            if cfg.get("ragged"):
                c.append_rows(k, v, lens)
            else:
                c.append(k, v)
            c.flush()
            caches.append(c)
            if r == 0 and layer in pf_layers[:1] + pf_layers[-1:]:
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
    qd = kv.KIVI_BF16 if q_dtype == torch.bfloat16 else kv.KIVI_F16
    nfl = ctypes.c_int32()
    kvp = [(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr())) for a, b in new_kv]
    qp = [ctypes.c_void_p(x.data_ptr()) for x in queries]
    outp = ctypes.c_void_p(out.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)
    handles = [ctypes.c_void_p(c.handle) for c in caches]

    def run_step(i):
        r = i % n_rot
        for layer in range(layers):
            kp, vp = kvp[i % pool]
            rc = lib.kivi_decode_step(handles[r * layers + layer], kp, vp, qp[i % pool], qd, outp, sp,
                                      ctypes.byref(nfl))
            if rc != 0:
                raise kv.KiviError(rc, kv.kivi_last_error())

    # the bytes of each step follow from the host counters alone: replay the
    # counter arithmetic of the warm-up and timed steps before any of them runs
    # (so that no host pause falls between the two; checked against the caches
    # afterwards), counting the timed steps' bytes
    bytes_total = 0
    sim_state = [row_groups(c) for c in caches]
    for i in range(total_steps):
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
                if i >= args.warmup:
                    bytes_total += b
                groups.append((nt, nq, nr, w))
            sim_state[ci] = groups
    # settle: attention launches over the caches back to back for about
    # SETTLE_S, enqueued right before the warm-up steps. On MI355X the first
    # ~15 ms of back-to-back work after a pause is a power-management transient
    # (on the GQA streaming layer its launches ran 100 us for ~1.6 ms, then
    # 121-126 us, easing back to ~103 us ~15 ms in), longer than the warm-up
    # steps of a one-layer workload; the timed steps should see the steady
    # state. The launches read the caches and change no state.
    _settle(kv, lib, caches, qp, qd, outp, sp)
    for i in range(args.warmup):
        run_step(i)
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

    # the attention launches alone: every cache in step order, back to back
    rounds = max(2, min(200 // len(caches), 25)) if len(caches) < 200 else 1
    rounds = max(rounds, 5) if layers > 1 else max(rounds, -(-160 // len(caches)))
    att_us, att_bytes, n_att = _time_attend(kv, lib, caches, list(range(len(caches))), qp, qd, outp, sp, out,
                                            rounds)
    att_gbs = att_bytes / (att_us * 1e-6) / 1e9
    # and per bit width (their kernels differ), when the layers mix them
    by_bits = {}
    if len(set(layer_bits)) > 1:
        for bw in sorted(set(layer_bits)):
            idx = [i for i in range(len(caches)) if caches[i].cfg.bits == bw]
            us, nb, n = _time_attend(kv, lib, caches, idx, qp, qd, outp, sp, out, max(5, rounds))
            by_bits[str(bw)] = {"kernel": _attend_kernel_name(caches[idx[0]]), "layers": len(idx),
                                "achieved": round(nb / (us * 1e-6) / 1e9, 2),
                                "frac": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                "algorithmic_bytes_per_launch": int(nb), "avg_launch_us": round(us, 3),
                                "timed_launches": n}
    single_us = _time_attend_single(kv, lib, caches, list(range(min(len(caches), 32))), qp, qd, outp, sp)
    if args.profile:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # known traffic: 256 MiB read + 256 MiB written per copy
        torch.cuda.synchronize()
        print(f"[bench] profile: the last {n_att} attention calls (before the single-launch ones) carry "
              f"{att_bytes:.0f} algorithmic bytes each ({att_us:.2f} us back to back, {single_us:.2f} us one at a "
              f"time); then 3 copies of {256 << 20} bytes", file=sys.stderr, flush=True)
        return

    # prefill quantize-append: append(T) + flush into an empty cache, on the
    # first and last layer of each bit width (the first and last input kept),
    # PF_REPS sweeps back to back; each cache's median prefill counts
    pf_idx = pf_layers if layers > 1 else list(range(min(len(caches), max(4, n_rot))))
    pf_ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in pf_idx]
             for _ in range(PF_REPS)]
    pf_bytes = pf_tokens = pf_unit_tokens = 0
    for rep in range(PF_REPS):
        for e, i in zip(pf_ev[rep], pf_idx):
            c = caches[i]
            k, v = prefill_inputs.get(i % layers, prefill_inputs[min(prefill_inputs)])
            c.reset()
            e[0].record(stream)
            if cfg.get("ragged"):
                c.append_rows(k, v, lens)
            else:
                c.append(k, v)
            c.flush()
            e[1].record(stream)
            if rep == 0:
                pf_bytes += sum(prefill_bytes(Hkv * w, d, c.cfg.bits, nt, nq) for nt, nq, _, w in row_groups(c))
                pf_tokens += sum(lens)
                pf_unit_tokens += Hkv * sum(lens)
    torch.cuda.synchronize()
    pf_us_each = [sorted(pf_ev[rep][j][0].elapsed_time(pf_ev[rep][j][1]) * 1e3 for rep in range(PF_REPS))
                  for j in range(len(pf_idx))]
    pf_ms = sum(t[len(t) // 2] for t in pf_us_each) * 1e-3
    pf_tok_s = pf_tokens / (pf_ms * 1e-3)
    pf_gbs = pf_bytes / (pf_ms * 1e-3) / 1e9

    # single-token appends (ring writes only) and one 32-token flush, on the
    # caches just prefilled: n_res = R there, so 32 appends fit before the ring
    # is full and the flush then quantizes exactly one group (rows at one length only)
    ap_us = fl_us = fl_gbs = None
    if not cfg.get("ragged"):
        ap_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in pf_idx]
        n_ap = 32
        for e, i in zip(ap_ev, pf_idx):
            h = handles[i]
            assert caches[i].state()[2] == 128
            e[0].record(stream)
            for t in range(n_ap):
                kp, vp = kvp[t % pool]
                rc = lib.kivi_append(h, kp, vp, 1, sp)
                if rc != 0:
                    raise kv.KiviError(rc, kv.kivi_last_error())
            e[1].record(stream)
            rc = lib.kivi_flush(h, sp, ctypes.byref(nfl))
            if rc != 0:
                raise kv.KiviError(rc, kv.kivi_last_error())
            e[2].record(stream)
            assert nfl.value == 32, nfl.value
        torch.cuda.synchronize()
        ap_us = sum(e[0].elapsed_time(e[1]) for e in ap_ev) * 1e3 / (len(pf_idx) * n_ap)
        fl_us = sum(e[1].elapsed_time(e[2]) for e in ap_ev) * 1e3 / len(pf_idx)
        fl_gbs = (sum(flush_bytes(units, d, caches[i].cfg.bits, 32) for i in pf_idx) / len(pf_idx) /
                  (fl_us * 1e-6) / 1e9)

    squat_line = _squat_measure(kv, cfg, dev, caches, prefill_inputs) if cfg.get("squat_rank") else None
    probe = _stream_probe(dev)
    traffic = _traffic_from_profile(args.workload)
    if by_bits:
        for bw, e in by_bits.items():
            e["traffic"] = _traffic_from_profile(args.workload, bits=bw)
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
        "dtype": _arith_dtype(caches),
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
        # prefill: append(T) + flush into an empty cache; a token is one sequence's token (B*T per layer)
        "quantize_append_tokens_per_s": round(pf_tok_s, 1),
        "quantize_append_unit_tokens_per_s": round(pf_unit_tokens / (pf_ms * 1e-3), 1),
        "quantize_append_gbs": round(pf_gbs, 2),
        "quantize_append_pct_of_peak": round(100.0 * pf_gbs / PEAK_HBM_GBS, 2),
        "quantize_append_layers_timed": pf_idx if layers > 1 else None,
        "quantize_append_us_each": [[round(x, 2) for x in t] for t in pf_us_each],
        "quantize_append_reps": PF_REPS,
        "append_1_token_us": round(ap_us, 3) if ap_us else None,
        # B tokens per call (one per sequence)
        "append_1_token_tokens_per_s": round(B / (ap_us * 1e-6), 1) if ap_us else None,
        "flush_32_tokens_us": round(fl_us, 3) if fl_us else None,
        "flush_32_tokens_gbs": round(fl_gbs, 2) if fl_gbs else None,
        "roofline": {
            "bound": "hbm",
            "kernel": "kivi_attend_decode = " + " / ".join(sorted({_attend_kernel_name(c) for c in caches})),
            "achieved": round(att_gbs, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(att_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(att_bytes),
            "avg_launch_us": round(att_us, 3),
            "timed_launches": n_att,
            "single_launch_us": round(single_us, 3),
            "by_bits": by_bits or None,
        },
        "stream_probe": probe,
        "squat": squat_line,
        "cpu_baseline": None,
    }
    if args.workload == "full_stack" and not args.no_side_workload:
        # the Llama-2-7B-shaped layer alongside the full stack's line
        line["llama2_7b_layer"] = _side_workload("llama2_7b_layer", args.warmup)
    if not args.no_cpu_baseline:
        try:
            line["cpu_baseline"] = _cpu_baseline(cfg, seconds=args.cpu_seconds)
        except Exception as e:  # the GPU line stands on its own
            line["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
