"""CPU checks of bench.py's contract: its byte model against the record layout
the library reports, the gate on the committed counter summaries, and the
one-GPU refusal. No GPU work and no timing."""

import os
import subprocess
import sys

import pytest

import bench
from kv_cache_compression_kivi_amd import _native as native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 4])
def test_quantized_token_bytes_equal_the_record(d, bits):
    """A 32-token key-block record holds exactly the algorithmic bytes the
    byte model charges for its tokens (codes, scales and zeros, no padding),
    and a ring slot holds one token's fp16 key and value rows."""
    L = native.kivi_cache_layout(native.make_config(1, 1, 1, d, bits, 1024))
    assert bench.bytes_per_quant_token(d, bits) * 32 == L.block_bytes
    # 2-bit: 128 B per token at d = 128 (32 key codes + 32 value codes + 32 + 32 of statistics)
    if d == 128:
        assert bench.bytes_per_quant_token(d, bits) == {2: 128, 4: 192}[bits]


def test_attend_bytes_hand_count():
    """One call over 2 units with 4 query heads, 96 quantized and 40 fp16
    tokens each, d = 64, b = 2: 96 x (16 + 16 + 16 + 16) + 40 x 256 per unit,
    and 64 x 2 (query) + 64 x 4 (output) per query head."""
    want = 2 * (96 * 64 + 40 * 256) + 4 * (128 + 256)
    assert bench.attend_bytes(2, 4, 64, 2, 96, 40) == want


def test_prefill_bytes_are_read_plus_writes():
    """append(T) + flush into an empty cache: the fp16 input read once, the
    quantized part written as records, the rest written to the ring."""
    u, d, b, T, nq = 3, 128, 4, 300, 160
    assert bench.prefill_bytes(u, d, b, T, nq) == u * (T * 4 * d) + u * nq * 192 + u * (T - nq) * 4 * d


def _tree_with_profile(tmp_path, text):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "attend_w_pmc.txt").write_text(text)
    src = tmp_path / "kv_cache_compression_kivi_amd" / "csrc"
    src.mkdir(parents=True)
    for name in bench.ATTEND_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_compression_kivi_amd", "csrc", name), encoding="utf-8") as f:
            (src / name).write_text(f.read())
    return tmp_path


def test_traffic_reported_only_for_the_current_kernels(tmp_path, monkeypatch):
    h = bench._kernel_source_hash()
    root = _tree_with_profile(tmp_path, f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 1234\n"
                                        f"hbm_bytes_per_launch_b2: 1000\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench._kernel_source_hash() == h
    assert bench._traffic_from_profile("w") == 1234.0
    assert bench._traffic_from_profile("w", bits=2) == 1000.0
    assert bench._traffic_from_profile("w", bits=4) is None  # no such line
    assert bench._traffic_from_profile("other") is None  # no summary
    # a change to the code of an attention source (not its comments) voids the summary
    p = root / "kv_cache_compression_kivi_amd" / "csrc" / "split.hpp"
    p.write_text(p.read_text() + "\n// a comment\n")
    assert bench._traffic_from_profile("w") == 1234.0
    p.write_text(p.read_text() + "static const int kProbe = 1;\n")
    assert bench._traffic_from_profile("w") is None


def test_committed_summaries_parse():
    """Every committed counter summary carries a hash and the per-launch
    bytes bench.py reads."""
    names = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("attend_") and f.endswith("_pmc.txt")]
    assert names
    for f in names:
        text = open(os.path.join(ROOT, "profiles", f), encoding="utf-8").read()
        assert "kernel_source_sha256_16:" in text, f
        assert "hbm_bytes_per_launch:" in text, f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr
    assert r.stdout == ""


def test_side_workload_line(monkeypatch):
    """The default line's llama2_7b_layer entry: the child's JSON line (its
    last line starting with '{', after any progress output) reduced to the
    fields that sit beside the main workload's; a failed child gives an
    error entry, and the main line still prints."""
    import json

    child = {"metric": bench.METRIC, "value": 5250.3, "unit": "GB/s", "pct_of_peak": 65.63, "ms_per_step": 0.028,
             "steps": 200, "warmup": 5, "dtype": "f32", "config": {"workload": "llama2_7b_layer"},
             "quantize_append_tokens_per_s": 2.7e8, "quantize_append_gbs": 5613.5,
             "quantize_append_pct_of_peak": 70.2,
             "roofline": {"kernel": "attend_kernel", "achieved": 5295.3, "frac": 0.6619, "avg_launch_us": 28.4,
                          "algorithmic_bytes_per_launch": 150355968, "timed_launches": 200, "traffic": None,
                          "bound": "hbm", "peak": 8000.0}}
    calls = []

    def fake_run(cmd, stdout=None, text=None, timeout=None):
        calls.append(cmd)
        return subprocess.CompletedProcess(cmd, 0, stdout="progress\n" + json.dumps(child) + "\n")

    monkeypatch.setattr(subprocess, "run", fake_run)
    got = bench._side_workload("llama2_7b_layer", 7)
    assert calls and calls[0][-4:] == ["llama2_7b_layer", "--no-cpu-baseline", "--warmup", "7"]
    assert got["workload"] == "llama2_7b_layer" and got["pct_of_peak"] == 65.63
    assert got["roofline"]["frac"] == 0.6619 and "bound" not in got["roofline"]
    assert got["quantize_append_pct_of_peak"] == 70.2

    def failing_run(cmd, stdout=None, text=None, timeout=None):
        return subprocess.CompletedProcess(cmd, 1, stdout="")

    monkeypatch.setattr(subprocess, "run", failing_run)
    assert bench._side_workload("llama2_7b_layer", 7) == {"workload": "llama2_7b_layer", "error": "exit 1"}
