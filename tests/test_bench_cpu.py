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
