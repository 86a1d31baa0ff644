"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte counts the roofline divides by, and the rule that a traffic figure is
only reported for the kernel source it was measured on."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_per_unit_bytes(bench):
    # quantize+scatter at head_dim 128: 2 x (256 B bf16 read + 128 B codes +
    # 4 B scale) per (token, KV head), plus the token's 8-byte slot id
    assert bench.quant_bytes(1, 1, 128) == 776 + 8
    assert bench.quant_bytes(4096, 8, 128) == 4096 * 8 * 776 + 8 * 4096
    # decode at head_dim 128: 264 B of codes and scales per (token, KV head)
    total, kv = bench.decode_bytes([1], 1, 128, 1, 1, 1, 16)
    assert kv == 264
    assert total == 264 + 4 + 2 * 128 * 2        # one table entry, q and out rows


def test_decode_bytes_count_table_entries_per_request(bench):
    lens = [1, 16, 17, 1000]
    B, R, Hq, Hkv, D, bs = 4, 2, 8, 2, 64, 16
    total, kv = bench.decode_bytes(lens, Hkv, D, B, R, Hq, bs)
    assert kv == sum(lens) * Hkv * 2 * (D + 4)
    entries = 1 + 1 + 2 + 63
    assert total == kv + entries * 4 + 2 * B * R * Hq * D * 2


def test_traffic_only_for_the_measured_source(bench, tmp_path, monkeypatch):
    good = {"kernel_source_hash": bench.kernel_source_hash(), "bytes_per_launch": 12345,
            "pool_layout": bench.POOL}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_entry(1) == 12345
    f.write_text(json.dumps(dict(good, kernel_source_hash="0" * 16)))
    assert bench.traffic_entry(1) is None
    other = "slot" if bench.POOL == "head" else "head"
    f.write_text(json.dumps(dict(good, pool_layout=other)))      # another pool layout
    assert bench.traffic_entry(1) is None
    f.write_text("not json")
    assert bench.traffic_entry(1) is None


def test_traffic_only_for_the_measured_scale_layout(bench, tmp_path, monkeypatch):
    """Counters taken on head-major scale planes (the record names none or
    "head") do not apply to a run on K/V-interleaved planes, and back."""
    good = {"kernel_source_hash": bench.kernel_source_hash(), "bytes_per_launch": 777,
            "pool_layout": bench.POOL}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    monkeypatch.setattr(bench, "SCALES", "head")
    assert bench.traffic_entry(1) == 777
    monkeypatch.setattr(bench, "SCALES", "interleaved")
    assert bench.traffic_entry(1) is None
    f.write_text(json.dumps(dict(good, scale_layout="interleaved")))
    assert bench.traffic_entry(1) == 777
    monkeypatch.setattr(bench, "SCALES", "head")
    assert bench.traffic_entry(1) is None
