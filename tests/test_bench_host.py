"""Host-side logic of bench.py (no GPU): the one-GPU contract and the
digest gate on stored counter readings."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_stored_traffic_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    digest = bench.source_digest()
    monkeypatch.setattr(bench, "source_digest", lambda: digest)
    rec = {"w/a": {"bytes_per_launch": 123, "source_digest": digest},
           "w/b": {"bytes_per_launch": 456, "source_digest": "0000000000000000"}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("w/a") == 123
    assert bench.stored_traffic("w/b") is None  # taken on other sources
    assert bench.stored_traffic("w/c") is None  # absent


def test_source_digest_covers_every_kernel_source():
    csrc = os.path.join(ROOT, "paged_kv_cache_138_amd", "csrc")
    names = [f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))]
    assert "pa_attn_prefill.h" in names and "pa_inst_prefill_shared.hip" in names
    assert len(bench.source_digest()) == 16
