"""Host-side pieces of the benchmark line (no GPU): the refusal of more than one
GPU, the algorithmic byte count the roofline divides, and the rule that the
measured traffic is reported only while the kernel sources it was taken on are
unchanged."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_verify_bytes_of_the_headline_forward():
    import bench
    from block_verify_amd.shapes import QWEN_1_5B as S
    # weights read once (every linear and the LM head, the norm gains; the
    # embedding table is gathered): 3,087,313,920 bytes for the 1.5B shape,
    # then per position 28 layers x 2 (K, V) x 2 kv heads x 128 dims x 2 bytes
    weights = 3_087_313_920
    kv = 28 * 2 * 2 * 128 * 2
    assert kv == 28_672
    T, M = 2048, 5
    expect = weights + kv * (T + M) + kv * M + 4 * S.vocab * M + 2 * S.hidden * M
    assert bench.verify_bytes(S, T, M) == expect == 3_149_374_976


def test_traffic_is_dropped_once_a_hashed_source_changes(tmp_path, monkeypatch):
    import bench
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source")
    import hashlib
    good = hashlib.sha256(b"kernel source").hexdigest()
    prof = tmp_path / "traffic.md"
    rel = os.path.relpath(src, ROOT)
    prof.write_text(f"    traffic_bytes_per_forward = 123456\n    sha256 {rel} {good}\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic() == 123456
    src.write_bytes(b"kernel source, changed")
    assert bench.measured_traffic() is None
    prof.unlink()
    assert bench.measured_traffic() is None
