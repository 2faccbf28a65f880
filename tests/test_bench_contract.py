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


def test_acceptance_measures_of_a_table_job():
    """Round by round with table drafts: a draft passes while it equals the greedy token;
    accepted/examined counts the first failed draft of each round, accepted/drafted all k."""
    import bench
    ar = list(range(100, 140))
    k = 4
    m, acc = bench.accept_pattern(list(ar), ar, k, 20)           # every draft right
    assert m == [4, 4, 4, 4] and acc == {"accepted_over_examined": 1.0, "accepted_over_drafted": 1.0}
    m, acc = bench.accept_pattern([0] * 40, ar, k, 5)            # every draft wrong
    assert m == [0] * 5 and acc == {"accepted_over_examined": 0.0, "accepted_over_drafted": 0.0}
    table = list(ar)
    table[2] = -1                                                 # round 1 stops at its third draft
    m, acc = bench.accept_pattern(table, ar, k, 8)
    assert m == [2, 4]                                           # rounds at n0 = 0 and 3
    assert acc["accepted_over_examined"] == round(6 / (3 + 4), 4)
    assert acc["accepted_over_drafted"] == round(6 / 8, 4)


def test_protocol_alternates_order_and_times_every_leg():
    import bench
    calls = []

    def leg(name):
        def f(steps):
            calls.append((name, steps))
            return 0.5
        return f
    out = bench.protocol({"A": leg("A"), "B": leg("B"), "AR": leg("AR")}, steps=3, warmup=1, repeats=4, n_new=64)
    timed = [c for c in calls if c[1] == 3]
    assert [c[0] for c in timed] == ["A", "B", "AR", "AR", "B", "A", "A", "B", "AR", "AR", "B", "A"]
    assert out["B"] == [64 * 3 / 0.5] * 4
    assert bench.stats([3.0, 1.0, 2.0]) == {"median": 2.0, "min": 1.0, "max": 3.0, "n": 3}
