"""CPU checks of bench.py's contract pieces that need no GPU: the one-GPU guard and the
lookup of recorded HBM traffic, which must be reported only while the kernel's code is the
code the counters were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_recorded_traffic_is_reported_only_for_unchanged_code():
    doc = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert doc["calibration"]["fetch_factor"] > 0 and doc["calibration"]["write_factor"] > 0
    for e in doc["kernels"]:
        current = bench.code_digest(e["sources"]) == e["code_sha256"]
        assert bench.measured_traffic(e["kernel"]) == (e["traffic_bytes"] if current else None), e["kernel"]
        # the scaled counters add up to the reported traffic
        assert abs(e["fetch_bytes"] + e["write_bytes"] - e["traffic_bytes"]) <= 1
    assert bench.measured_traffic("no such kernel") is None


def test_digest_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    csrc = tmp_path / "bit_quantized_gemm_bitlinear_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("int f() {\n  return 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.code_digest(["a.hip"])
    (csrc / "a.hip").write_text("/* a block\n   comment */\nint f() {\n\n  return 1;  // the value one\n}\n")
    assert bench.code_digest(["a.hip"]) == d0
    (csrc / "a.hip").write_text("int f() {\n  return 2;\n}\n")
    assert bench.code_digest(["a.hip"]) != d0


@pytest.mark.parametrize("K,abits,xb,want", [(16384, 4, 2, 40964), (16384, 8, 2, 49156), (256, 4, 4, 1156)])
def test_activation_bytes_per_token(K, abits, xb, want):
    assert bench.act_bytes_per_token(K, abits, xb) == want
