"""Host-side checks of bench.py: the refusal of several GPUs and the stored
HBM traffic figure of the lm_head GEMM (no GPU needed)."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

PROFILE = os.path.join(ROOT, "profiles", "lmhead_gemm_qwen38_27b_throughput_traffic.txt")


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8", "--steps", "1"]])
def test_several_gpus_refused_with_message(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_matches_its_profile():
    """The bytes and source hash in bench.py are the ones the committed
    counter summary records."""
    text = open(PROFILE).read()
    sha = re.search(r"lmhead_gemm\.hip SHA-256 at measurement: ([0-9a-f]{64})", text).group(1)
    assert sha == bench.GEMM_TRAFFIC["source_sha256"]
    m = re.search(r"lm_head GEMM [^\n]*?per launch: ([0-9.]+) GB read (?:\([^)]*\) )?\+ ([0-9.]+) GB "
                  r"written = ([0-9.]+) GB", text)
    rd, wr, tot = (float(x) for x in m.groups())
    assert abs(rd + wr - tot) < 0.002
    assert abs(bench.GEMM_TRAFFIC["bytes"] / 1e9 - tot) < 0.001
    # the per-kernel row gives the raw counters behind the GB figures
    row = re.search(r"^lmhead_gemm_w4\s+\d+\s+(\d+)\s+(\d+)\s+([0-9.]+)\s+([0-9.]+)$", text, re.M)
    fetch_kib, write_kib = int(row.group(1)), int(row.group(2))
    scale = re.search(r"FETCH_SIZE reads .* -> scale ([0-9.]+);", text).group(1)
    assert abs(fetch_kib * 1024 * float(scale) / 1e9 - rd) < 0.001
    assert abs(write_kib * 1024 / 1e9 - wr) < 0.001


def test_traffic_reported_only_for_its_source_and_workload():
    t = bench.GEMM_TRAFFIC
    if bench.gemm_source_sha256() == t["source_sha256"]:
        assert bench.measured_traffic(t["workload"]) == t["bytes"]
    else:
        assert bench.measured_traffic(t["workload"]) is None
    assert bench.measured_traffic("qwen3_8b") is None
