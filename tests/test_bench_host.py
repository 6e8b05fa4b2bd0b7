"""Host-side logic of bench.py (CPU): flop and byte accounting, the roofline
traffic lookup in a counter summary, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_io_aware_58_amd import inputs  # noqa: E402


def test_flops_follow_the_contraction_count():
    w = inputs.Workload("x", 1, 2, 3, 100, 64, "bf16", False, True)
    f, b = bench.flops(w)
    assert f == 4.0 * 2 * 3 * 100 * 100 * 64          # S = QK^T and O = PV
    assert b == 10.0 * 2 * 3 * 100 * 100 * 64         # dV, dP, dQ, dK, and S again
    wc = inputs.Workload("x", 1, 2, 3, 100, 64, "bf16", True, True)
    assert bench.flops(wc) == (f / 2, b / 2)
    wf = inputs.Workload("x", 1, 2, 3, 100, 64, "bf16", False, False)
    assert bench.flops(wf)[1] == 0.0


def test_kernel_work_per_launch():
    w = inputs.WORKLOADS["c5"]
    unit = 2.0 * w.B * w.H * w.N * w.N * w.D / 2      # one N^2 D contraction, causal
    alg = bench.kernel_algorithmic(w)
    assert alg["fwd"] == ("mfma", 2 * unit)
    assert alg["bwd_dkdv"] == ("mfma", 4 * unit)
    assert alg["bwd_dq"] == ("mfma", 1 * unit)
    assert alg["bwd_dkdv_dq"] == ("mfma", 5 * unit)
    rows = w.B * w.H * w.N
    assert alg["bwd_delta"] == ("hbm", 2.0 * rows * w.D * 2 + 4.0 * rows)
    assert alg["merge"] == ("hbm", 3.0 * rows * (w.D * 2 + 4))
    # the step's credited work is the forward plus the backward contractions
    f, b = bench.flops(w)
    assert alg["fwd"][1] + alg["bwd_dkdv"][1] + alg["bwd_dq"][1] == f + b


def test_profiled_traffic_reads_matching_rows(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "wl.md").write_text(
        "| id | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read bytes | scaled write bytes | sha |\n"
        "|---|---|---|---|---|---|---|\n"
        "| bwd_dkdv | `k` | 10 | 2 | 2.5e+09 | 1.5e+08 | aaaa |\n"
        "| fwd | `k` | 10 | 2 | 1e+09 | 1e+08 | bbbb |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda k: {"bwd_dkdv": "aaaa", "fwd": "zzzz"}[k])
    assert bench.profiled_traffic("wl", "bwd_dkdv") == pytest.approx(2.65e9)
    assert bench.profiled_traffic("wl", "fwd") is None        # source changed since
    assert bench.profiled_traffic("missing", "fwd") is None   # no summary


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""
