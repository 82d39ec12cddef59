"""The benchmark's host-side logic, on the CPU: the refusal of more than one GPU,
the committed HBM-traffic figure and the source digest that gates it, and the
percentile summary. Nothing here touches a GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})],
                         ids=["gpus_flag", "world_size"])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_committed_traffic_matches_the_summary():
    path = os.path.join(ROOT, "profiles", "grouped_glu_gemm_skewed_zipf_counters.md")
    text = open(path).read()
    line = [x for x in text.splitlines() if x.startswith("hbm_bytes_per_launch:")][0]
    expect = float(line.split(":")[1])
    digest = [x for x in text.splitlines() if x.startswith("source_sha256_16:")][0].split()[1]
    got = bench.committed_traffic("grouped_glu_gemm", "skewed_zipf")
    if digest == bench.source_digest("grouped_glu_gemm"):
        assert got == expect
    else:
        assert got is None  # counters taken on other kernel source are not reported


def test_committed_traffic_is_dropped_when_the_source_changes(monkeypatch):
    monkeypatch.setattr(bench, "source_digest", lambda step: "0" * 16)
    assert bench.committed_traffic("grouped_glu_gemm", "skewed_zipf") is None
    assert bench.committed_traffic("grouped_glu_gemm", "no_such_workload") is None


def test_source_digest_covers_the_gemm_sources():
    names = bench.KERNEL_SOURCES["grouped_glu_gemm"]
    assert "grouped_gemm_core.hpp" in names and "grouped_gemm.hip" in names
    d = bench.source_digest("grouped_glu_gemm")
    assert len(d) == 16 and int(d, 16) >= 0


def test_percentiles():
    p = bench.percentiles([3.0, 1.0, 2.0, 4.0, 5.0])
    assert p["median"] == 3.0
    assert p["p10"] == pytest.approx(np.percentile([1, 2, 3, 4, 5], 10))
    assert p["p90"] == pytest.approx(np.percentile([1, 2, 3, 4, 5], 90))
