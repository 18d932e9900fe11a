"""Host-side checks of bench.py that need no GPU: the one-GPU refusal, and the
committed HBM-traffic counters being tied to the kernel sources they were
taken on (bench.py reports roofline.traffic only while the hashes agree)."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402

STAGES = ("x_quant", "gate_up_gemm", "swiglu_quant", "down_gemm")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("stage", STAGES)
def test_committed_traffic_matches_the_current_kernel_sources(stage):
    with open(os.path.join(ROOT, "profiles", f"traffic_{stage}.json")) as f:
        rec = json.load(f)
    assert rec["source_sha"] == bench.kernel_source_sha(), (
        "profiles/ holds counters of older kernel sources: re-take them")
    t = bench.load_traffic(stage, 1.0)
    assert t is not None and t > 0


def test_traffic_summary_names_the_same_sources():
    text = open(os.path.join(ROOT, "profiles", "hbm_traffic_c5.md")).read()
    assert bench.kernel_source_sha() in text
