"""Host-side checks of bench.py's contract (no GPU): one GPU only, the
counter summary it reads, and the committed profile summaries."""
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
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--template-sweep", "--ablation", "--calibration"):
        assert flag in r.stdout


def test_counter_summary_fields_and_traffic_gate():
    with open(bench.PMC_FILE) as f:
        d = json.load(f)
    for key in ("kernel_source_sha256_16", "hbm_bytes_per_launch", "alg_bytes_per_launch", "fetch_scale",
                "write_scale", "commands"):
        assert key in d, key
    assert d["alg_bytes_per_launch"] == 976 * 151936 * 2 + 976 * 8 * 4
    assert 0.99 < d["hbm_bytes_per_launch"] / d["alg_bytes_per_launch"] < 1.05
    traffic, note = bench.load_traffic(d["alg_bytes_per_launch"])
    if d["kernel_source_sha256_16"] == bench.kernel_source_hash():
        assert traffic == d["hbm_bytes_per_launch"]
    else:
        assert traffic is None and "changed" in note


@pytest.mark.parametrize("name", ["graft_step_b16_v151936_kernel_trace.md", "topk_rows_b16_v151936_pmc.json"])
def test_profile_summaries_are_committed_and_small(name):
    p = os.path.join(ROOT, "profiles", name)
    assert os.path.exists(p) and os.path.getsize(p) < 16384
    text = open(p).read()
    assert "rocprofv3" in text
