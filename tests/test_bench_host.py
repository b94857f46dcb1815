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
    for flag in ("--steps", "--warmup", "--gpus", "--template-sweep", "--ablation", "--calibration", "--all-configs"):
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


def test_summary_tool_hash_matches_bench():
    from hybrid_draft_tree_amd import rocprof_summary as rs
    assert rs.kernel_source_hash() == bench.kernel_source_hash()
    assert [os.path.join(ROOT, p) for p in rs.KERNEL_SRCS] == bench.KERNEL_SRCS


def test_summary_tool_scales_counters_by_the_copy(tmp_path):
    """Two verify dispatches at the metric shape, one at another shape (left
    out) and the 1 GiB copy: bytes per launch = mean counter x (1 GiB / copy's
    counter)."""
    from hybrid_draft_tree_amd import rocprof_summary as rs
    hdr = "Correlation_Id,Dispatch_Id,Grid_Size,Kernel_Name,Workgroup_Size,Counter_Name,Counter_Value\n"

    def write(name, counter, verify_vals, copy_val):
        p = tmp_path / name
        lines = [hdr]
        for i, v in enumerate(verify_vals):
            lines.append('%d,%d,%d,"void graft::(anonymous namespace)::k_topk_mw<graft::(anonymous namespace)::Bf16Traits, false, true, 2>(graft::TopkArgs, graft::VerifyArgs)",%d,%s,%f\n'
                         % (i, i, rs.VERIFY_GRID, rs.VERIFY_WG, counter, v))
        lines.append('9,9,%d,"void graft::(anonymous namespace)::k_topk_rows<graft::(anonymous namespace)::Bf16Traits, false, true, true, false, 4>(graft::TopkArgs, graft::VerifyArgs)",256,%s,1.0\n'
                     % (1092 * 256, counter))
        lines.append('10,10,131072,"__amd_rocclr_copyBuffer",512,%s,%f\n' % (counter, copy_val))
        p.write_text("".join(lines))
        return str(p)

    f = write("f.csv", "FETCH_SIZE", [100.0, 300.0], float(1 << 19))   # reads half the copied bytes
    w = write("w.csv", "WRITE_SIZE", [10.0, 10.0], float(1 << 20))
    d = rs.pmc(f, w, ["cmd"])
    assert d["dispatches"] == 2
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["hbm_read_bytes_per_launch"] == 200 * 2 * 1024
    assert d["hbm_write_bytes_per_launch"] == 10 * 1024
    assert d["alg_bytes_per_launch"] == 976 * 151936 * 2 + 976 * 8 * 4


def test_summary_tool_step_breakdown(tmp_path):
    """Build / verify / build triples in a kernel trace give the per-step
    durations and the two inter-launch gaps (medians)."""
    from hybrid_draft_tree_amd import rocprof_summary as rs
    hdr = ("Kernel_Name,Workgroup_Size_X,Workgroup_Size_Y,Workgroup_Size_Z,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,"
           "Start_Timestamp,End_Timestamp\n")
    build = '"void graft::(anonymous namespace)::k_build_tree(graft::BuildKernelArgs)",128,1,1,2048,1,1'
    verify = ('"void graft::(anonymous namespace)::k_topk_mw<graft::(anonymous namespace)::Bf16Traits, false, '
              'true, 2>(graft::TopkArgs, graft::VerifyArgs)",256,1,1,%d,1,1' % rs.VERIFY_GRID)
    lines, t = [hdr], 1000000
    for _ in range(5):       # build 5 us, gap 0.5, verify 48 us, gap 0.7
        lines.append("%s,%d,%d\n" % (build, t, t + 5000))
        lines.append("%s,%d,%d\n" % (verify, t + 5500, t + 53500))
        t += 54200
    lines.append("%s,%d,%d\n" % (build, t, t + 5000))
    p = tmp_path / "trace.csv"
    p.write_text("".join(lines))
    text = rs.trace(str(p))
    assert "5 steps" in text
    assert "build 5.00, gap build -> verify 0.50, verify 48.00, gap verify -> next build 0.70, " \
           "step (build start to next build start) 54.20" in text
