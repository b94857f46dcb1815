"""Summaries of rocprofv3 CSV output for the committed profile files.

    python -m hybrid_draft_tree_amd.rocprof_summary trace KERNEL_TRACE_CSV > profiles/<name>.md
    python -m hybrid_draft_tree_amd.rocprof_summary pmc FETCH_CSV WRITE_CSV > profiles/<name>.json

``trace`` groups a ``--kernel-trace`` CSV by kernel and launch shape
(workgroups x threads) and reports calls and begin-to-end durations.  ``pmc``
averages ``FETCH_SIZE`` / ``WRITE_SIZE`` (KiB per dispatch) over the verify
launches at the B=16, V=151936 shape (976 rows + 4 coordinator workgroups of
256 threads: 3 streaming wavefronts and a merge wavefront per row) and scales each counter by what it reads for the run's plain 1 GiB
device copy (``__amd_rocclr_copyBuffer``, 1 GiB read and 1 GiB written), giving
HBM bytes per launch.  Reads CSV text only.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# sources the verify kernel is compiled from; the hash marks which build the counters describe
KERNEL_SRCS = ["hybrid_draft_tree_amd/csrc/topk_kernels.hip", "hybrid_draft_tree_amd/csrc/device_utils.hpp",
               "hybrid_draft_tree_amd/csrc/launchers.hpp"]

B, T1, V, K = 16, 61, 151936, 8
VERIFY_WG = 256                        # 3 streaming wavefronts and a merge wavefront per row at the metric shape
VERIFY_GRID = (B * T1 + 4) * VERIFY_WG  # threads of the metric-shape verify launch (4 coordinator workgroups)
ALG_BYTES = B * T1 * V * 2 + B * T1 * K * 4
COPY_KIB = 1 << 20                      # 1 GiB

# bench.py's top-k launches: (kernel with its template flags, workgroups, threads) -> label.
# k_topk_mw<element traits, softmax statistics, acceptance, blocks per batch>: rows with a merge wavefront;
# k_topk_rows<element traits, softmax statistics, acceptance, non-temporal, split rows, blocks per batch>
VERIFY = "k_topk_mw<Bf16, false, true, 2>"
SHAPES = {
    (VERIFY, 980, 256): "verify, 976 rows (the timed step's launch)",
    ("k_topk_mw<Bf16, true, true, 4>", 980, 256): "verify with row statistics (coverage leg)",
    ("k_topk_rows<Bf16, false, true, true, true, 4>", 1096, 128): "TAIL verify, 272 rows in 4 slices",
    ("k_topk_mw<Bf16, false, true, 4>", 2049, 256): "ingest chunk, 2048 rows, update fused",
    ("k_topk_rows<Bf16, false, true, true, true, 4>", 245, 512):
        "61 rows in 4 slices: B=1, V=128256 verify; one request's rows at V=151936",
    ("k_topk_rows<Bf16, false, true, true, false, 4>", 245, 512): "B=4 decode verify, 244 rows x 151936, 8 waves each",
    ("k_topk_rows<F32, false, true, true, true, 2>", 245, 512): "B=1, V=32000 fp32 verify, 61 rows in 4 slices",
    ("k_build_tree", 16, 128): "build, B=16 (the timed step's launch)",
    ("k_build_tree", 4, 128): "build, B=4",
    ("k_build_tree", 1, 128): "build, B=1",
    ("k_stream_read", 976, 256): "read ceiling of the verify launch's rows (graft_stream_read)",
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SRCS:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """Kernel name without namespaces; the top-k kernels keep their template
    arguments (their instantiations differ in what they compute)."""
    t = re.search(r"(k_topk_rows|k_topk_mw)<(.*)>\(", name)
    if t:
        args = [a.strip().split("::")[-1].replace("Traits", "") for a in t.group(2).split(",")]
        return "%s<%s>" % (t.group(1), ", ".join(args))
    m = re.search(r"graft::\(anonymous namespace\)::(\w+)", name)
    return m.group(1) if m else name[:60]


def _median(xs):
    ys = sorted(xs)
    return ys[len(ys) // 2] if ys else float("nan")


def trace(path: str) -> str:
    groups = defaultdict(list)
    seq = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            key = (short_name(r["Kernel_Name"]), grid // max(wg, 1), wg)
            groups[key].append((t1 - t0) / 1000.0)
            seq.append((t0, t1, key))
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    out = ["| kernel | workgroups x threads | shape | calls | avg us | min us | max us |",
           "|---|---|---|---:|---:|---:|---:|"]
    for (name, nwg, wg), d in rows:
        out.append("| `%s` | %d x %d | %s | %d | %.2f | %.2f | %.2f |"
                   % (name, nwg, wg, SHAPES.get((name, nwg, wg), ""), len(d), sum(d) / len(d), min(d), max(d)))
    # the timed steps: a build launch followed by the metric-shape verify launch,
    # followed by the next step's build launch
    seq.sort()
    build, verify, g_bv, g_vb, step = [], [], [], [], []
    for i in range(len(seq) - 2):
        (b0, b1, kb), (v0, v1, kv), (n0, _, kn) = seq[i], seq[i + 1], seq[i + 2]
        if kb[0] == "k_build_tree" and kb[1] == B and kv == (VERIFY, 980, VERIFY_WG) and kn[0] == "k_build_tree":
            build.append((b1 - b0) / 1000.0)
            verify.append((v1 - v0) / 1000.0)
            g_bv.append((v0 - b1) / 1000.0)
            g_vb.append((n0 - v1) / 1000.0)
            step.append((n0 - b0) / 1000.0)
    if step:
        out.append("")
        out.append("Timed steps (a `k_build_tree` launch, the metric-shape verify launch, the next step's build; "
                   "%d steps, medians in us): build %.2f, gap build -> verify %.2f, verify %.2f, "
                   "gap verify -> next build %.2f, step (build start to next build start) %.2f."
                   % (len(step), _median(build), _median(g_bv), _median(verify), _median(g_vb), _median(step)))
    return "\n".join(out) + "\n"


def _counter(path: str):
    verify, copies = [], []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            val = float(r["Counter_Value"])
            if short_name(r["Kernel_Name"]) == VERIFY and int(r["Grid_Size"]) == VERIFY_GRID \
                    and int(r["Workgroup_Size"]) == VERIFY_WG:
                verify.append(val)
            elif "copyBuffer" in r["Kernel_Name"]:
                copies.append(val)
    if not verify or not copies:
        raise SystemExit("%s: no verify launches at the metric shape or no device copy" % path)
    return sum(verify) / len(verify), max(copies), len(verify)


def pmc(fetch_csv: str, write_csv: str, commands) -> dict:
    f_avg, f_copy, n = _counter(fetch_csv)
    w_avg, w_copy, _ = _counter(write_csv)
    fs, ws = COPY_KIB / f_copy, COPY_KIB / w_copy
    rd, wr = int(round(f_avg * fs * 1024)), int(round(w_avg * ws * 1024))
    return {
        "kernel": "k_topk_mw (graft_verify_update / graft_verify_accept), bf16, 976 rows x 151936",
        "kernel_source_sha256_16": kernel_source_hash(),
        "kernel_sources": KERNEL_SRCS,
        "dispatches": n,
        "fetch_kib_per_dispatch_raw": round(f_avg, 1),
        "write_kib_per_dispatch_raw": round(w_avg, 1),
        "copy_1GiB_fetch_kib_raw": round(f_copy, 1),
        "copy_1GiB_write_kib_raw": round(w_copy, 1),
        "fetch_scale": round(fs, 5),
        "write_scale": round(ws, 5),
        "hbm_read_bytes_per_launch": rd,
        "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": rd + wr,
        "alg_bytes_per_launch": ALG_BYTES,
        "traffic_over_alg": round((rd + wr) / ALG_BYTES, 4),
        "commands": list(commands),
        "note": "FETCH_SIZE/WRITE_SIZE averaged over the run's plain verify launches at the metric shape "
                "(k_topk_mw dispatches of 980 workgroups x 256 threads: 976 rows and 4 coordinators; the "
                "other shapes the run times are left out), scaled by what the same counter reads for the run's "
                "plain 1 GiB device copy (__amd_rocclr_copyBuffer, 1048576 KiB read and written)",
    }


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        sys.stdout.write(trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "pmc":
        cmds = [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- python3 bench.py "
            "--steps 40 --warmup 8 --kernel-iters 20 --no-cpu-baseline --copy-calib",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- python3 bench.py "
            "--steps 40 --warmup 8 --kernel-iters 20 --no-cpu-baseline --copy-calib",
            "python -m hybrid_draft_tree_amd.rocprof_summary pmc gpurun_out/pmc_fetch/fetch_counter_collection.csv "
            "gpurun_out/pmc_write/write_counter_collection.csv",
        ]
        print(json.dumps(pmc(argv[1], argv[2], cmds), indent=1))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
