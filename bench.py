#!/usr/bin/env python3
"""Graft per-step hot path benchmark on one MI355X.

Workload: the batched static-slot step -- B=16 requests, V=151936, 60 candidate
slots + the root (61 verified rows per request), k=8, bf16 target logits
[16, 61, V] (296.6 MB per step), in-place layout.  One step = prune-select ->
retrieval expansion -> flatten/mask -> row-wise top-k + acceptance walk ->
matrix update, all through the C ABI; the target forward is outside the path,
so each step reads one buffer of a rotating pool of pre-generated logits
(pool >= 4 x 296.6 MB, larger than the 256 MB Infinity Cache).

The pool is filled from a real seeded trajectory (warm-up first, table warmed
up); during timing the matrix and roots keep evolving, so accepted lengths
differ from the pool's own trajectory but every byte is still read.

Timed region: exactly `--warmup` untimed steps, then `--repeats` windows of
exactly `--steps` steps each, every window one HIP-graph replay (one graph per
window, captured beforehand), each bracketed by HIP events
on the replay stream; the first event is recorded behind the queued warm-up,
the host synchronises before the warm-up and after the last window.  The value
is the median window.
The dominant kernel (graft_verify_update's single launch: row-wise top-k,
acceptance walk and matrix update) is then timed on its own with HIP events on
the stream it is launched on: one pair around back-to-back launches (the
roofline figure) and one pair around each launch (reported beside it).  The CPU
oracle is timed on host copies of the same inputs.

    python bench.py [--steps K] [--warmup W] [--repeats R] [--pool P] [--no-cpu-baseline] [--no-shapes]

A second mode, ``--template-sweep``, measures the retrieval template instead of
speed: mean accepted length per step on workloads 2 and 4 for rank-chain and
branching templates over a grid of depths and widths (one JSON line per point).
A third, ``--ablation``, compares the pruning/retrieval variants of the
write-up's ablations (no retrieval, fixed splits, a dense tree, per-node
thresholds) with the adaptive default on workloads 2, 3 and 4.  A fourth,
``--calibration``, sets the thresholds from warm-up quantiles and moves them
between workloads.  A fifth, ``--all-configs``, times the full step on each
of the five workloads at its own shape (one JSON line each).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Graft steps/sec at batch 16, V=151936, 60 slots; achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "topk_rows_b16_v151936_pmc.json")
# sources the dominant kernel is compiled from (the counter summary is valid for them only)
KERNEL_SRCS = [os.path.join(ROOT, "hybrid_draft_tree_amd", "csrc", f)
               for f in ("topk_kernels.hip", "device_utils.hpp", "launchers.hpp")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--repeats", type=int, default=5, help="timed windows of --steps steps (median reported)")
    ap.add_argument("--shape-steps", type=int, default=400,
                    help="steps per window of the full-step diagnostic at the other workloads")
    ap.add_argument("--no-shapes", action="store_true", help="skip the full-step diagnostic at other workloads")
    ap.add_argument("--pool", type=int, default=4)
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--template-sweep", action="store_true",
                    help="accept length vs retrieval template on workloads 2 and 4 (no timing)")
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--sweep-depths", default="2,4,6,8,10,12")
    ap.add_argument("--sweep-widths", default="4,6,8")
    ap.add_argument("--sweep-configs", default="2,4")
    ap.add_argument("--ablation", action="store_true",
                    help="accept length of the pruning/retrieval variants (no timing)")
    ap.add_argument("--ablation-configs", default="2,3,4")
    ap.add_argument("--all-configs", action="store_true",
                    help="time the full step (build + verify/update, HIP graph) on each workload's own shape")
    ap.add_argument("--config-list", default="1,2,3,4,5")
    ap.add_argument("--calibration", action="store_true",
                    help="calibrated thresholds vs quantile level, and their transfer across workloads")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class _Adapter:
    """Drives the HIP pipeline through synth.runner (input generation only)."""

    def __init__(self, pipe, torch):
        from synth.device import DeviceRows
        self.p = pipe
        self.torch = torch
        self.DeviceRows = DeviceRows
        self.rows = None

    def set_roots(self, roots, base_pos):
        self.p.set_roots(roots, base_pos)

    def get_roots(self):
        return self.p.roots.cpu().numpy()

    def build(self, draft):
        return {k: v.cpu().numpy() for k, v in self.p.build(draft).items()}

    def materialize(self, pool, desc):
        if self.rows is None:
            self.rows = self.DeviceRows(pool, self.p.device)
        return self.rows.materialize(desc)

    def verify_update(self, rows):
        return {k: v.cpu().numpy() for k, v in self.p.verify_update(rows).items()}

    def ingest_chunk(self, row_tok, rows):
        return self.p.ingest_chunk(row_tok, rows)

    def begin_calibration(self):
        self.p.begin_calibration()

    def end_calibration(self, q):
        self.samples = self.p.calibration_samples().cpu().numpy()
        return self.p.end_calibration(q)


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(bytes_alg):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since counters were taken"
    return d.get("hbm_bytes_per_launch"), d.get("note", "")


def _accept_run(cfg, steps, dev, warmup=None, log_thr=None):
    """One fresh pipeline through the workload's warm-up and `steps` steps:
    accepted tokens per request-step, the share of request-steps that retrieved
    anything, whose accepted path reaches a retrieved row, and the coverage gain.
    With cfg.calib_q the thresholds are calibrated over the warm-up; log_thr
    (fp32 ln tau) replaces them after the warm-up instead."""
    import numpy as np
    import torch

    from hybrid_draft_tree_amd import _lib as L
    from hybrid_draft_tree_amd.driver import GraftPipeline
    from synth import generators as G
    from synth import runner as R

    pipe = GraftPipeline.from_config(cfg, want_coverage=True, device=dev)
    ad = _Adapter(pipe, torch)
    wl = R.Workload(cfg)
    R.start(ad, wl)
    if warmup is None:
        warmup = cfg.warmup_steps if cfg.cfg_id != 4 else 0
    thr = R.warm_up(ad, wl, warmup)
    if log_thr is not None:
        for i in range(3):
            pipe.cfg.log_thr[i] = float(log_thr[i])
    acc = via_ret = n = with_ret = kept = 0
    stages = np.zeros(5, np.int64)
    gain = 0.0
    for s in range(steps):
        flat, res = R.step(ad, wl, s)
        alen = np.asarray(res["accept_len"])
        aidx = np.asarray(res["accept_idx"])
        src = np.asarray(flat["row_src"])
        for b in range(cfg.B):
            via_ret += int((src[b, aidx[b, :alen[b]]] == L.ROW_RETRIEVED).any())
        acc += int(alen.sum())
        with_ret += int((np.asarray(flat["n_ret"]) > 0).sum())
        kept += int(np.asarray(flat["n_keep"]).sum())
        stages += np.bincount(np.asarray(flat["stage"]), minlength=5)[:5]
        gain += float(np.asarray(res["coverage"]).sum())
        n += cfg.B
    out = {"template_nodes": int(pipe.tpl.size) if pipe.tpl is not None else 0, "steps": steps, "requests": cfg.B,
           "mean_accept_len": round(acc / n, 4), "tokens_per_step": round(acc / n + 1, 4),
           "mean_draft_kept": round(kept / n, 2), "steps_with_retrieval": round(with_ret / n, 4),
           "accepted_via_retrieval": round(via_ret / n, 4), "mean_coverage_gain": round(gain / n, 5),
           "stage_share": [round(float(x) / n, 4) for x in stages[:4]],
           "log_thr": [float(pipe.cfg.log_thr[i]) for i in range(3)]}
    if thr is not None:
        out["calibrated_tau"] = [round(float(np.exp(np.float64(t))), 5) for t in thr]
        # where the workload's fixed thresholds sit in the warm-up statistics
        smp = ad.samples
        lt = np.log(np.asarray(cfg.tau, np.float64)).astype(np.float32)
        out["fixed_tau_quantile"] = [round(float((smp[:, i][~np.isnan(smp[:, i])] < lt[i]).mean()), 4)
                                     for i in range(3)]
    del pipe, ad
    torch.cuda.empty_cache()
    return out


def ablation(args):
    """Accept length of the variants behind the write-up's ablations, all with
    the same 60-slot budget: the adaptive default, no retrieval (freed slots
    stay empty), fixed draft/retrieval splits, the dense draft tree (never
    prune, no retrieval) and the per-node static-slot threshold."""
    import torch

    from synth import WORKLOADS

    assert torch.cuda.is_available(), "the ablation runs on the GPU"
    dev = torch.device("cuda", 0)
    inf = float("inf")
    variants = [("graft (adaptive)", {}), ("no retrieval", {"tpl_kind": "none"}),
                ("fixed 8/52", {"tau": (inf, 0.0, 0.0)}), ("fixed 24/36", {"tau": (0.0, inf, 0.0)}),
                ("fixed 40/20", {"tau": (0.0, 0.0, inf)}), ("dense (no prune)", {"tau": (0.0, 0.0, 0.0)})]
    variants += [("per-node tau=%g" % t, {"node_tau": t}) for t in (0.05, 0.1, 0.2, 0.3)]
    for cfg_id in [int(x) for x in args.ablation_configs.split(",")]:
        base = WORKLOADS[cfg_id]
        for name, kw in variants:
            t0 = time.time()
            rec = {"ablation": name, "workload": base.name}
            rec.update(_accept_run(base.scaled(**kw), args.sweep_steps, dev))
            rec["seconds"] = round(time.time() - t0, 1)
            print(json.dumps(rec), flush=True)


def calibration(args):
    """Thresholds calibrated over 5 warm-up steps at quantile levels q, the
    accept length they give, where the fixed thresholds (0.3, 0.2, 0.1) sit in
    the same warm-up statistics, and transfer: the thresholds of one workload
    applied to another (the write-up's cross-task table).  No timing."""
    import math

    import numpy as np
    import torch

    from synth import WORKLOADS

    assert torch.cuda.is_available(), "the calibration study runs on the GPU"
    dev = torch.device("cuda", 0)
    ids = [int(x) for x in args.ablation_configs.split(",")]
    levels = [(0.1, 0.1, 0.1), (0.25, 0.25, 0.25), (0.5, 0.5, 0.5), (0.75, 0.75, 0.75),
              (0.1, 0.4, 0.9), (0.1, 0.5, 0.97)]
    own = {}
    for cfg_id in ids:
        base = WORKLOADS[cfg_id]
        fixed = [float(np.float32(math.log(t))) for t in base.tau]
        rec = {"calibration": "fixed tau %s" % (base.tau,), "workload": base.name}
        # calibrate only to record the statistics; the fixed thresholds are kept
        rec.update(_accept_run(base.scaled(calib_q=(0.5, 0.5, 0.5)), args.sweep_steps, dev,
                               warmup=base.warmup_steps, log_thr=fixed))
        rec.pop("calibrated_tau", None)
        print(json.dumps(rec), flush=True)
        for q in levels:
            rec = {"calibration": "q=%s" % (q,), "workload": base.name}
            rec.update(_accept_run(base.scaled(calib_q=q), args.sweep_steps, dev, warmup=base.warmup_steps))
            own[(cfg_id, q)] = rec["log_thr"]
            print(json.dumps(rec), flush=True)
    for q in [levels[2], levels[5]]:
        for src in ids:
            for dst in ids:
                if src == dst:
                    continue
                rec = {"calibration": "q=%s transferred" % (q,), "from": WORKLOADS[src].name,
                       "workload": WORKLOADS[dst].name}
                rec.update(_accept_run(WORKLOADS[dst], args.sweep_steps, dev, warmup=WORKLOADS[dst].warmup_steps,
                                       log_thr=own[(src, q)]))
                print(json.dumps(rec), flush=True)


def template_sweep(args):
    """Accepted tokens per step vs the retrieval template (no timing).  For every
    workload, template family, depth and width: a fresh pipeline (matrix reset,
    prompt re-ingested for workload 4), the workload's warm-up, then
    --sweep-steps steps; reports the mean accepted length, the share of steps
    whose accepted path reaches a retrieved row, and the mean coverage gain."""
    import torch

    from synth import WORKLOADS

    assert torch.cuda.is_available(), "the template sweep runs on the GPU"
    dev = torch.device("cuda", 0)
    families = [("chain", (1, 1)), ("branching", (1, 1)), ("branching", (2, 1))]
    depths = [int(x) for x in args.sweep_depths.split(",")]
    widths = [int(x) for x in args.sweep_widths.split(",")]
    for cfg_id in [int(x) for x in args.sweep_configs.split(",")]:
        base = WORKLOADS[cfg_id]
        for kind, beta in families:
            for D in depths:
                for W in widths:
                    t0 = time.time()
                    cfg = base.scaled(tpl_kind=kind, tpl_beta=beta, tpl_depth=D, tpl_width=W)
                    rec = {"sweep": "template", "workload": cfg.name, "template": kind,
                           "beta": list(beta) if kind == "branching" else None, "depth": D, "width": W}
                    rec.update(_accept_run(cfg, args.sweep_steps, dev))
                    rec["seconds"] = round(time.time() - t0, 1)
                    print(json.dumps(rec), flush=True)


def setup_pool(cfg, P, dev, torch):
    """A fresh pipeline through the workload's start (prompt ingest for workload
    4) and warm-up, then P steps of its seeded trajectory; each step's draft is
    kept on the device and its logits in a pool buffer, so a replayed step does
    the whole build + verify/update work on real inputs.  Returns the pipeline,
    the pool (drafts, logits) and the accepted tokens of each pool step."""
    from hybrid_draft_tree_amd.driver import GraftPipeline
    from synth import generators as G
    from synth import runner as R

    pipe = GraftPipeline.from_config(cfg, device=dev)
    ad = _Adapter(pipe, torch)
    wl = R.Workload(cfg)
    R.start(ad, wl)
    for s_ in range(cfg.warmup_steps if cfg.cfg_id != 4 else 0):
        R.step(ad, wl, s_, G.WARMUP_STREAM_OFFSET)
    n_rows = cfg.B * cfg.rows_per_request
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    pool_logits, pool_drafts, acc = [], [], []
    for p in range(P):
        roots = ad.get_roots()
        draft = wl.draft(p, roots)
        flat = ad.build(draft)
        desc = wl.logit_desc(p, flat)
        buf = torch.empty(n_rows, cfg.V, dtype=tdt, device=dev)
        if ad.rows is None:
            ad.rows = ad.DeviceRows(wl.pool, dev)
        ad.rows.materialize(desc, out=buf)
        res = ad.verify_update(buf)
        wl.commit(roots, flat, res)
        acc.append(int(res["accept_len"].sum()))
        bufs = pipe.draft_buffers()
        if cfg.mode == "tree":
            bufs["parent"].copy_(torch.as_tensor(draft["parent"]))
            bufs["layer"].copy_(torch.as_tensor(draft["layer"]))
            bufs["score"].copy_(torch.as_tensor(draft["logp"]))
        else:
            bufs["score"].copy_(torch.as_tensor(draft["conf"]))
        bufs["tok"].copy_(torch.as_tensor(draft["tok"]))
        pool_logits.append(buf)
        pool_drafts.append(bufs)
    torch.cuda.synchronize()
    return pipe, pool_drafts, pool_logits, acc


class StepReplayer:
    """Enqueues steps i = s .. s+n-1 of a rotating pool (step i uses pool entry
    i mod P).  Untimed runs replay a whole pass over the pool as one HIP graph
    where the rotation allows and every other step as its own one-step graph;
    each timed window of exactly K steps is one HIP graph of its own, so a
    window pays one graph launch whatever K is and the rotation never repeats
    a buffer back to back."""

    def __init__(self, pipe, pool_drafts, pool_logits, torch, use_graph=True):
        self.P = len(pool_logits)
        self.pipe, self.drafts, self.logits = pipe, pool_drafts, pool_logits
        self.use_graph = use_graph
        self.torch = torch
        self.g_win = {}
        if use_graph:
            self._pass()            # warm the launch path before capture
            torch.cuda.synchronize()
            self.g_pool = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.g_pool):
                self._pass()
            self.g_one = []
            for p in range(self.P):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self._step(p)
                self.g_one.append(g)
            torch.cuda.synchronize()

    def _step(self, p):
        self.pipe.build_device(self.drafts[p])
        self.pipe.verify_update_device(self.logits[p])

    def _pass(self):
        for p in range(self.P):
            self._step(p)

    def prepare_window(self, r, s, n):
        """Capture the graph of window r: steps s .. s+n-1.  Each window has a
        graph of its own, so consecutive windows never replay one graph twice
        in a row (a replay of a graph waits for that graph's previous replay
        to finish, which would leave the device idle while the host launches)."""
        if self.use_graph and r not in self.g_win:
            g = self.torch.cuda.CUDAGraph()
            with self.torch.cuda.graph(g):
                for i in range(s, s + n):
                    self._step(i % self.P)
            self.torch.cuda.synchronize()
            g.replay()              # the first launch of a graph also uploads it
            self.torch.cuda.synchronize()
            self.g_win[r] = g

    def window(self, r, s, n):
        """Enqueue window r (steps s .. s+n-1) as one graph replay."""
        if self.use_graph:
            self.g_win[r].replay()
        else:
            for i in range(s, s + n):
                self._step(i % self.P)
        return s + n

    def run(self, s, n):
        while n > 0:
            p = s % self.P
            if p == 0 and n >= self.P:
                if self.use_graph:
                    self.g_pool.replay()
                else:
                    self._pass()
                s, n = s + self.P, n - self.P
            else:
                if self.use_graph:
                    self.g_one[p].replay()
                else:
                    self._step(p)
                s, n = s + 1, n - 1
        return s


class WindowEvents:
    """Timing events for the timed windows, made with the HIP runtime torch has
    loaded (one runtime per process) and recorded with a device-scope release
    (hipEventReleaseToDevice, which HIP documents for timing the commands between
    events): torch's events release at system scope, which at every window
    boundary also writes back and invalidates the caches, work that is no part of
    a step.  The marker still waits for the window's last kernel before it takes
    its timestamp.  Falls back to torch's events if the runtime cannot be found."""

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, torch):
        import ctypes as C
        self.torch, self.C, self.H = torch, C, None
        try:
            path = next((l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l), None)
            if path:
                H = C.CDLL(path)
                H.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
                H.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
                H.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
                H.hipEventDestroy.argtypes = [C.c_void_p]
                self.H = H
        except OSError:
            self.H = None
        self.kind = "hip_release_to_device" if self.H is not None else "torch"

    def make(self, n):
        if self.H is None:
            return [self.torch.cuda.Event(enable_timing=True) for _ in range(n)]
        evs = []
        for _ in range(n):
            e = self.C.c_void_p()
            if self.H.hipEventCreateWithFlags(self.C.byref(e), self.RELEASE_TO_DEVICE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            evs.append(e)
        return evs

    def record(self, e, stream):
        if self.H is None:
            e.record(stream)
        elif self.H.hipEventRecord(e, self.C.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        if self.H is None:
            return a.elapsed_time(b)
        f = self.C.c_float()
        if self.H.hipEventElapsedTime(self.C.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def free(self, evs):
        if self.H is not None:
            for e in evs:
                self.H.hipEventDestroy(e)


def timed_steps(rep, K, W, repeats, torch):
    """Capture the window graphs, synchronise, enqueue exactly W untimed
    warm-up steps, then `repeats` windows of exactly K steps (one graph replay
    each), each bracketed by HIP events on the replay stream; the first event
    is recorded behind the queued warm-up, so no window starts on an idle
    device, and the host synchronises once all are done.  Returns the
    per-window milliseconds and the wall-clock seconds."""
    for r in range(repeats):
        rep.prepare_window(r, W + r * K, K)
    stream = torch.cuda.current_stream()
    we = WindowEvents(torch)
    evs = we.make(repeats + 1)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    s = rep.run(0, W)
    we.record(evs[0], stream)
    for r in range(repeats):
        s = rep.window(r, s, K)
        we.record(evs[r + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = [we.elapsed_ms(evs[r], evs[r + 1]) for r in range(repeats)]
    we.free(evs)
    timed_steps.events = we.kind
    return ms, wall


def _median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def time_workload(cid, steps, warmup, P, dev, torch, repeats=3):
    """Full step (build + verify/update) of workload `cid` at its own shape:
    a pool of P steps of its trajectory, replayed exactly `steps` steps per
    window, median over `repeats` windows."""
    from synth import WORKLOADS

    cfg = WORKLOADS[cid]
    t0 = time.time()
    pipe, drafts, logits, _ = setup_pool(cfg, P, dev, torch)
    rep = StepReplayer(pipe, drafts, logits, torch)
    ms, _ = timed_steps(rep, steps, warmup, repeats, torch)
    us = _median(ms) * 1e3 / steps
    n_rows = cfg.B * cfg.rows_per_request
    lb = n_rows * cfg.V * cfg.elem_bytes
    step_bytes = lb + n_rows * cfg.k * 4
    rec = {"workload": cfg.name, "config": cid, "batch": cfg.B, "vocab": cfg.V,
           "rows_per_request": cfg.rows_per_request, "verified_rows": n_rows, "dtype": cfg.dtype,
           "layout": cfg.layout, "steps": steps, "repeats": repeats, "us_per_step": round(us, 3),
           "us_per_step_min": round(min(ms) * 1e3 / steps, 3), "us_per_step_max": round(max(ms) * 1e3 / steps, 3),
           "steps_per_s": round(1e6 / us, 1), "logits_bytes_per_step": lb,
           "step_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
           "step_frac_of_peak": round(step_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
           "setup_s": round(time.time() - t0, 1)}
    del rep, pipe, drafts, logits
    torch.cuda.empty_cache()
    return rec


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, pipe, pool_drafts, pool_logits, step_bytes, seconds, torch):
    """The CPU oracle as it stands, on host copies of the pool's inputs (drafts,
    logits, the matrix and roots as the GPU left them): full steps (prune,
    retrieve, flatten, top-k, accept, update) for about seconds/2 on one thread,
    then on all the threads OpenMP is given.  The headline value is the all-thread
    rate; cores = the threads it used."""
    import numpy as np

    from oracle import oracle as O
    from oracle.driver import OracleGraft

    P = len(pool_logits)
    host_logits = [b.view(torch.int16).cpu().numpy().view(np.uint16) for b in pool_logits]
    host_drafts = [{"parent": d["parent"].cpu().numpy(), "layer": d["layer"].cpu().numpy(),
                    "logp": d["score"].cpu().numpy(), "tok": d["tok"].cpu().numpy()} for d in pool_drafts]
    table = pipe.table.cpu().numpy()
    roots, base = pipe.roots.cpu().numpy(), pipe.base_pos.cpu().numpy()
    all_threads = O.num_threads()
    runs = {}
    for threads in (1, all_threads):
        O.set_threads(threads)
        og = OracleGraft(cfg)
        og.table = table.copy()
        og.set_roots(roots, base)
        n = 0
        c0 = time.perf_counter()
        while True:
            p = n % P
            og.build(host_drafts[p])
            og.verify_update(host_logits[p])
            n += 1
            el = time.perf_counter() - c0
            if el >= seconds / 2 or n >= 1000:
                break
        runs[threads] = (n, el)
        log("cpu oracle: %d steps in %.1f s with %d thread(s)" % (n, el, threads))
    O.set_threads(all_threads)
    n, el = runs[all_threads]
    n1, el1 = runs[1]
    return {"value": round(n / el, 3), "unit": "steps/s", "cores": all_threads, "kind": "oracle",
            "sample": "%d full oracle steps (B=16, V=151936, 61 rows/request) on host copies of the same pool "
                      "inputs in %.1f s on %d threads; %d steps in %.1f s on 1 thread" % (n, el, all_threads, n1, el1),
            "ms_per_step": round(el / n * 1e3, 2), "GBps": round(step_bytes * n / el / 1e9, 2),
            "one_thread": {"steps_per_s": round(n1 / el1, 3), "ms_per_step": round(el1 / n1 * 1e3, 2),
                           "GBps": round(step_bytes * n1 / el1 / 1e9, 3)},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "host_cpus_usable": len(os.sched_getaffinity(0))}


def all_configs(args):
    """The full Graft step on each of the five workloads at its own shape: one
    build launch + one verify/update launch per step, replayed from HIP graphs
    over a pool of `--pool` steps of a real seeded trajectory (after the
    workload's warm-up; workload 4 ingests its prompt first).  One JSON line per
    workload: time per step and the step's logits bytes against 8 TB/s."""
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    P = max(1, args.pool)
    for cid in [int(x) for x in args.config_list.split(",") if x.strip()]:
        rec = time_workload(cid, args.steps, args.warmup, P, dev, torch, repeats=args.repeats)
        log("workload %d (%s): %.2f us/step, %.0f GB/s (setup %.1fs)"
            % (cid, rec["workload"], rec["us_per_step"], rec["step_GBps"], rec["setup_s"]))
        rec.update({"mode": "all_configs", "hip_graph": True, "data": "synthetic"})
        print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.all_configs:
        return all_configs(args)
    if args.template_sweep:
        return template_sweep(args)
    if args.ablation:
        return ablation(args)
    if args.calibration:
        return calibration(args)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: it measures the single-GPU Graft step "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from hybrid_draft_tree_amd import _lib as L
    from hybrid_draft_tree_amd.driver import GraftPipeline
    from synth import WORKLOADS
    from synth import generators as G
    from synth import runner as R

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = WORKLOADS[3]
    B, T1, V, k = cfg.B, cfg.rows_per_request, cfg.V, cfg.k
    n_rows = B * T1
    P = max(1, args.pool)
    bytes_logits = n_rows * V * 2

    t0 = time.time()
    pipe, pool_drafts, pool_logits, acc_pool = setup_pool(cfg, P, dev, torch)
    log("setup %.1fs: pool of %d steps (%.1f MB each), accepted per step in pool: %s"
        % (time.time() - t0, P, bytes_logits / 1e6, acc_pool))

    # ---------------- timed region: whole steps ----------------
    # exactly --warmup untimed steps, then --repeats windows of exactly --steps
    # steps each (HIP events on the replay stream, the first recorded behind the
    # queued warm-up); the reported step time is the median window
    K, W = max(1, args.steps), max(0, args.warmup)
    rep = StepReplayer(pipe, pool_drafts, pool_logits, torch, use_graph=not args.no_graph)
    win_ms, wall = timed_steps(rep, K, W, args.repeats, torch)
    stream = torch.cuda.current_stream()
    ms_step = _median(win_ms) / K
    steps_per_s = 1000.0 / ms_step
    step_bytes = bytes_logits + n_rows * k * 4
    log("timed %d x %d steps after %d warm-up steps: windows %s ms (median %.2f us/step), %.3f s wall"
        % (args.repeats, K, W, ["%.3f" % x for x in win_ms], ms_step * 1e3, wall))

    # ---------------- dominant kernel alone ----------------
    # graft_verify_update: one launch of k_topk_mw (row-wise top-k + acceptance
    # walk + matrix update), the kernel that carries the step's logits traffic.
    def verify_call(i):
        L.graft_verify_update(B, T1, V, k, pipe.dtype, pool_logits[i % P].data_ptr(), pipe.tok.data_ptr(),
                              pipe.parent.data_ptr(), pipe.depth.data_ptr(), pipe.table.data_ptr(), None,
                              pipe.topk.data_ptr(), None, None, pipe.accept_len.data_ptr(), pipe.accept_idx.data_ptr(),
                              pipe.dmax, pipe.roots.data_ptr(), None, pipe.ws.data_ptr(), pipe.ws_bytes,
                              stream.cuda_stream)

    iters = max(P, args.kernel_iters)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(min(iters, 8)):
        verify_call(i)
    torch.cuda.synchronize()
    for i in range(iters):
        a, b = evs[i]
        a.record(stream)
        verify_call(i)
        b.record(stream)
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) for a, b in evs)
    kb_ms = sum(durs) / len(durs)        # one event pair around each launch: adds its dispatch latency
    kb_med = durs[len(durs) // 2]
    # the launch's average duration: one event pair around `iters` back-to-back
    # launches on the launch stream (each launch still pays the gap to the next)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for i in range(iters):
        verify_call(i)
    f1.record(stream)
    torch.cuda.synchronize()
    k_ms = f0.elapsed_time(f1) / iters
    alg_bytes = bytes_logits + n_rows * k * 4
    achieved = alg_bytes / (k_ms * 1e-3) / 1e9
    traffic, tnote = load_traffic(alg_bytes)
    log("dominant kernel: %.2f us per launch back to back (%.0f GB/s algorithmic); bracketed one by one: mean "
        "%.2f us, median %.2f us" % (k_ms * 1e3, achieved, kb_ms * 1e3, kb_med * 1e3))

    # ---------------- measured read ceiling of the same rows ----------------
    # graft_stream_read: the pool's logits read with the verify launch's geometry
    # (one workgroup of four wavefronts per row, 16-byte non-temporal loads) and
    # nothing else, back to back like the dominant kernel above
    sink = torch.zeros(n_rows, dtype=torch.int32, device=dev)

    def stream_call(i):
        L.graft_stream_read(pool_logits[i % P].data_ptr(), n_rows, V * 2, sink.data_ptr(), stream.cuda_stream)

    for i in range(min(iters, 8)):
        stream_call(i)
    torch.cuda.synchronize()
    f0.record(stream)
    for i in range(iters):
        stream_call(i)
    f1.record(stream)
    torch.cuda.synchronize()
    s_ms = f0.elapsed_time(f1) / iters
    ceiling = bytes_logits / (s_ms * 1e-3) / 1e9
    log("read ceiling of the same rows (graft_stream_read): %.2f us per launch, %.0f GB/s (%.1f %% of peak); the "
        "dominant kernel reaches %.1f %% of it, the step %.1f %%" % (s_ms * 1e3, ceiling, 100 * ceiling / PEAK_HBM_GBPS,
                                                                  100 * achieved / ceiling,
                                                                  100 * step_bytes / (ms_step * 1e-3) / 1e9 / ceiling))

    # ---------------- coverage-gain diagnostic (outside the step) ----------------
    # The verify launch with per-row softmax statistics, then graft_coverage_gain,
    # on pool step 0 rebuilt with row sources.
    row_src = torch.zeros(B, T1, dtype=torch.uint8, device=dev)
    row_stats = torch.zeros(B, T1, 2, dtype=torch.float32, device=dev)
    gain = torch.zeros(B, dtype=torch.float32, device=dev)
    pipe.row_src = row_src
    pipe.build_device(pool_drafts[0])
    pipe.row_src = None

    def verify_stats_call(i):
        L.graft_verify_update(B, T1, V, k, pipe.dtype, pool_logits[i % P].data_ptr(), pipe.tok.data_ptr(),
                              pipe.parent.data_ptr(), pipe.depth.data_ptr(), pipe.table.data_ptr(), None,
                              pipe.topk.data_ptr(), None, row_stats.data_ptr(), pipe.accept_len.data_ptr(),
                              pipe.accept_idx.data_ptr(), pipe.dmax, pipe.bonus_scratch.data_ptr(), None,
                              pipe.ws.data_ptr(), pipe.ws_bytes, stream.cuda_stream)

    def coverage_call(i):
        L.graft_coverage_gain(B, T1, V, pipe.dtype, pool_logits[0].data_ptr(), pipe.tok.data_ptr(),
                              pipe.parent.data_ptr(), row_src.data_ptr(), row_stats.data_ptr(),
                              gain.data_ptr(), stream.cuda_stream)

    def time_calls(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(min(n, 4)):
            fn(i)
        torch.cuda.synchronize()
        for i in range(n):
            a, b = ev[i]
            a.record(stream)
            fn(i)
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n

    pipe.bonus_scratch = torch.zeros(B, dtype=torch.int32, device=dev)  # roots stay untouched
    vs_ms = time_calls(verify_stats_call, 52)
    verify_stats_call(0)  # statistics of pool step 0 for the coverage launch
    cov_ms = time_calls(coverage_call, 50)
    gain_mean = float(gain.mean().item())
    n_ret_mean = float(pipe.n_ret.float().mean().item())
    log("coverage diagnostic: verify with row statistics %.2f us (+%.2f us), coverage launch %.2f us, "
        "mean gain %.4f over %.1f retrieved rows/request" % (vs_ms * 1e3, (vs_ms - kb_ms) * 1e3, cov_ms * 1e3,
                                                              gain_mean, n_ret_mean))

    # ---------------- retrieval ahead of the draft (outside the step) ----------------
    # Section 二: retrieval needs only the roots and the matrix, so it can run
    # while the drafter works; what remains after the draft is prune + flatten.
    def build_call(i):
        pipe.build_device(pool_drafts[i % P])

    def retrieve_call(i):
        L.graft_retrieve_expand(B, V, k, pipe.mode, pipe.slots, pipe.table.data_ptr(), pipe.roots.data_ptr(), None,
                                None, pipe.Nd, pipe.tpl, pipe.cfg, pipe.ret_tok.data_ptr(), pipe.ret_parent.data_ptr(),
                                pipe.n_ret.data_ptr(), pipe.r_out, stream.cuda_stream)

    def after_call(i):
        d = pool_drafts[i % P]
        L.graft_build_after_retrieval(
            B, pipe.Nd, T1, pipe.layout, pipe.slots, pipe.cfg, pipe.roots.data_ptr(), pipe.base_pos.data_ptr(),
            d["parent"].data_ptr(), d["layer"].data_ptr(), d["score"].data_ptr(), d["tok"].data_ptr(),
            pipe.stage.data_ptr(), pipe.n_keep.data_ptr(), pipe.keep.data_ptr(), pipe.cum.data_ptr(),
            pipe.ret_tok.data_ptr(), pipe.ret_parent.data_ptr(), pipe.n_ret.data_ptr(), pipe.r_out,
            pipe.tok.data_ptr(), pipe.parent.data_ptr(), pipe.depth.data_ptr(), pipe.pos_id.data_ptr(),
            pipe.anc.data_ptr(), None, stream.cuda_stream)

    def time_after(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            retrieve_call(i)        # ahead, outside the bracket
            a, b = ev[i]
            a.record(stream)
            after_call(i)
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n

    build_ms = time_calls(build_call, 50)
    ret_ms = time_calls(retrieve_call, 50)
    time_after(4)
    after_ms = time_after(50)
    log("retrieval ahead: one-launch build %.2f us; retrieval alone %.2f us; prune + flatten after it %.2f us"
        % (build_ms * 1e3, ret_ms * 1e3, after_ms * 1e3))

    # ---------------- the same kernel on the other shapes (outside the step) ----------------
    # TAIL (16 requests x 17 rows: a 16-token block plus its anchor, 82.65 MB of
    # logits) and one prompt-ingest chunk (2048 rows, 622.3 MB): each a single
    # top-k launch, timed like the dominant kernel.
    tcfg = WORKLOADS[5]
    tp = GraftPipeline.from_config(tcfg, device=dev)
    tad = _Adapter(tp, torch)
    twl = R.Workload(tcfg)
    R.start(tad, twl)
    for s_ in range(2):
        R.step(tad, twl, s_, G.WARMUP_STREAM_OFFSET)
    tflat = tad.build(twl.draft(0, tad.get_roots()))
    tbuf = torch.empty(tcfg.B * tcfg.rows_per_request, V, dtype=torch.bfloat16, device=dev)
    tad.rows = tad.DeviceRows(twl.pool, dev)
    tad.rows.materialize(twl.logit_desc(0, tflat), out=tbuf)
    t_scratch = torch.zeros(tcfg.B, dtype=torch.int32, device=dev)

    def tail_call(i):
        L.graft_verify_update(tcfg.B, tp.T1, V, k, tp.dtype, tbuf.data_ptr(), tp.tok.data_ptr(), tp.parent.data_ptr(),
                              tp.depth.data_ptr(), tp.table.data_ptr(), None, tp.topk.data_ptr(), None, None,
                              tp.accept_len.data_ptr(), tp.accept_idx.data_ptr(), tp.dmax, t_scratch.data_ptr(), None,
                              tp.ws.data_ptr(), tp.ws_bytes, stream.cuda_stream)

    tail_bytes = tbuf.numel() * 2 + tbuf.shape[0] * k * 4
    tail_ms = time_calls(tail_call, 50)
    chunk = 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(20240)
    ibuf = torch.randn(chunk, V, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    irow = torch.randint(0, V, (chunk,), generator=gen, device=dev, dtype=torch.int32)
    itab = torch.zeros(V, k, dtype=torch.int32, device=dev)
    iout = torch.empty(chunk, k, dtype=torch.int32, device=dev)
    iws_n = L.graft_workspace_bytes(chunk, V, k, pipe.dtype)
    iws = torch.zeros(iws_n, dtype=torch.uint8, device=dev)

    def ingest_call(i):
        L.graft_update_topk(chunk, V, k, pipe.dtype, ibuf.data_ptr(), None, None, irow.data_ptr(), itab.data_ptr(),
                            None, iout.data_ptr(), iws.data_ptr(), iws_n, stream.cuda_stream)

    ingest_bytes = ibuf.numel() * 2 + chunk * k * 4
    ingest_ms = time_calls(ingest_call, 20)
    # one request's tree (61 rows of the same vocabulary): top-k + matrix update
    b1 = T1

    def b1_call(i):
        L.graft_update_topk(b1, V, k, pipe.dtype, ibuf.data_ptr(), None, None, irow.data_ptr(), itab.data_ptr(),
                            None, iout.data_ptr(), iws.data_ptr(), iws_n, stream.cuda_stream)

    b1_bytes = b1 * V * 2 + b1 * k * 4
    b1_ms = time_calls(b1_call, 50)
    log("other shapes: TAIL verify %.2f us (%.0f GB/s); ingest chunk of %d rows %.2f us (%.0f GB/s); "
        "one request's %d rows %.2f us (%.0f GB/s)"
        % (tail_ms * 1e3, tail_bytes / (tail_ms * 1e-3) / 1e9, chunk, ingest_ms * 1e3,
           ingest_bytes / (ingest_ms * 1e-3) / 1e9, b1, b1_ms * 1e3, b1_bytes / (b1_ms * 1e-3) / 1e9))
    del ibuf, iws, tbuf

    copy_gbps = None
    if args.copy_calib:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            y.copy_(x)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * (1 << 30) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        log("plain 1 GiB copy: %.0f GB/s (read + write)" % copy_gbps)

    # ---------------- small shapes: the full step at other workloads ----------------
    shapes = []
    if not args.no_shapes:
        for cid in (1, 2, 4, 5):
            rec = time_workload(cid, args.shape_steps, 8, P, dev, torch, repeats=3)
            log("full step, workload %d (%s): %.2f us/step (%.0f GB/s)"
                % (cid, rec["workload"], rec["us_per_step"], rec["step_GBps"]))
            shapes.append({key: rec[key] for key in ("workload", "batch", "vocab", "verified_rows", "dtype",
                                                     "us_per_step", "us_per_step_min", "us_per_step_max",
                                                     "steps_per_s", "step_GBps", "step_frac_of_peak")})

    # ---------------- CPU oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, pipe, pool_drafts, pool_logits, step_bytes, args.cpu_seconds, torch)

    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 6),
        "repeats": {"n": args.repeats, "steps_each": K, "us_per_step_median": round(ms_step * 1e3, 3),
                    "us_per_step_min": round(min(win_ms) * 1e3 / K, 3),
                    "us_per_step_max": round(max(win_ms) * 1e3 / K, 3),
                    "timing": "HIP events on the replay stream around each window of exactly K steps, "
                              "each window one HIP-graph replay (replayed once untimed before the warm-up, "
                              "since a graph's first launch also uploads it); the first event is recorded "
                              "behind the queued warm-up steps; value = the median",
                    "events": getattr(timed_steps, "events", "torch")},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "graft_step_static_slots_b16_v151936", "batch": B, "vocab": V, "slots": cfg.slots,
                   "rows_per_request": T1, "k": k, "layout": cfg.layout, "logits_bytes_per_step": bytes_logits,
                   "pool_steps": P, "hip_graph": not args.no_graph},
        "step_hbm_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "step_frac_of_ceiling": round(step_bytes / (ms_step * 1e-3) / 1e9 / ceiling, 4),
        "read_ceiling": {"GBps": round(ceiling, 1), "frac_of_peak": round(ceiling / PEAK_HBM_GBPS, 4),
                         "us_per_launch": round(s_ms * 1e3, 3), "bytes": bytes_logits,
                         "what": "graft_stream_read over the same pool rows with the verify launch's geometry "
                                 "(976 workgroups x 4 wavefronts, 16-byte non-temporal loads, two 1 KB blocks per "
                                 "batch with the next in flight), %d back-to-back launches" % iters},
        "coverage_diagnostic": {"verify_with_row_stats_us": round(vs_ms * 1e3, 3),
                                "row_stats_overhead_us": round((vs_ms - kb_ms) * 1e3, 3),
                                "coverage_kernel_us": round(cov_ms * 1e3, 3),
                                "mean_gain": round(gain_mean, 6),
                                "note": "outside the timed step; pool step 0's draft rebuilt with row "
                                        "sources against the evolved matrix"},
        "retrieval_ahead_diagnostic": {"build_one_launch_us": round(build_ms * 1e3, 3),
                                       "retrieval_us": round(ret_ms * 1e3, 3),
                                       "build_after_retrieval_us": round(after_ms * 1e3, 3),
                                       "note": "event-timed single launches (dispatch included) outside the timed "
                                               "step; with retrieval run ahead on a side stream during drafting, "
                                               "the post-draft build is build_after_retrieval_us"},
        "other_shapes_diagnostic": {
            "tail_verify_us": round(tail_ms * 1e3, 3),
            "tail_GBps": round(tail_bytes / (tail_ms * 1e-3) / 1e9, 1),
            "ingest_chunk_us": round(ingest_ms * 1e3, 3),
            "ingest_GBps": round(ingest_bytes / (ingest_ms * 1e-3) / 1e9, 1),
            "one_request_61_rows_us": round(b1_ms * 1e3, 3),
            "one_request_61_rows_GBps": round(b1_bytes / (b1_ms * 1e-3) / 1e9, 1),
            "note": "the top-k launch on the TAIL shape (16 x 17 rows, graft_verify_update) and on one 2048-row "
                    "prompt-ingest chunk and on one request's 61 rows (graft_update_topk with logits), "
                    "event-timed single launches outside the timed step"},
        "full_step_other_workloads": shapes or None,
        "roofline": {"kernel": "k_topk_mw (graft_verify_update: row-wise top-k + acceptance walk + matrix update)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "frac_of_ceiling": round(achieved / ceiling, 4),
                     "kernel_us_mean": round(k_ms * 1e3, 3),
                     "kernel_us_bracketed_mean": round(kb_ms * 1e3, 3),
                     "kernel_us_bracketed_median": round(kb_med * 1e3, 3),
                     "timing": "HIP events on the launch stream around %d back-to-back launches of "
                               "graft_verify_update (the bracketed figures put one event pair around each "
                               "launch, which adds its dispatch latency)" % iters,
                     "alg_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
    }
    if copy_gbps is not None:
        out["copy_1GiB_GBps"] = round(copy_gbps, 1)
    if traffic is None:
        out["roofline"]["traffic_note"] = tnote
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
