"""Drive any Graft backend (CPU oracle or HIP path) through seeded synthetic
steps.  This module only generates inputs and keeps the synthetic drafter's and
target's context (the committed token stream); every step of the method runs
inside the backend.

Backend protocol:
    set_roots(roots, base_pos) / get_roots() / get_table()
    build(draft) -> dict with host arrays "tok", "parent" ([B, T1]) at least
    verify_update(logits_rows) -> dict with host "accept_len", "accept_idx", "bonus"
    ingest_chunk(row_tok, logits_rows) -> top-k rows (host or device)
    materialize(pool, desc) -> logits rows in the backend's own memory
    begin_calibration() / end_calibration(q) -> fp32 log-thresholds [3]
        (only when the workload sets calib_q)
"""
from __future__ import annotations

import numpy as np

from . import generators as G
from .configs import GraftConfig


class Workload:
    """Per-run synthetic context: topology, noise pool, per-request intents and
    the committed stream."""

    def __init__(self, cfg: GraftConfig, pool: G.NoisePool | None = None, prompt=None):
        self.cfg = cfg
        self.pool = pool if pool is not None else G.NoisePool(cfg)
        self.topo = G.static_tree(cfg.layer_sizes, cfg.tree_width) if cfg.mode == "tree" else None
        self.prompt = prompt
        if cfg.cfg_id == 4:
            if self.prompt is None:
                self.prompt = G.long_prompt(cfg)
            base = G.PromptCopyIntent(cfg, self.prompt)
            self.intents = [base.clone() for _ in range(cfg.B)]
            self.prevs = [int(self.prompt[-1])] * cfg.B
        else:
            roots, prevs = G.initial_roots(cfg)
            self.init_roots = roots
            self.prevs = list(prevs)
            if cfg.cfg_id == 2:
                shared = G.Order2Intent(cfg).shared
                self.intents = [G.Order2Intent(cfg, shared) for _ in range(cfg.B)]
            else:
                it = G.BigramIntent(cfg)
                self.intents = [it] * cfg.B
            for b in range(cfg.B):
                self.intents[b].commit([self.prevs[b], int(roots[b])])

    # -- per-step inputs -------------------------------------------------------
    def draft(self, step: int, roots, stream_off: int = 0):
        cfg = self.cfg
        if cfg.mode == "tree":
            par, lay, _ = self.topo
            Nd = len(par)
            out = {"parent": np.tile(par, (cfg.B, 1)), "layer": np.tile(lay, (cfg.B, 1)),
                   "logp": np.zeros((cfg.B, Nd), np.float32), "tok": np.zeros((cfg.B, Nd), np.int32)}
            for b in range(cfg.B):
                rng = G.rng_for(cfg.cfg_id, b, step, G.STREAM_DRAFT + stream_off)
                lp, tk = G.draft_tree_inputs(cfg, self.topo, rng, int(roots[b]), self.prevs[b], self.intents[b])
                out["logp"][b] = lp
                out["tok"][b] = tk
            return out
        L = cfg.tail_block
        out = {"conf": np.zeros((cfg.B, L), np.float32), "tok": np.zeros((cfg.B, L), np.int32)}
        for b in range(cfg.B):
            rng = G.rng_for(cfg.cfg_id, b, step, G.STREAM_DRAFT + stream_off)
            conf, tk = G.tail_block_inputs(cfg, rng, int(roots[b]), self.prevs[b], self.intents[b])
            out["conf"][b] = conf
            out["tok"][b] = tk
        return out

    def logit_desc(self, step: int, flat, stream_off: int = 0):
        cfg = self.cfg
        descs = []
        for b in range(cfg.B):
            cols = G.tree_row_cols(self.intents[b], flat["tok"][b], flat["parent"][b], self.prevs[b])
            rng = G.rng_for(cfg.cfg_id, b, step, G.STREAM_LOGITS + stream_off)
            descs.append(G.row_descriptors(self.pool, rng, cols))
        return {key: np.concatenate([d[key] for d in descs]) for key in descs[0]}

    def commit(self, roots, flat, res):
        """Advance the synthetic context by what the backend committed."""
        for b in range(self.cfg.B):
            n = int(res["accept_len"][b])
            path = [int(flat["tok"][b][int(i)]) for i in res["accept_idx"][b][:n]]
            committed = path + [int(res["bonus"][b])]
            self.intents[b].commit(committed)
            seq = [int(roots[b])] + committed
            self.prevs[b] = seq[-2]

    # -- prompt ingest (workload 4) ----------------------------------------------
    def ingest_descs(self):
        cfg = self.cfg
        cols = G.prompt_row_cols(self.prompt, G.PromptCopyIntent(cfg, self.prompt[:-1],
                                                                 shared=self.intents[0].bigram))
        n = len(self.prompt)
        for c0 in range(0, n, cfg.ingest_chunk):
            c1 = min(n, c0 + cfg.ingest_chunk)
            rng = G.rng_for(cfg.cfg_id, 0, c0 // cfg.ingest_chunk, G.STREAM_INGEST)
            yield c0, c1, G.row_descriptors(self.pool, rng, cols[c0:c1])


def start(backend, wl: Workload):
    """Initial roots; for workload 4 the prompt is ingested first and every request
    starts from the greedy token of the last prompt row."""
    cfg = wl.cfg
    if cfg.cfg_id == 4:
        last = None
        for c0, c1, desc in wl.ingest_descs():
            rows = backend.materialize(wl.pool, desc)
            last = backend.ingest_chunk(wl.prompt[c0:c1], rows)
        g_last = int(np.asarray(_host(last))[-1][0])
        backend.set_roots(np.full(cfg.B, g_last, np.int32), np.full(cfg.B, len(wl.prompt), np.int32))
        for b in range(cfg.B):
            wl.intents[b].commit([g_last])
    else:
        backend.set_roots(wl.init_roots, np.full(cfg.B, cfg.init_base_pos, np.int32))


def _host(x):
    if hasattr(x, "cpu"):
        return x.cpu().numpy()
    return x


def step(backend, wl: Workload, step_idx: int, stream_off: int = 0, record=None):
    roots = np.asarray(backend.get_roots())
    draft = wl.draft(step_idx, roots, stream_off)
    flat = backend.build(draft)
    desc = wl.logit_desc(step_idx, flat, stream_off)
    rows = backend.materialize(wl.pool, desc)
    res = backend.verify_update(rows)
    wl.commit(roots, flat, res)
    if record is not None:
        record.append({"draft": draft, "flat": flat, "res": res})
    return flat, res


def warm_up(backend, wl: Workload, n: int):
    """n warm-up steps on their own seed streams; with cfg.calib_q set, the
    backend calibrates its checkpoint thresholds over them."""
    calib = bool(wl.cfg.calib_q) and wl.cfg.mode == "tree"
    if calib:
        backend.begin_calibration()
    for s in range(n):
        step(backend, wl, s, G.WARMUP_STREAM_OFFSET)
    if calib:
        return backend.end_calibration(wl.cfg.calib_q)
    return None


def run(backend, wl: Workload, n_steps: int, warmup: int | None = None, on_step=None):
    """start + warm-up (own seed streams) + n_steps measured steps."""
    cfg = wl.cfg
    start(backend, wl)
    w = cfg.warmup_steps if warmup is None else warmup
    if cfg.cfg_id == 4:
        w = 0 if warmup is None else warmup
    warm_up(backend, wl, w)
    for s in range(n_steps):
        flat, res = step(backend, wl, s)
        if on_step is not None:
            on_step(s, flat, res)
