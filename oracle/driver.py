"""Step-level composition of the CPU oracle: one Graft decode step is
prune -> retrieve -> flatten -> (target scores the rows) -> top-k -> accept ->
update, in the order of the write-up's "three gears" section.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check, the benchmark's CPU-baseline
leg).  State: the continuation matrix (int32 [V, k], every row starting as
0..k-1), one root token and root position per request.
"""
from __future__ import annotations

import numpy as np

from . import oracle as O


class OracleGraft:
    def __init__(self, cfg):
        self.cfg = cfg
        V, k = cfg.V, cfg.k
        self.table = np.tile(np.arange(k, dtype=np.int32), (V, 1))
        self.table_prob = None
        if cfg.mode == "tree":
            Rmax = cfg.slots - min(cfg.keep)
            if cfg.tpl_kind == "branching":
                self.tpl = O.template_branching(W=cfg.tpl_width, D=cfg.tpl_depth, beta=cfg.tpl_beta, Rmax=Rmax)
            elif cfg.tpl_kind == "none":
                self.tpl = {k: np.zeros(0, np.int32) for k in ("parent", "rank", "depth")}
            else:
                self.tpl = O.template(W=cfg.tpl_width, D=cfg.tpl_depth, Rmax=Rmax)
        self.roots = np.zeros(cfg.B, np.int32)
        self.base_pos = np.zeros(cfg.B, np.int32)
        self.last = {}
        self.log_thr = None        # calibrated fp32 log-thresholds, else (float) ln cfg.tau
        self._calib = None

    # -- threshold calibration over warm-up steps (section 二) ----------------
    def begin_calibration(self):
        self._calib = []

    def end_calibration(self, q):
        """Thresholds from the checkpoint statistics of the steps built since
        begin_calibration(); used by every later step.  Returns them (fp32 ln)."""
        samples = np.concatenate(self._calib) if self._calib else np.zeros((0, 3), np.float32)
        self._calib = None
        self.log_thr = O.calibrate(samples, q)
        return self.log_thr.copy()

    # -- state -------------------------------------------------------------
    def set_roots(self, roots, base_pos):
        self.roots = np.array(roots, np.int32)
        self.base_pos = np.array(base_pos, np.int32)

    def get_roots(self):
        return self.roots.copy()

    def get_table(self):
        return self.table.copy()

    # -- gear 1 + 2 + flatten ----------------------------------------------
    def build(self, draft):
        cfg = self.cfg
        B = cfg.B
        T1 = cfg.rows_per_request
        if cfg.mode == "tree":
            if self._calib is not None:
                self._calib.append(O.checkpoint_stats(draft["parent"], draft["layer"], draft["logp"],
                                                      cfg.ckpt_layers, cfg.keep))
            pr = O.prune_tree(draft["parent"], draft["layer"], draft["logp"], cfg.ckpt_layers, cfg.tau,
                              cfg.keep, want_cum=True, node_tau=cfg.node_tau, log_thr=self.log_thr)
            ret = O.retrieve_tree(self.table, self.roots, pr["n_keep"], cfg.slots, self.tpl)
        else:
            pr = O.prune_tail(draft["conf"], cfg.tail_thr)
            ret = O.retrieve_tail(self.table, self.roots, draft["tok"], pr["n_keep"])
        fl = O.flatten(cfg.layout, T1, self.roots, self.base_pos, draft["tok"],
                       draft.get("parent", np.tile(np.arange(-1, cfg.n_draft - 1, dtype=np.int32), (B, 1))),
                       pr["keep"], pr["n_keep"], ret)
        out = dict(pr)
        out.update(ret)
        out.update(fl)
        self.last = out
        return out

    # -- verify + update ----------------------------------------------------
    def verify_update(self, logits, want_prob=False, want_coverage=False):
        cfg = self.cfg
        B, T1, k = cfg.B, cfg.rows_per_request, cfg.k
        Dmax = T1 - 1
        if want_prob:
            tk, prob = O.topk(logits.reshape(B * T1, cfg.V), k, cfg.dtype, want_prob=True)
        else:
            tk, prob = O.topk(logits.reshape(B * T1, cfg.V), k, cfg.dtype), None
        tk = tk.reshape(B, T1, k)
        fl = self.last
        acc = O.accept(fl["tok"], fl["parent"], tk[:, :, 0], Dmax)
        if want_prob and self.table_prob is None:
            self.table_prob = np.zeros((cfg.V, k), np.float32)
        O.update(self.table, fl["tok"].reshape(-1), tk.reshape(-1, k),
                 prob if want_prob else None, self.table_prob if want_prob else None)
        out = dict(acc)
        out["topk"] = tk
        if want_prob:
            out["topk_prob"] = prob.reshape(B, T1, k)
        if want_coverage:
            # coverage gain of the tree just verified (section 三), fp64
            out["coverage"] = O.coverage_gain(logits.reshape(B, T1, cfg.V), fl["tok"], fl["parent"],
                                              fl["row_src"], cfg.dtype)
        self.roots = acc["bonus"].copy()
        self.base_pos = self.base_pos + acc["accept_len"] + 1
        return out

    # -- prompt ingest (long-context section) --------------------------------
    def ingest_chunk(self, row_tok, logits):
        tk = O.topk(logits, self.cfg.k, self.cfg.dtype)
        O.update(self.table, row_tok, tk)
        return tk
