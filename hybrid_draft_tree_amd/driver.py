"""Device-resident Graft pipeline over the C ABI.

PyTorch provides device memory and the stream; every step of the method runs
in libgraft.so.  One ``GraftPipeline`` holds, for a batch of B requests:

* the continuation matrix ``table`` int32 [V, k] (every row starts as 0..k-1),
* the roots (last committed token per request) and their positions,
* per-step buffers for the draft tree, the hybrid tree and the verification
  outputs, and one workspace for the row-wise top-k.

A decode step is ``build(draft)`` (prune -> retrieve -> flatten), the target
forward that scores the flattened rows (outside this library), then
``verify_update(logits)`` (top-k -> accept -> matrix update).  By default each
half is one launch (graft_build_hybrid_tree, graft_verify_update); with
``fused=False`` the five separate entry points are used.  ``bonus`` is
written straight into the root buffer and ``base_pos`` is advanced on the
device, so consecutive steps need no host round trip.

With ``want_coverage`` the build also records each row's source (root, draft,
retrieved), verification exports every row's softmax statistics, and
``verify_update`` adds the coverage gain per request (graft_coverage_gain).

With ``overlap`` (TREE) the retrieval runs ahead on a side stream: it needs only
the roots and the matrix, so ``build`` launches it before the draft is loaded
and the prune + flatten launch (graft_build_after_retrieval) waits for it.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from . import _lib as L


class GraftPipeline:
    def __init__(self, *, V, B, k=8, slots=60, mode="tree", layout="compact", dtype="bf16",
                 n_draft=60, ckpt_layers=(0, 1, 5), tau=(0.3, 0.2, 0.1), keep=(8, 24, 40),
                 tail_thr=0.5, tpl_width=8, tpl_depth=8, tpl_kind="chain", tpl_beta=(1, 1), node_tau=0.0,
                 want_prob=False, want_coverage=False, device="cuda", fused=True, overlap=False,
                 debug_checks=None):
        L.load()
        self.fused = bool(fused)
        self.overlap = bool(overlap)
        # check every loaded draft on the device (graft_check_draft) and raise on a
        # failed precondition; default from GRAFT_DEBUG_CHECKS=1 in the environment
        if debug_checks is None:
            debug_checks = os.environ.get("GRAFT_DEBUG_CHECKS", "0") not in ("", "0")
        self.debug_checks = bool(debug_checks)
        self.V, self.B, self.k = int(V), int(B), int(k)
        self.mode = L.MODE_TREE if mode == "tree" else L.MODE_TAIL
        self.layout = L.LAYOUT[layout]
        self.dtype = L.DTYPE_BF16 if dtype == "bf16" else L.DTYPE_F32
        self.slots = int(slots)
        self.Nd = int(n_draft)
        self.T1 = self.slots + 1
        self.dmax = self.T1 - 1
        self.want_prob = bool(want_prob)
        self.want_coverage = bool(want_coverage)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        # fp32 thresholds; tau 0 never fires (-inf), tau +inf always fires
        log_thr = [-math.inf if t == 0 else float(np.float32(math.log(t))) for t in tau]
        node_thr = float(np.float32(math.log(node_tau))) if node_tau > 0 else None
        self.cfg = L.prune_cfg(ckpt_layers, log_thr, keep, tail_thr, node_thr)

        self.table = torch.arange(self.k, **i32).repeat(self.V, 1).contiguous()
        self.table_prob = torch.zeros(self.V, self.k, dtype=torch.float32, device=dev) if want_prob else None
        self.roots = torch.zeros(self.B, **i32)
        self.base_pos = torch.zeros(self.B, **i32)

        B, Nd, T1 = self.B, self.Nd, self.T1
        self.d_parent = torch.full((B, Nd), -1, **i32)
        self.d_layer = torch.zeros(B, Nd, **i32)
        self.d_score = torch.zeros(B, Nd, dtype=torch.float32, device=dev)
        self.d_tok = torch.zeros(B, Nd, **i32)
        self.stage = torch.zeros(B, **i32)
        self.n_keep = torch.zeros(B, **i32)
        self.keep = torch.zeros(B, Nd, dtype=torch.uint8, device=dev)
        self.cum = torch.zeros(B, Nd, dtype=torch.float32, device=dev)

        if self.mode == L.MODE_TREE:
            cap = self.slots - min(keep)
            if tpl_kind == "branching":
                par, rk, dp = L.graft_template_branching(tpl_width, tpl_depth, tpl_beta[0], tpl_beta[1], cap)
            elif tpl_kind == "chain":
                par, rk, dp = L.graft_template_master(tpl_width, tpl_depth, cap)
            elif tpl_kind == "none":      # no retrieval: freed slots stay empty
                par, rk, dp = [], [], []
            else:
                raise ValueError("unknown template kind %r" % (tpl_kind,))
            self.tpl_parent = torch.tensor(par, **i32)
            self.tpl_rank = torch.tensor(rk, **i32)
            self.tpl_depth = torch.tensor(dp, **i32)
            self.tpl = L.Template(len(par), self.tpl_parent.data_ptr(), self.tpl_rank.data_ptr(),
                                  self.tpl_depth.data_ptr())
            self.r_out = max(len(par), 1)
        else:
            self.tpl = None
            self.r_out = self.slots
        self.ret_tok = torch.zeros(B, self.r_out, **i32)
        self.ret_parent = torch.zeros(B, self.r_out, **i32)
        self.n_ret = torch.zeros(B, **i32)

        self.tok = torch.zeros(B, T1, **i32)
        self.parent = torch.zeros(B, T1, **i32)
        self.depth = torch.zeros(B, T1, **i32)
        self.pos_id = torch.zeros(B, T1, **i32)
        self.anc = torch.zeros(B, T1, dtype=torch.int64, device=dev)
        self.row_src = torch.zeros(B, T1, dtype=torch.uint8, device=dev) if want_coverage else None
        self.row_stats = torch.zeros(B, T1, 2, dtype=torch.float32, device=dev) if want_coverage else None
        self.gain = torch.zeros(B, dtype=torch.float32, device=dev) if want_coverage else None

        self.topk = torch.zeros(B, T1, self.k, **i32)
        self.topk_prob = torch.zeros(B, T1, self.k, dtype=torch.float32, device=dev) if want_prob else None
        self.accept_len = torch.zeros(B, **i32)
        self.accept_idx = torch.zeros(B, max(self.dmax, 1), **i32)
        self.ws_bytes = L.graft_workspace_bytes(B * T1, self.V, self.k, self.dtype)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self._ingest_ws = None
        self._calib = None          # warm-up checkpoint statistics [steps * B, 3] while calibrating
        self._calib_rows = 0
        if self.overlap:
            if self.mode != L.MODE_TREE:
                raise ValueError("retrieval ahead of the draft applies to TREE mode only")
            self.side = torch.cuda.Stream(device=dev)   # default priority
            self._ev_inputs = torch.cuda.Event()
            self._ev_ret = torch.cuda.Event()

    @classmethod
    def from_config(cls, cfg, want_prob=False, want_coverage=False, device="cuda", fused=True, overlap=False):
        return cls(V=cfg.V, B=cfg.B, k=cfg.k,
                   slots=cfg.tail_block if cfg.mode == "tail" else cfg.slots,
                   mode=cfg.mode, layout=cfg.layout, dtype=cfg.dtype, n_draft=cfg.n_draft,
                   ckpt_layers=cfg.ckpt_layers, tau=cfg.tau, keep=cfg.keep, tail_thr=cfg.tail_thr,
                   tpl_width=cfg.tpl_width, tpl_depth=cfg.tpl_depth, tpl_kind=cfg.tpl_kind,
                   tpl_beta=cfg.tpl_beta, node_tau=cfg.node_tau, want_prob=want_prob,
                   want_coverage=want_coverage, device=device, fused=fused, overlap=overlap)

    # ------------------------------------------------------------------ state
    def stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def set_roots(self, roots, base_pos):
        self.roots.copy_(torch.as_tensor(np.asarray(roots, np.int32)))
        self.base_pos.copy_(torch.as_tensor(np.asarray(base_pos, np.int32)))

    # ------------------------------------------------------------------ gear 1 + 2 + flatten
    def load_draft(self, draft):
        """Copy one step's draft inputs into the device buffers."""
        if self.mode == L.MODE_TREE:
            self.d_parent.copy_(torch.as_tensor(np.asarray(draft["parent"], np.int32)))
            self.d_layer.copy_(torch.as_tensor(np.asarray(draft["layer"], np.int32)))
            self.d_score.copy_(torch.as_tensor(np.asarray(draft["logp"], np.float32)))
        else:
            self.d_score.copy_(torch.as_tensor(np.asarray(draft["conf"], np.float32)))
        self.d_tok.copy_(torch.as_tensor(np.asarray(draft["tok"], np.int32)))

    def check_draft(self, bufs=None):
        """graft_check_draft on a draft already on the device: per-request flag
        words (host int32 [B], 0 = every precondition holds).  Synchronises."""
        if bufs is None:
            bufs = {"parent": self.d_parent, "layer": self.d_layer, "score": self.d_score, "tok": self.d_tok}
        st = torch.empty(self.B, dtype=torch.int32, device=self.device)
        tree = self.mode == L.MODE_TREE
        L.graft_check_draft(self.B, self.Nd, self.mode, self.V, bufs["parent"].data_ptr() if tree else None,
                            bufs["layer"].data_ptr() if tree else None, bufs["score"].data_ptr(),
                            bufs["tok"].data_ptr(), st.data_ptr(), self.stream())
        return st.cpu().numpy()

    def check_tree(self):
        """graft_check_tree on the flattened tree of the last build (host int32 [B])."""
        st = torch.empty(self.B, dtype=torch.int32, device=self.device)
        L.graft_check_tree(self.B, self.T1, self.V, self.tok.data_ptr(), self.parent.data_ptr(),
                           self.depth.data_ptr(), st.data_ptr(), self.stream())
        return st.cpu().numpy()

    def _raise_if_bad(self, flags, what):
        bad = np.nonzero(flags)[0]
        if bad.size:
            names = [n for n, f in (("parent", L.BAD_PARENT), ("layer", L.BAD_LAYER), ("score", L.BAD_SCORE),
                                    ("token", L.BAD_TOKEN), ("depth", L.BAD_DEPTH)) if int(flags[bad[0]]) & f]
            raise ValueError("%s fails its preconditions for request(s) %s (first: %s)"
                             % (what, bad.tolist(), ", ".join(names)))

    def draft_buffers(self):
        """A fresh set of device draft buffers shaped like the pipeline's own."""
        return {"parent": torch.empty_like(self.d_parent), "layer": torch.empty_like(self.d_layer),
                "score": torch.empty_like(self.d_score), "tok": torch.empty_like(self.d_tok)}

    def build_device(self, bufs=None):
        """prune -> retrieve -> flatten on a draft already on the device (the
        pipeline's own buffers, or ``bufs`` from draft_buffers())."""
        s = self.stream()
        B, Nd, T1 = self.B, self.Nd, self.T1
        if bufs is None:
            bufs = {"parent": self.d_parent, "layer": self.d_layer, "score": self.d_score, "tok": self.d_tok}
        d_parent, d_layer, d_score, d_tok = bufs["parent"], bufs["layer"], bufs["score"], bufs["tok"]
        if self._calib is not None:
            self._record_stats(d_parent, d_layer, d_score)
        if self.fused:
            L.graft_build_hybrid_tree(
                B, Nd, T1, self.mode, self.layout, self.slots, self.cfg, self.tpl, self.V, self.k,
                self.table.data_ptr(), self.roots.data_ptr(), self.base_pos.data_ptr(), d_parent.data_ptr(),
                d_layer.data_ptr(), d_score.data_ptr(), d_tok.data_ptr(), self.stage.data_ptr(),
                self.n_keep.data_ptr(), self.keep.data_ptr(),
                self.cum.data_ptr() if self.mode == L.MODE_TREE else None, self.ret_tok.data_ptr(),
                self.ret_parent.data_ptr(), self.n_ret.data_ptr(), self.r_out, self.tok.data_ptr(),
                self.parent.data_ptr(), self.depth.data_ptr(), self.pos_id.data_ptr(), self.anc.data_ptr(),
                self._ptr(self.row_src), s)
            return
        L.graft_prune_select(B, Nd, self.mode, d_parent.data_ptr(), d_layer.data_ptr(),
                             d_score.data_ptr(), self.cfg, self.stage.data_ptr(),
                             self.n_keep.data_ptr(), self.keep.data_ptr(),
                             self.cum.data_ptr() if self.mode == L.MODE_TREE else None, s)
        L.graft_retrieve_expand(B, self.V, self.k, self.mode, self.slots, self.table.data_ptr(),
                                self.roots.data_ptr(), self.n_keep.data_ptr(), d_tok.data_ptr(),
                                Nd, self.tpl, self.cfg if self.mode == L.MODE_TREE else None,
                                self.ret_tok.data_ptr(), self.ret_parent.data_ptr(),
                                self.n_ret.data_ptr(), self.r_out, s)
        L.graft_build_tree_mask(B, Nd, T1, self.layout, self.roots.data_ptr(), self.base_pos.data_ptr(),
                                d_tok.data_ptr(), d_parent.data_ptr(), self.keep.data_ptr(),
                                self.n_keep.data_ptr(), self.ret_tok.data_ptr(),
                                self.ret_parent.data_ptr(), self.n_ret.data_ptr(), self.r_out,
                                self.tok.data_ptr(), self.parent.data_ptr(), self.depth.data_ptr(),
                                self.pos_id.data_ptr(), self.anc.data_ptr(), self._ptr(self.row_src), s)

    # ------------------------------------------------------------------ threshold calibration
    def begin_calibration(self, max_steps=64):
        """Record the checkpoint statistics of every tree built from now on (up to
        max_steps builds) for end_calibration()."""
        if self.mode != L.MODE_TREE:
            raise ValueError("threshold calibration applies to TREE pruning")
        self._calib = torch.full((max_steps * self.B, 3), float("nan"), dtype=torch.float32,
                                 device=self.device)
        self._calib_rows = 0

    def _record_stats(self, d_parent, d_layer, d_score):
        if self._calib_rows + self.B > self._calib.shape[0]:
            raise RuntimeError("more calibration steps than begin_calibration(max_steps) allows")
        out = self._calib[self._calib_rows:self._calib_rows + self.B]
        L.graft_checkpoint_stats(self.B, self.Nd, d_parent.data_ptr(), d_layer.data_ptr(), d_score.data_ptr(),
                                 self.cfg, out.data_ptr(), self.stream())
        self._calib_rows += self.B

    def calibration_samples(self):
        """The checkpoint statistics recorded so far (device fp32 [n, 3], NaN = not reached)."""
        return self._calib[:self._calib_rows]

    def end_calibration(self, q):
        """Set the checkpoint thresholds to the q-quantiles of the recorded
        statistics (graft_calibrate_thresholds); returns them (fp32 ln tau)."""
        thr = torch.empty(3, dtype=torch.float32, device=self.device)
        L.graft_calibrate_thresholds(self._calib_rows, self._calib.data_ptr(), q, thr.data_ptr(), self.stream())
        host = thr.cpu().numpy()
        for s in range(3):
            self.cfg.log_thr[s] = float(host[s])
        self._calib = None
        return host

    def retrieve_ahead(self):
        """Section 二: the retrieval tree from each root (the whole template)
        on the side stream, once the roots and the matrix of the last step are
        final; it needs no draft, so it runs while the draft is produced."""
        main = torch.cuda.current_stream(self.device)
        self._ev_inputs.record(main)
        self.side.wait_event(self._ev_inputs)
        L.graft_retrieve_expand(self.B, self.V, self.k, self.mode, self.slots, self.table.data_ptr(),
                                self.roots.data_ptr(), None, None, self.Nd, self.tpl, self.cfg,
                                self.ret_tok.data_ptr(), self.ret_parent.data_ptr(), self.n_ret.data_ptr(),
                                self.r_out, self.side.cuda_stream)
        self._ev_ret.record(self.side)

    def build_after_retrieval(self, bufs=None):
        """prune -> keep the first R retrieved nodes -> flatten, once the draft is
        on the device and retrieve_ahead() has finished (the stream waits)."""
        B, Nd, T1 = self.B, self.Nd, self.T1
        if bufs is None:
            bufs = {"parent": self.d_parent, "layer": self.d_layer, "score": self.d_score, "tok": self.d_tok}
        if self._calib is not None:
            self._record_stats(bufs["parent"], bufs["layer"], bufs["score"])
        main = torch.cuda.current_stream(self.device)
        main.wait_event(self._ev_ret)
        L.graft_build_after_retrieval(
            B, Nd, T1, self.layout, self.slots, self.cfg, self.roots.data_ptr(), self.base_pos.data_ptr(),
            bufs["parent"].data_ptr(), bufs["layer"].data_ptr(), bufs["score"].data_ptr(), bufs["tok"].data_ptr(),
            self.stage.data_ptr(), self.n_keep.data_ptr(), self.keep.data_ptr(), self.cum.data_ptr(),
            self.ret_tok.data_ptr(), self.ret_parent.data_ptr(), self.n_ret.data_ptr(), self.r_out,
            self.tok.data_ptr(), self.parent.data_ptr(), self.depth.data_ptr(), self.pos_id.data_ptr(),
            self.anc.data_ptr(), self._ptr(self.row_src), main.cuda_stream)

    def build(self, draft):
        if self.debug_checks:
            self.load_draft(draft)
            self._raise_if_bad(self.check_draft(), "draft tree")
        if self.overlap:
            self.retrieve_ahead()          # overlaps the draft's upload below
            self.load_draft(draft)
            self.build_after_retrieval()
        else:
            self.load_draft(draft)
            self.build_device()
        out = {"stage": self.stage, "n_keep": self.n_keep, "keep": self.keep, "ret_tok": self.ret_tok,
               "ret_parent": self.ret_parent, "n_ret": self.n_ret, "tok": self.tok, "parent": self.parent,
               "depth": self.depth, "pos_id": self.pos_id, "anc": self.anc}
        if self.mode == L.MODE_TREE:
            out["cum"] = self.cum
        if self.want_coverage:
            out["row_src"] = self.row_src
        return out

    @staticmethod
    def _ptr(t):
        return None if t is None else t.data_ptr()

    # ------------------------------------------------------------------ verify + update
    def verify_update_device(self, logits):
        """top-k -> accept -> matrix update for logits [B*T1, V] on the device."""
        s = self.stream()
        B, T1 = self.B, self.T1
        if self.fused:
            L.graft_verify_update(B, T1, self.V, self.k, self.dtype, logits.data_ptr(), self.tok.data_ptr(),
                                  self.parent.data_ptr(), self.depth.data_ptr(), self.table.data_ptr(),
                                  self.table_prob.data_ptr() if self.want_prob else None,
                                  self.topk.data_ptr(), self.topk_prob.data_ptr() if self.want_prob else None,
                                  self._ptr(self.row_stats), self.accept_len.data_ptr(),
                                  self.accept_idx.data_ptr(), self.dmax, self.roots.data_ptr(),
                                  self.base_pos.data_ptr(), self.ws.data_ptr(), self.ws_bytes, s)
            self._coverage(logits, s)
            return
        L.graft_verify_accept(B, T1, self.V, self.k, self.dtype, logits.data_ptr(), self.tok.data_ptr(),
                              self.parent.data_ptr(), self.depth.data_ptr(), self.topk.data_ptr(),
                              self.topk_prob.data_ptr() if self.want_prob else None,
                              self._ptr(self.row_stats), self.accept_len.data_ptr(),
                              self.accept_idx.data_ptr(), self.dmax, self.roots.data_ptr(),
                              self.base_pos.data_ptr(), self.ws.data_ptr(), self.ws_bytes, s)
        self._coverage(logits, s)
        L.graft_update_topk(B * T1, self.V, self.k, self.dtype, None, self.topk.data_ptr(),
                            self.topk_prob.data_ptr() if self.want_prob else None, self.tok.data_ptr(),
                            self.table.data_ptr(), self.table_prob.data_ptr() if self.want_prob else None,
                            None, None, 0, s)

    def _coverage(self, logits, s):
        if not self.want_coverage:
            return
        L.graft_coverage_gain(self.B, self.T1, self.V, self.dtype, logits.data_ptr(), self.tok.data_ptr(),
                              self.parent.data_ptr(), self.row_src.data_ptr(), self.row_stats.data_ptr(),
                              self.gain.data_ptr(), s)

    def raise_if_gave_up(self):
        """accept_len == -1 marks a request whose coordinator gave up waiting for
        its rows (about a second; never in normal operation).  The step's outputs
        are then invalid and rows that finished late may have left words in the
        workspace, so once the launch has drained the workspace is zero-filled
        again and an error is raised.  Synchronises."""
        al = self.accept_len.cpu().numpy()
        bad = np.nonzero(al < 0)[0]
        if bad.size:
            torch.cuda.synchronize(self.device)
            self.ws.zero_()
            torch.cuda.synchronize(self.device)
            raise RuntimeError("verification gave up waiting for the rows of request(s) %s; "
                               "the workspace was reset" % bad.tolist())

    def verify_update(self, logits, check=True):
        self._check_logits(logits, self.B * self.T1)
        self.verify_update_device(logits)
        if check:
            self.raise_if_gave_up()
        out = {"accept_len": self.accept_len, "accept_idx": self.accept_idx, "bonus": self.roots.clone(),
               "topk": self.topk, "base_pos": self.base_pos}
        if self.want_prob:
            out["topk_prob"] = self.topk_prob
        if self.want_coverage:
            out["coverage"] = self.gain
            out["row_stats"] = self.row_stats
        return out

    # ------------------------------------------------------------------ prompt ingest
    def ingest_chunk(self, row_tok, logits):
        """table[row_tok[p]] <- top-k(logits[p]) for the rows in order; returns the
        chunk's top-k rows (device)."""
        n = int(logits.shape[0])
        self._check_logits(logits, n)
        rt = torch.as_tensor(np.asarray(row_tok, np.int32)).to(self.device)
        need = L.graft_workspace_bytes(n, self.V, self.k, self.dtype)
        if self._ingest_ws is None or self._ingest_ws.numel() < need:
            self._ingest_ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
        out = torch.empty(n, self.k, dtype=torch.int32, device=self.device)
        L.graft_update_topk(n, self.V, self.k, self.dtype, logits.data_ptr(), None, None, rt.data_ptr(),
                            self.table.data_ptr(), self.table_prob.data_ptr() if self.want_prob else None,
                            out.data_ptr(), self._ingest_ws.data_ptr(), self._ingest_ws.numel(),
                            self.stream())
        return out

    def _check_logits(self, logits, n_rows):
        want = torch.bfloat16 if self.dtype == L.DTYPE_BF16 else torch.float32
        if logits.dtype != want or not logits.is_contiguous() or logits.device != self.device:
            raise ValueError("logits must be a contiguous %s tensor on %s" % (want, self.device))
        if logits.numel() != n_rows * self.V:
            raise ValueError("logits must hold %d rows of %d" % (n_rows, self.V))
