"""Backend adapters that plug the CPU oracle and the HIP path into
synth.runner.  Test infrastructure."""
from __future__ import annotations

import numpy as np

from synth import generators as G


class OracleBackend:
    def __init__(self, cfg, want_prob=False, want_coverage=False):
        from oracle.driver import OracleGraft
        self.o = OracleGraft(cfg)
        self.cfg = cfg
        self.want_prob = want_prob
        self.want_coverage = want_coverage

    def set_roots(self, roots, base_pos):
        self.o.set_roots(roots, base_pos)

    def get_roots(self):
        return self.o.get_roots()

    def get_table(self):
        return self.o.get_table()

    def build(self, draft):
        return self.o.build(draft)

    def materialize(self, pool, desc):
        # one host buffer reused across steps (a fresh one per step would page-fault
        # hundreds of MB each time at the full shapes)
        buf = getattr(self, "_rows", None)
        rows = G.materialize_rows_np(pool, desc, out=buf)
        if buf is None or rows.base is not buf:
            self._rows = rows if rows.base is None else rows.base
        return rows if self.cfg.dtype == "bf16" else rows.view(np.float32)

    def verify_update(self, rows):
        return self.o.verify_update(rows, want_prob=self.want_prob, want_coverage=self.want_coverage)

    def ingest_chunk(self, row_tok, rows):
        return self.o.ingest_chunk(row_tok, rows)

    def begin_calibration(self):
        self.o.begin_calibration()

    def end_calibration(self, q):
        return self.o.end_calibration(q)


class HipBackend:
    """HIP path through the C-ABI; host copies of the small outputs are made for
    the synthetic generator and for comparison."""

    def __init__(self, cfg, want_prob=False, device="cuda", fused=True, want_coverage=False, overlap=False):
        import torch
        from hybrid_draft_tree_amd.driver import GraftPipeline
        from synth.device import DeviceRows
        self.torch = torch
        self.cfg = cfg
        self.p = GraftPipeline.from_config(cfg, want_prob=want_prob, want_coverage=want_coverage,
                                           device=device, fused=fused, overlap=overlap)
        self.rows = None
        self._DeviceRows = DeviceRows
        self.want_prob = want_prob

    def set_roots(self, roots, base_pos):
        self.p.set_roots(roots, base_pos)

    def get_roots(self):
        return self.p.roots.cpu().numpy()

    def get_table(self):
        return self.p.table.cpu().numpy()

    def build(self, draft):
        out = self.p.build(draft)
        return {k: v.cpu().numpy() for k, v in out.items()}

    def materialize(self, pool, desc):
        if self.rows is None or self.rows.pool is not pool:
            self.rows = self._DeviceRows(pool, self.p.device)
        return self.rows.materialize(desc)

    def verify_update(self, rows):
        out = self.p.verify_update(rows)
        return {k: v.cpu().numpy() for k, v in out.items()}

    def ingest_chunk(self, row_tok, rows):
        return self.p.ingest_chunk(row_tok, rows)

    def begin_calibration(self):
        self.p.begin_calibration()

    def end_calibration(self, q):
        return self.p.end_calibration(q)
