"""Workload definitions for the five seeded synthetic Graft workloads.

These are plain configuration records (sizes, thresholds, seeds).  They hold
none of the method's arithmetic; both the CPU oracle and the HIP path read
them through the generators in this package.

Sources (arXiv 2605.20104 news write-up, "Graft ... three gears" section):
* 60 verification slots, splits 8/52, 24/36, 40/20, none -> no retrieval.
* checkpoints at draft depths 0, 1 and 5.
* retrieval template depth 8, width 8 (ablation section).
* 16-token DFlash blocks for the TAIL variant (block-draft section).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class GraftConfig:
    name: str
    cfg_id: int
    V: int                     # vocabulary size (rows of the continuation matrix)
    B: int                     # requests per step
    steps: int                 # decode steps of the full workload
    dtype: str = "bf16"        # target-logit dtype: "bf16" | "f32"
    k: int = 8                 # successors per matrix row
    slots: int = 60            # candidate verification slots per request (root excluded)
    mode: str = "tree"         # "tree" | "tail"
    layout: str = "compact"    # "compact" | "in_place" | "chain"
    layer_sizes: tuple = (8, 16, 12, 10, 8, 6)   # static draft tree, 60 nodes, depth 6
    tree_width: int = 8
    draft_sigma: float = 1.5
    draft_hit: float = 0.9
    tau: tuple = (0.3, 0.2, 0.1)
    ckpt_layers: tuple = (0, 1, 5)
    keep: tuple = (8, 24, 40)
    tpl_width: int = 8
    tpl_depth: int = 8
    tpl_kind: str = "chain"          # "chain" (rank chains), "branching", or "none" (no retrieval)
    tpl_beta: tuple = (1, 1)         # branching: rank charge num/den
    node_tau: float = 0.0            # > 0: per-node pruning threshold instead of the checkpoints
    calib_q: tuple = ()              # (q0, q1, q2): thresholds from warm-up quantiles instead of tau
    tail_block: int = 16
    tail_thr: float = 0.5
    warmup_steps: int = 5
    bump: float = 6.0
    noise_pool_rows: int = 64
    hot_frac: float = 0.30
    n_hot: int = 256
    init_base_pos: int = 127
    # config 4 only
    prompt_len: int = 0
    ingest_chunk: int = 2048
    ident_vocab: int = 4096
    span_len: int = 64
    span_frac: float = 0.35
    # config 2 only
    zipf_s: float = 1.1
    copy_frac: float = 0.2
    extra: dict = field(default_factory=dict)

    @property
    def rows_per_request(self) -> int:
        """Verified rows per request: the root plus every candidate slot."""
        return (self.tail_block if self.mode == "tail" else self.slots) + 1

    @property
    def n_draft(self) -> int:
        return self.tail_block if self.mode == "tail" else sum(self.layer_sizes)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def logits_bytes_per_step(self) -> int:
        return self.B * self.rows_per_request * self.V * self.elem_bytes

    def scaled(self, **kw) -> "GraftConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return GraftConfig(**d)


WORKLOADS = {
    1: GraftConfig(name="toy_v32000_f32", cfg_id=1, V=32000, B=1, steps=500, dtype="f32",
                   layout="compact"),
    2: GraftConfig(name="llama8b_v128256_b1", cfg_id=2, V=128256, B=1, steps=2000,
                   layout="compact"),
    3: GraftConfig(name="qwen8b_v151936_b16_static_slots", cfg_id=3, V=151936, B=16,
                   steps=1000, layout="in_place"),
    4: GraftConfig(name="longctx_ingest32768_v151936_b4", cfg_id=4, V=151936, B=4, steps=1000,
                   layout="compact", prompt_len=32768),
    5: GraftConfig(name="tail_block16_v151936_b16", cfg_id=5, V=151936, B=16, steps=2000,
                   mode="tail", layout="chain"),
}


def get(cfg_id: int) -> GraftConfig:
    return WORKLOADS[cfg_id]
