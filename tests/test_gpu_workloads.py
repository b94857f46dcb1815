"""End-to-end lockstep parity on the five synthetic workloads.  The oracle and
the HIP path each run their own trajectory (their own roots, matrix and
committed stream) through the same seeded generators; every per-step output and
the whole continuation matrix must agree bit for bit after every step.

Default sizes keep each case to seconds; the full-size cases run a few steps at
the real shapes (B=16, V=151936) and check the prompt ingest at 32768 rows on
sampled matrix rows."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from synth import WORKLOADS  # noqa: E402
from synth import generators as G  # noqa: E402
from synth import runner as R  # noqa: E402
from tests.backends import HipBackend, OracleBackend  # noqa: E402

pytestmark = pytest.mark.gpu

KEYS_BUILD = ("stage", "n_keep", "keep", "n_ret", "ret_tok", "tok", "parent", "depth", "pos_id", "anc")
KEYS_VERIFY = ("topk", "accept_len", "accept_idx", "bonus")


def _compare_runs(cfg, n_steps, warmup, table_every=1, fused=True, want_prob=False, overlap=False):
    ob = OracleBackend(cfg, want_prob=want_prob)
    hb = HipBackend(cfg, want_prob=want_prob, fused=fused, overlap=overlap)
    wl_o, wl_h = R.Workload(cfg), R.Workload(cfg, pool=None)
    R.start(ob, wl_o)
    R.start(hb, wl_h)
    np.testing.assert_array_equal(hb.get_table(), ob.get_table())
    np.testing.assert_array_equal(hb.get_roots(), ob.get_roots())
    stats = {"accepted": 0, "stages": set()}
    calib = bool(cfg.calib_q) and cfg.mode == "tree"
    if calib:
        ob.begin_calibration()
        hb.begin_calibration()
    for s in range(warmup + n_steps):
        if calib and s == warmup:
            to, th = ob.end_calibration(cfg.calib_q), hb.end_calibration(cfg.calib_q)
            np.testing.assert_array_equal(th, to, err_msg="calibrated thresholds")
            stats["log_thr"] = to
        off = G.WARMUP_STREAM_OFFSET if s < warmup else 0
        idx = s if s < warmup else s - warmup
        fo, ro = R.step(ob, wl_o, idx, off)
        fh, rh = R.step(hb, wl_h, idx, off)
        for k in KEYS_BUILD:
            if k in fo:
                a, b = np.asarray(fh[k]), np.asarray(fo[k])
                if k == "anc":
                    a = a.view(np.uint64)
                if k == "ret_tok":
                    a, b = a[:, : b.shape[1]], b
                np.testing.assert_array_equal(a, b, err_msg="step %d %s" % (s, k))
        if cfg.mode == "tree":
            np.testing.assert_array_equal(fh["cum"].view(np.uint32), fo["cum"].view(np.uint32))
        for k in KEYS_VERIFY:
            np.testing.assert_array_equal(np.asarray(rh[k]), np.asarray(ro[k]), err_msg="step %d %s" % (s, k))
        if (s + 1) % table_every == 0 or s == warmup + n_steps - 1:
            np.testing.assert_array_equal(hb.get_table(), ob.get_table(), err_msg="table after step %d" % s)
        stats["accepted"] += int(np.asarray(ro["accept_len"]).sum())
        if cfg.mode == "tree":
            stats["stages"].update(np.asarray(fo["stage"]).tolist())
    return stats


def _small(cfg_id, **kw):
    cfg = WORKLOADS[cfg_id]
    d = dict(noise_pool_rows=16)
    d.update(kw)
    return cfg.scaled(**d)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "five_calls"])
@pytest.mark.parametrize("cfg_id,kw,steps", [
    (1, {}, 60),                                   # toy, full V=32000 fp32
    (2, {}, 30),                                   # V=128256 bf16, B=1
    (3, {"V": 20000, "B": 16}, 12),                # in-place layout, batch collisions
    (5, {"V": 20000}, 20),                         # TAIL
])
def test_lockstep_reduced(cfg_id, kw, steps, fused):
    cfg = _small(cfg_id, **kw)
    st = _compare_runs(cfg, steps, warmup=cfg.warmup_steps, fused=fused)
    assert st["accepted"] > 0
    if cfg.mode == "tree":
        assert len(st["stages"]) >= 2


def test_lockstep_with_probabilities():
    """Probability outputs (fused softmax statistics) through whole steps: the
    matrix's probability table and every top-k probability within 1e-5 relative."""
    cfg = _small(3, V=30000, B=4)
    ob, hb = OracleBackend(cfg, want_prob=True), HipBackend(cfg, want_prob=True)
    wo, wh = R.Workload(cfg), R.Workload(cfg)
    R.start(ob, wo)
    R.start(hb, wh)
    for s in range(4):
        fo, ro = R.step(ob, wo, s)
        fh, rh = R.step(hb, wh, s)
        np.testing.assert_array_equal(rh["topk"], ro["topk"])
        np.testing.assert_allclose(rh["topk_prob"], ro["topk_prob"], rtol=1e-5, atol=0)
    np.testing.assert_array_equal(hb.get_table(), ob.get_table())
    tp_h = hb.p.table_prob.cpu().numpy()
    np.testing.assert_allclose(tp_h, ob.o.table_prob, rtol=1e-5, atol=0)


@pytest.mark.parametrize("cfg_id,kw", [
    (2, {"tpl_kind": "branching", "tpl_beta": (1, 1)}),
    (3, {"V": 20000, "B": 8, "tpl_kind": "branching", "tpl_beta": (2, 1), "tpl_depth": 10}),
    (2, {"tpl_depth": 3}),                                   # 24-node chains: empty slots every step
], ids=["cfg2_branching", "cfg3_branching_deep", "cfg2_short_chains"])
def test_lockstep_templates(cfg_id, kw):
    cfg = _small(cfg_id, **kw)
    st = _compare_runs(cfg, 15, warmup=cfg.warmup_steps)
    assert st["accepted"] > 0


@pytest.mark.parametrize("kw", [
    {"node_tau": 0.15},                         # per-node static-slot replacement
    {"tpl_kind": "none"},                       # pruning without retrieval: empty slots
    {"tau": (0.0, 0.0, float("inf"))},          # fixed 40/20 draft/retrieval split
], ids=["per_node", "no_retrieval", "fixed_split"])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "five_calls"])
def test_lockstep_ablation_variants(kw, fused):
    cfg = _small(3, V=20000, B=8, **kw)
    st = _compare_runs(cfg, 10, warmup=cfg.warmup_steps, fused=fused)
    assert st["accepted"] > 0


@pytest.mark.parametrize("cfg_id,kw", [(3, {"V": 20000, "B": 16}), (1, {}), (3, {"V": 20000, "B": 8,
                                                                                 "calib_q": (0.1, 0.4, 0.9)})])
def test_lockstep_retrieval_ahead_of_the_draft(cfg_id, kw):
    """Retrieval on a side stream before the draft is loaded, then prune +
    flatten (graft_build_after_retrieval): every output as the oracle's."""
    cfg = _small(cfg_id, **kw)
    st = _compare_runs(cfg, 12, warmup=cfg.warmup_steps, overlap=True)
    assert st["accepted"] > 0 and len(st["stages"]) >= 2


@pytest.mark.parametrize("q", [(0.2, 0.2, 0.2), (0.5, 0.3, 0.1)])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "five_calls"])
def test_lockstep_calibrated_thresholds(q, fused):
    """Thresholds calibrated on the warm-up steps (each side its own statistics
    and quantiles) agree bit for bit, and the later steps prune with them."""
    cfg = _small(3, V=20000, B=16, calib_q=q)
    st = _compare_runs(cfg, 10, warmup=cfg.warmup_steps, fused=fused)
    assert st["accepted"] > 0 and np.isfinite(st["log_thr"]).all()
    assert len(st["stages"]) >= 2


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "five_calls"])
def test_lockstep_coverage_gain(fused):
    """The coverage-gain diagnostic through whole steps (row sources from the
    build, softmax statistics from the verify launch): within 1e-5 relative of
    the oracle's fp64 gain every step, exactly 0 where nothing was retrieved."""
    cfg = _small(3, V=30000, B=8)
    ob, hb = OracleBackend(cfg, want_coverage=True), HipBackend(cfg, want_coverage=True, fused=fused)
    wo, wh = R.Workload(cfg), R.Workload(cfg)
    R.start(ob, wo)
    R.start(hb, wh)
    seen_pos = seen_zero = False
    for s in range(cfg.warmup_steps + 6):
        off = G.WARMUP_STREAM_OFFSET if s < cfg.warmup_steps else 0
        idx = s if s < cfg.warmup_steps else s - cfg.warmup_steps
        fo, ro = R.step(ob, wo, idx, off)
        fh, rh = R.step(hb, wh, idx, off)
        np.testing.assert_array_equal(fh["row_src"], fo["row_src"], err_msg="step %d" % s)
        np.testing.assert_array_equal(rh["topk"], ro["topk"])
        np.testing.assert_allclose(rh["coverage"], ro["coverage"], rtol=1e-5, atol=0, err_msg="step %d" % s)
        seen_pos |= bool((ro["coverage"] > 0).any())
        seen_zero |= bool((np.asarray(fo["n_ret"]) == 0).any())
        assert (ro["coverage"][np.asarray(fo["n_ret"]) == 0] == 0).all()
    assert seen_pos
    np.testing.assert_array_equal(hb.get_table(), ob.get_table())


def test_lockstep_ingest_reduced():
    cfg = _small(4, V=30000, prompt_len=5000, ingest_chunk=1024)
    st = _compare_runs(cfg, 10, warmup=0)
    assert st["accepted"] > 0


def test_lockstep_longctx_full_vocab():
    """Workload 4 at its real vocabulary and batch (V=151936, B=4: 244 split rows
    per step) after an 8192-token prompt ingested in four 2048-row chunks (tokens
    repeated across chunks: the last position wins): every output and the full
    matrix."""
    cfg = _small(4, prompt_len=8192)
    st = _compare_runs(cfg, 12, warmup=0, table_every=4)
    assert st["accepted"] > 0


@pytest.mark.parametrize("cfg_id,steps", [(3, 3), (5, 3), (2, 20)])
def test_lockstep_full_size(cfg_id, steps):
    """Real shapes (B=16, V=151936, 61 or 17 rows per request; B=1, V=128256):
    every output and the full matrix, for a few steps after warm-up."""
    cfg = WORKLOADS[cfg_id]
    st = _compare_runs(cfg, steps, warmup=2, table_every=steps + 2)
    assert st["accepted"] > 0


def test_full_config1_500_steps():
    """Workload 1 end to end at its full length (500 steps after 5 warm-up steps)."""
    cfg = WORKLOADS[1]
    if os.environ.get("GRAFT_QUICK"):
        pytest.skip("quick mode")
    st = _compare_runs(cfg, cfg.steps, warmup=cfg.warmup_steps, table_every=50)
    assert st["accepted"] > cfg.steps


def test_ingest_full_size_sampled():
    """The full 32768-row prompt ingest (16 chunks of 2048 x 151936 bf16) on the
    GPU; matrix rows and the first root checked against the oracle on a sample
    of prompt tokens (each row's expected value is the top-k of the last prompt
    row holding that token)."""
    cfg = WORKLOADS[4]
    hb = HipBackend(cfg)
    wl = R.Workload(cfg)
    R.start(hb, wl)
    tab = hb.get_table()
    prompt = wl.prompt
    last = {}
    for p, x in enumerate(prompt):
        last[int(x)] = p
    descs = list(wl.ingest_descs())
    rng = np.random.default_rng(0)
    sample = rng.choice(sorted(last), size=48, replace=False).tolist()
    # most frequent tokens (collisions across chunks) too
    vals, cnt = np.unique(prompt, return_counts=True)
    sample += vals[np.argsort(-cnt)[:16]].tolist()
    for x in sample:
        p = last[int(x)]
        c = p // cfg.ingest_chunk
        c0, c1, desc = descs[c]
        one = {k: v[p - c0: p - c0 + 1] for k, v in desc.items()}
        row = G.materialize_rows_np(wl.pool, one)
        np.testing.assert_array_equal(tab[int(x)], O.topk(row, cfg.k, "bf16")[0], err_msg="token %d" % x)
    c0, c1, desc = descs[-1]
    one = {k: v[-1:] for k, v in desc.items()}
    g_last = O.topk(G.materialize_rows_np(wl.pool, one), 1, "bf16")[0, 0]
    assert (hb.get_roots() == g_last).all()
    untouched = np.setdiff1d(np.arange(cfg.V), prompt)[:100]
    np.testing.assert_array_equal(tab[untouched], np.tile(np.arange(8), (len(untouched), 1)))
