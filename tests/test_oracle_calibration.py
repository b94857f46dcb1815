"""Pins of threshold calibration (news write-up, section 二: a few warm-up rounds
show how confident the drafter is at each checkpoint, and the thresholds are
set from that spread).  The statistic is the one each checkpoint compares; the
threshold is a quantile of it.  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pins import TOPO, _stage_logps, _tree_batch

CK, KEEP = (0, 1, 5), (8, 24, 40)


def test_stats_closed_form_half_probabilities():
    par, lay, _ = TOPO
    lp = np.full((1, 60), np.float32(math.log(0.5)))
    st = O.checkpoint_stats(par[None], lay[None], lp, CK, KEEP)[0]
    # every node on layer c has confidence 0.5^(c+1)
    for s, c in enumerate(CK):
        assert st[s] == pytest.approx((c + 1) * math.log(0.5), rel=1e-6)


def test_unreached_checkpoints_are_nan():
    par, lay, _ = TOPO
    lp = np.full((1, 60), np.float32(-0.1))
    # layer 5 does not exist in a tree cut after layer 3; keep 30 > 24 nodes up to layer 1
    shallow = lay <= 3
    n = int(shallow.sum())
    st = O.checkpoint_stats(par[None, :n], lay[None, :n], lp[:, :n], CK, (8, 30, 40))[0]
    assert not np.isnan(st[0]) and np.isnan(st[1]) and np.isnan(st[2])


def _path_best(par, lay, lp, c):
    """Brute force: walk every layer-c node's path from the root and sum in order."""
    best = None
    for i in np.nonzero(lay == c)[0]:
        path = []
        j = int(i)
        while j >= 0:
            path.append(j)
            j = int(par[j])
        acc = np.float32(0.0)
        for j in reversed(path):
            acc = np.float32(acc + lp[j])
        best = acc if best is None else max(best, acc)
    return best


def test_stats_match_path_walks_and_decide_the_stage():
    rng = np.random.default_rng(11)
    par, lay, _ = TOPO
    B = 30
    lp = np.log(rng.uniform(0.02, 1.0, size=(B, 60))).astype(np.float32)
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    st = O.checkpoint_stats(P, Ly, lp, CK, KEEP)
    for b in range(B):
        for s, c in enumerate(CK):
            assert st[b, s] == _path_best(par, lay, lp[b], c)
    # the checkpoint that fires is the first whose statistic is below its threshold
    for tau in [(0.3, 0.2, 0.1), (0.6, 0.3, 0.05), (0.9, 0.9, 0.9)]:
        lt = O.log_thresholds(tau)
        stage = O.prune_tree(P, Ly, lp, CK, tau, KEEP)["stage"]
        want = [next((s for s in range(3) if st[b, s] < lt[s]), 3) for b in range(B)]
        np.testing.assert_array_equal(stage, want)
    # the staged trees of the prune pins cross each threshold where they are built to
    par_b, lay_b, lp_b = _tree_batch(_stage_logps())
    st_b = O.checkpoint_stats(par_b, lay_b, lp_b, CK, KEEP)
    lt = O.log_thresholds((0.3, 0.2, 0.1))
    assert st_b[0, 0] < lt[0] and st_b[1, 1] < lt[1] and st_b[2, 2] < lt[2]


@pytest.mark.parametrize("n", [1, 2, 7, 80, 1000])
def test_quantile_matches_numpy_inverted_cdf(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((n, 3)).astype(np.float32)
    x[rng.random((n, 3)) < 0.2] = np.nan
    for q in (1e-6, 0.1, 0.2, 0.25, 0.5, 0.9, 1.0):
        thr = O.calibrate(x, (q, q, q))
        for s in range(3):
            v = x[:, s][~np.isnan(x[:, s])]
            qf = float(np.float32(q))   # the quantile level is an fp32 value
            want = -np.inf if v.size == 0 else np.quantile(v.astype(np.float64), qf, method="inverted_cdf")
            assert thr[s] == np.float32(want)


def test_quantile_fire_share_on_distinct_samples():
    rng = np.random.default_rng(3)
    m = 97
    x = rng.permutation(np.arange(m, dtype=np.float32) - 50.0)
    S = np.stack([x, -x, x * 0.5], 1)
    for q in (0.01, 0.1, 0.3, 0.5, 0.99, 1.0):
        thr = O.calibrate(S, (q, q, q))
        for s in range(3):
            assert (S[:, s] < thr[s]).sum() == math.ceil(float(np.float32(q)) * m) - 1


def test_quantile_special_cases():
    const = np.full((40, 3), np.float32(-1.25))
    np.testing.assert_array_equal(O.calibrate(const, (0.2, 0.5, 1.0)), [-1.25] * 3)   # never fires
    x = np.array([[3.0, -2.0, np.nan], [-7.0, np.inf, np.nan], [1.0, -np.inf, np.nan]], np.float32)
    np.testing.assert_array_equal(O.calibrate(x, (1.0, 1e-9, 0.5)), [3.0, -np.inf, -np.inf])
    np.testing.assert_array_equal(O.calibrate(x, (0.0, 1.0, 1.0)), [-np.inf, np.inf, -np.inf])
    np.testing.assert_array_equal(O.calibrate(np.zeros((0, 3), np.float32), (0.5, 0.5, 0.5)), [-np.inf] * 3)
    for bad in [(1.5, 0.5, 0.5), (-0.1, 0.5, 0.5), (0.5, np.nan, 0.5)]:
        with pytest.raises(RuntimeError):
            O.calibrate(x, bad)


def test_calibrated_run_uses_the_quantile_thresholds():
    """OracleGraft: the thresholds after warm-up are the quantiles of what the
    warm-up drafts showed, and later steps prune with them."""
    from synth import WORKLOADS
    from synth import runner as R
    from tests.backends import OracleBackend

    cfg = WORKLOADS[1].scaled(calib_q=(0.5, 0.5, 0.5))
    be = OracleBackend(cfg)
    drafts = []
    orig = be.o.build

    def build(draft):
        drafts.append(draft)
        return orig(draft)

    be.build = build
    wl = R.Workload(cfg)
    R.start(be, wl)
    thr = R.warm_up(be, wl, cfg.warmup_steps)
    assert len(drafts) == cfg.warmup_steps
    seen = [O.checkpoint_stats(d["parent"], d["layer"], d["logp"], CK, KEEP) for d in drafts]
    np.testing.assert_array_equal(thr, O.calibrate(np.concatenate(seen), cfg.calib_q))
    for s in range(4):
        flat, _ = R.step(be, wl, s)
        d = drafts[-1]
        want = O.prune_tree(d["parent"], d["layer"], d["logp"], CK, keep=KEEP, log_thr=thr)
        np.testing.assert_array_equal(flat["stage"], want["stage"])
        np.testing.assert_array_equal(flat["keep"], want["keep"])
