"""Pins of the pruning variants behind the ablations of the news write-up's
section 五 and the per-node static-slot replacement of section 四: a fixed
draft/retrieval split (a checkpoint that always fires), no retrieval (an empty
template), and a per-node confidence threshold.  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pins import TOPO, _tree_batch, _stage_logps


def _cum(par, lp):
    cum = np.zeros(len(par), np.float32)
    for i in range(len(par)):
        cum[i] = np.float32((0.0 if par[i] < 0 else cum[par[i]]) + np.float32(lp[i]))
    return cum


def test_per_node_closed_form_half_probabilities():
    par, lay, _ = TOPO
    lp = np.full((1, 60), np.float32(math.log(0.5)))
    r = O.prune_tree(par[None], lay[None], lp, node_tau=0.3)
    # depth-1 nodes: ln 0.5 = -0.69 >= ln 0.3 = -1.20; depth 2: -1.39 < -1.20
    np.testing.assert_array_equal(r["keep"][0], (lay == 0).astype(np.uint8))
    assert r["n_keep"][0] == 8 and r["stage"][0] == 4
    r = O.prune_tree(par[None], lay[None], lp, node_tau=1e-30)
    assert r["n_keep"][0] == 60 and r["stage"][0] == 3


def test_per_node_keeps_exactly_the_nodes_at_or_above_the_threshold():
    rng = np.random.default_rng(9)
    par, lay, _ = TOPO
    B = 40
    lp = np.log(rng.uniform(0.05, 1.0, size=(B, 60))).astype(np.float32)
    for tau in (0.05, 0.2, 0.5):
        r = O.prune_tree(np.tile(par, (B, 1)), np.tile(lay, (B, 1)), lp, node_tau=tau)
        thr = np.float32(math.log(tau))
        for b in range(B):
            want = _cum(par, lp[b]) >= thr
            np.testing.assert_array_equal(r["keep"][b].astype(bool), want)
            kept = np.nonzero(want)[0]
            assert all(par[i] < 0 or want[par[i]] for i in kept)     # ancestor-closed
            assert r["n_keep"][b] == want.sum()


@pytest.mark.parametrize("tau,stage,n", [((math.inf, 0, 0), 0, 8), ((0, math.inf, 0), 1, 24),
                                         ((0, 0, math.inf), 2, 40), ((0, 0, 0), 3, 60)])
def test_fixed_split_through_always_or_never_firing_checkpoints(tau, stage, n):
    par_b, lay_b, lp = _tree_batch(_stage_logps())
    r = O.prune_tree(par_b, lay_b, lp, tau=tau)
    assert (r["stage"] == stage).all() and (r["n_keep"] == n).all()


def test_no_retrieval_template_leaves_the_freed_slots_empty():
    par_b, lay_b, lp = _tree_batch(_stage_logps())
    B = par_b.shape[0]
    rng = np.random.default_rng(2)
    V = 100
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    pr = O.prune_tree(par_b, lay_b, lp)
    empty = {k: np.zeros(0, np.int32) for k in ("parent", "rank", "depth")}
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, empty, Rmax_out=1)
    assert (ret["n_ret"] == 0).all()
    fl = O.flatten("in_place", 61, roots, np.zeros(B, np.int32), rng.integers(0, V, size=(B, 60)).astype(np.int32),
                   par_b, pr["keep"], pr["n_keep"], ret)
    np.testing.assert_array_equal((fl["row_src"] == O.ROW_EMPTY).sum(1), 60 - pr["n_keep"])
