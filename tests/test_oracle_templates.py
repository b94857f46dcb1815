"""Pins of the branching retrieval template (the asymmetric shape of the news
write-up's section 二, gear 2: better-ranked successors get more children and
reach deeper) and of flattening with fewer retrieved nodes than freed slots.
CPU only."""
import itertools

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pins import _tree_batch, _stage_logps


def _as_paths(t):
    """Rank path of every node from the (parent, rank) arrays."""
    paths = []
    for p, r in zip(t["parent"], t["rank"]):
        paths.append((paths[p] if p >= 0 else ()) + (int(r),))
    return paths


def test_hand_order_w2_d3_beta1():
    # costs d + sum(ranks); ties by depth, then ranks lexicographically
    want = [(0,), (1,), (0, 0), (0, 1), (1, 0), (0, 0, 0), (1, 1), (0, 0, 1), (0, 1, 0), (1, 0, 0),
            (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, 1)]
    t = O.template_branching(2, 3, (1, 1), 64)
    assert _as_paths(t) == want
    np.testing.assert_array_equal(t["depth"], [len(p) for p in want])


@pytest.mark.parametrize("W,D,beta", [(2, 4, (1, 1)), (3, 3, (1, 2)), (4, 3, (3, 1)), (3, 4, (0, 1)),
                                      (5, 2, (2, 3)), (2, 6, (5, 1))])
def test_matches_sorted_enumeration(W, D, beta):
    num, den = beta
    allp = [p for d in range(1, D + 1) for p in itertools.product(range(W), repeat=d)]
    allp.sort(key=lambda p: (len(p) * den + num * sum(p), len(p), p))
    R = min(64, len(allp))
    t = O.template_branching(W, D, beta, R)
    assert _as_paths(t) == allp[:R]


def test_beta_zero_is_breadth_first():
    t = O.template_branching(3, 3, (0, 1), 39)
    want = [p for d in range(1, 4) for p in itertools.product(range(3), repeat=d)]
    assert _as_paths(t) == want


@pytest.mark.parametrize("W,D,beta,R", [(8, 8, (1, 1), 52), (8, 12, (2, 1), 64), (4, 5, (1, 2), 36)])
def test_structure(W, D, beta, R):
    t = O.template_branching(W, D, beta, R)
    n = len(t["parent"])
    assert n == R
    par, rk, dep = t["parent"], t["rank"], t["depth"]
    for i in range(n):
        assert par[i] < i                                  # topological: every prefix is a tree
        assert dep[i] == (1 if par[i] < 0 else dep[par[i]] + 1)
        assert 0 <= rk[i] < W and dep[i] <= D
    # siblings appear in rank order (a worse rank never precedes a better one)
    for i in range(n):
        sib = [j for j in range(n) if par[j] == par[i]]
        assert [rk[j] for j in sib] == sorted(rk[j] for j in sib)


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_flatten_with_a_small_template_leaves_empty_rows(layout):
    rng = np.random.default_rng(5)
    par_b, lay_b, lp = _tree_batch(_stage_logps())
    B = par_b.shape[0]
    V = 300
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    base = rng.integers(0, 100, size=B).astype(np.int32)
    pr = O.prune_tree(par_b, lay_b, lp)
    tpl = O.template_branching(8, 2, (1, 1), 20)          # 20 nodes: fewer than 52 / 36 freed slots
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, tpl)
    np.testing.assert_array_equal(ret["n_ret"], np.minimum(60 - pr["n_keep"], 20))
    fl = O.flatten(layout, 61, roots, base, d_tok, par_b, pr["keep"], pr["n_keep"], ret)
    src = fl["row_src"]
    empty = src == O.ROW_EMPTY
    np.testing.assert_array_equal(empty.sum(1), 60 - pr["n_keep"] - ret["n_ret"])
    assert (fl["tok"][empty] == -1).all() and (fl["parent"][empty] == -1).all()
    assert (fl["depth"][empty] == 0).all()
    rows = np.nonzero(empty)
    np.testing.assert_array_equal(fl["anc"][rows], (np.uint64(1) << rows[1].astype(np.uint64)))
    np.testing.assert_array_equal(fl["pos_id"][rows], base[rows[0]])
    # the filled rows still form a tree rooted at row 0
    for b in range(B):
        for f in np.nonzero(~empty[b])[0][1:]:
            assert 0 <= fl["parent"][b, f] < f and not empty[b, fl["parent"][b, f]]


def test_accept_ignores_empty_rows():
    # an empty row (parent -1, token -1) is never on an accepted path
    tok = np.array([[10, 11, -1, 12]], np.int32)
    par = np.array([[-1, 0, -1, 1]], np.int32)
    g = np.array([[11, 12, 5, 7]], np.int32)
    acc = O.accept(tok, par, g, 3)
    assert acc["accept_len"][0] == 2 and acc["bonus"][0] == 7
    np.testing.assert_array_equal(acc["accept_idx"][0], [1, 3, -1])


def test_update_skips_empty_rows():
    table = np.tile(np.arange(8, dtype=np.int32), (10, 1))
    tk = (np.arange(24, dtype=np.int32) + 100).reshape(3, 8)
    O.update(table, np.array([3, -1, 5], np.int32), tk)
    np.testing.assert_array_equal(table[3], tk[0])
    np.testing.assert_array_equal(table[5], tk[2])
    assert (table[[0, 1, 2, 4, 6, 7, 8, 9]] == np.arange(8)).all()
    with pytest.raises(RuntimeError):
        O.update(table, np.array([10], np.int32), tk[:1])      # an id >= V is still an error
