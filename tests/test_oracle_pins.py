"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the pages'
budget table, closed forms, textbook/library special cases, brute force on tiny
inputs, or an independent construction (transitive closure by matrix powers,
depth-first search, dictionary last-writer).  No GPU is needed.
"""
import itertools
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from synth import generators as G

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------- top-k

def _bf16_rows(rng, n, V, scale=1.0, quant=None):
    z = rng.standard_normal((n, V)).astype(np.float32) * scale
    if quant is not None:
        z = np.round(z * quant) / quant
    return G.f32_to_bf16_bits(z).reshape(n, V)


def _sort_topk(vals, k):
    """Reference: full stable sort by (value desc, id asc) through numpy."""
    ids = np.arange(vals.shape[-1])
    out = []
    for row in vals:
        order = np.lexsort((ids, -row.astype(np.float64)))
        out.append(order[:k])
    return np.array(out, np.int32)


@pytest.mark.parametrize("V,k,quant", [(257, 8, None), (1000, 8, 4.0), (64, 8, 2.0), (9, 8, 1.0), (50, 3, 1.0)])
def test_topk_matches_full_sort_bf16(V, k, quant):
    rng = np.random.default_rng(V * 31 + k)
    rows = _bf16_rows(rng, 24, V, quant=quant)
    got = O.topk(rows, k, "bf16")
    want = _sort_topk(G.bf16_bits_to_f32(rows), k)
    np.testing.assert_array_equal(got, want)


def test_topk_matches_full_sort_f32_with_signed_zeros():
    rng = np.random.default_rng(5)
    rows = np.round(rng.standard_normal((16, 300)) * 2.0).astype(np.float32)
    rows[rows == 0] = np.where(rng.random(int((rows == 0).sum())) < 0.5, -0.0, 0.0).astype(np.float32)
    rows[3] = -0.0
    rows[4] = 0.0
    rows[5, ::2] = -0.0
    got = O.topk(rows, 8, "f32")
    np.testing.assert_array_equal(got, _sort_topk(rows, 8))
    np.testing.assert_array_equal(got[3], np.arange(8))       # -0 == +0: ids ascend
    np.testing.assert_array_equal(got[4], np.arange(8))


def test_topk_signed_zero_bf16_equal():
    row = np.zeros((1, 20), np.uint16)
    row[0, 0:10] = 0x8000          # -0 at the low ids, +0 above: all equal
    got = O.topk(row, 8, "bf16")
    np.testing.assert_array_equal(got[0], np.arange(8))
    row[0, 15] = 0x3F80            # +1.0
    got = O.topk(row, 8, "bf16")
    assert got[0, 0] == 15
    np.testing.assert_array_equal(got[0, 1:], np.arange(7))


def test_topk_k1_is_first_argmax():
    rng = np.random.default_rng(7)
    rows = _bf16_rows(rng, 40, 500, quant=2.0)
    got = O.topk(rows, 1, "bf16")[:, 0]
    want = np.argmax(G.bf16_bits_to_f32(rows), axis=1)
    np.testing.assert_array_equal(got, want)


def test_topk_unique_bump_is_top1():
    rng = np.random.default_rng(8)
    z = rng.standard_normal((10, 4000)).astype(np.float32)
    z = np.clip(z, -5.0, 5.0)
    cols = rng.integers(0, 4000, size=10)
    z[np.arange(10), cols] = 6.0 + 5.0
    got = O.topk(G.f32_to_bf16_bits(z).reshape(z.shape), 8, "bf16")
    np.testing.assert_array_equal(got[:, 0], cols)


def test_topk_all_equal_rows_take_lowest_ids():
    rows = np.full((3, 100), 0x4040, np.uint16)
    np.testing.assert_array_equal(O.topk(rows, 8, "bf16"), np.tile(np.arange(8), (3, 1)))


def test_topk_prob_closed_forms():
    V = 1000
    eq = np.zeros((1, V), np.float32)
    _, p = O.topk(eq, 8, "f32", want_prob=True)
    np.testing.assert_allclose(p, 1.0 / V, rtol=1e-12)
    one = np.zeros((1, V), np.float32)
    one[0, 123] = 3.0
    tk, p = O.topk(one, 8, "f32", want_prob=True)
    assert tk[0, 0] == 123
    e3 = math.exp(3.0)
    np.testing.assert_allclose(p[0, 0], e3 / (e3 + V - 1), rtol=1e-12)
    np.testing.assert_allclose(p[0, 1:], 1.0 / (e3 + V - 1), rtol=1e-12)


def test_topk_prob_vs_scipy_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(9)
    rows = _bf16_rows(rng, 6, 2000, scale=3.0)
    tk, p = O.topk(rows, 8, "bf16", want_prob=True)
    sm = softmax(G.bf16_bits_to_f32(rows).astype(np.float64), axis=1)
    np.testing.assert_allclose(p, np.take_along_axis(sm, tk, axis=1), rtol=1e-12)


# ----------------------------------------------------------------------------- prune

TOPO = G.static_tree()


def _tree_batch(logp_rows):
    par, lay, _ = TOPO
    B = len(logp_rows)
    return np.tile(par, (B, 1)), np.tile(lay, (B, 1)), np.array(logp_rows, np.float32)


def test_static_tree_shape():
    par, lay, rank = TOPO
    assert len(par) == 60
    assert list(np.bincount(lay)) == [8, 16, 12, 10, 8, 6]
    assert (par < np.arange(60)).all()
    kids = np.bincount(par[par >= 0], minlength=60)
    assert kids.max() <= 8


def test_prune_closed_form_half_probabilities():
    # every draft prob 0.5: best cumulative confidence on layer l is 0.5^(l+1):
    # layer 0: 0.5 >= 0.3, layer 1: 0.25 >= 0.2, layer 5: 1/64 < 0.1 -> stage 2 (keep 40)
    par, lay, lp = _tree_batch([np.full(60, math.log(0.5))])
    r = O.prune_tree(par, lay, lp, want_cum=True)
    assert r["stage"][0] == 2 and r["n_keep"][0] == 40
    # cumulative confidence falls with depth, ties by lower index -> nodes 0..39
    np.testing.assert_array_equal(np.nonzero(r["keep"][0])[0], np.arange(40))
    np.testing.assert_allclose(r["cum"][0], (lay[0] + 1) * np.float32(math.log(0.5)), rtol=1e-6)


def test_prune_each_stage_forced():
    par, lay, _ = TOPO
    ln = math.log
    s0 = np.where(lay == 0, ln(0.25), ln(0.9))          # first-token conf 0.25 < 0.3
    s1 = np.where(lay == 0, ln(0.5), ln(0.35))          # layer-1 best 0.175 < 0.2
    s2 = np.full(60, ln(0.7))                           # 0.7^6 = 0.118 ... layer 5: 0.7^6
    s2[lay == 5] = ln(0.1)                              # 0.7^5*0.1 = 0.0168 < 0.1
    s3 = np.zeros(60)                                   # all confidences 1
    par_b, lay_b, lp = _tree_batch([s0, s1, s2, s3])
    r = O.prune_tree(par_b, lay_b, lp)
    np.testing.assert_array_equal(r["stage"], [0, 1, 2, 3])
    np.testing.assert_array_equal(r["n_keep"], [8, 24, 40, 60])
    np.testing.assert_array_equal(np.nonzero(r["keep"][0])[0], np.nonzero(lay == 0)[0])
    np.testing.assert_array_equal(np.nonzero(r["keep"][1])[0], np.nonzero(lay <= 1)[0])
    assert r["keep"][3].all()


def test_budget_table_from_pages():
    rows = _golden_rows("budget_splits.txt")
    par, lay, _ = TOPO
    ln = math.log
    forced = {0: np.where(lay == 0, ln(0.25), ln(0.9)), 1: np.where(lay == 0, ln(0.5), ln(0.35)),
              3: np.zeros(60)}
    s2 = np.full(60, ln(0.7))
    s2[lay == 5] = ln(0.1)
    forced[2] = s2
    tpl = O.template(8, 8, 52)
    table = np.tile(np.arange(8, dtype=np.int32), (100, 1))
    for st, _ck, kept, retr in rows:
        st, kept, retr = int(st), int(kept), int(retr)
        par_b, lay_b, lp = _tree_batch([forced[st]])
        r = O.prune_tree(par_b, lay_b, lp)
        assert r["stage"][0] == st
        assert r["n_keep"][0] == kept
        ret = O.retrieve_tree(table, [5], r["n_keep"], 60, tpl)
        assert ret["n_ret"][0] == retr
        assert kept + retr == 60
        assert (ret["n_ret"][0] == 0) == (st == 3)     # no prune -> no retrieval


def test_prune_threshold_is_strict_and_ties_keep_lower_index():
    par, lay, _ = TOPO
    lthr = np.float32(math.log(0.3))
    lp = np.zeros(60, np.float32)
    lp[lay == 0] = lthr                      # best == ln(0.3) exactly: not below -> no fire
    r = O.prune_tree(*_tree_batch([lp]))
    assert r["stage"][0] != 0
    # stage 2 keep boundary: give all layer-3 nodes the same cum; only the lowest ids survive
    lp = np.full(60, math.log(0.7), np.float32)
    lp[lay == 5] = math.log(0.05)
    r = O.prune_tree(*_tree_batch([lp]))
    assert r["stage"][0] == 2
    l3 = np.nonzero(lay == 3)[0]
    kept3 = [i for i in l3 if r["keep"][0][i]]
    assert kept3 == list(l3[: len(kept3)])


def test_prune_unreached_checkpoint_does_not_fire():
    # a tree with no layer 5: checkpoint 2 is not reached even with low confidences
    par = np.array([-1, -1, 0, 0, 1, 2, 2, 3], np.int32)
    lay = np.array([0, 0, 1, 1, 1, 2, 2, 2], np.int32)
    lp = np.full(8, math.log(0.9), np.float32)
    lp[lay == 2] = math.log(0.01)
    r = O.prune_tree(par[None], lay[None], lp[None], keep=(2, 5, 6))
    assert r["stage"][0] == 3 and r["n_keep"][0] == 8


def test_tail_prefix():
    conf = np.array([[0.9] * 16, [0.4] * 16, [0.9, 0.8, 0.5, 0.49] + [0.1] * 12,
                     [0.5] * 3 + [0.6] + [0.2] * 12], np.float32)
    r = O.prune_tail(conf, 0.5)
    np.testing.assert_array_equal(r["n_keep"], [16, 0, 3, 4])
    np.testing.assert_array_equal(r["stage"], [3, 0, 0, 0])


# ----------------------------------------------------------------------------- template / retrieve

def _chain_lengths(tpl, W=8):
    lens = [0] * W
    # rank of the chain = rank of its depth-1 head
    head = {}
    for t in range(len(tpl["parent"])):
        p = tpl["parent"][t]
        head[t] = tpl["rank"][t] if p < 0 else head[p]
        lens[head[t]] = max(lens[head[t]], tpl["depth"][t])
    return lens


def test_template_shape_and_chain_lengths():
    shape = dict((k, int(v)) for k, v in _golden_rows("template_shape.txt"))
    full = O.template(shape["width"], shape["depth"], 10_000)
    assert len(full) if False else len(full["parent"]) == 8 * 8   # every (rank, depth) node once
    assert full["depth"].max() == shape["depth"]
    assert sorted(full["rank"][full["parent"] < 0].tolist()) == list(range(shape["width"]))
    # Chain lengths for the three budgets, derived by hand from the ordering rule
    # (root children, rank-0 chain, then increasing depth+rank): higher-ranked
    # successors get longer chains, as the write-up's template description asks.
    for R, want in [(20, [8, 4, 3, 1, 1, 1, 1, 1]), (36, [8, 7, 6, 5, 4, 3, 2, 1]),
                    (52, [8, 8, 8, 8, 7, 6, 4, 3])]:
        tpl = O.template(8, 8, R)
        assert len(tpl["parent"]) == R
        assert _chain_lengths(tpl) == want
        assert all(want[j] >= want[j + 1] for j in range(7))
        # nesting: every budget's template is a prefix of the full order
        for key in ("parent", "rank", "depth"):
            np.testing.assert_array_equal(tpl[key], full[key][:R])
        # ancestor closure and topological order
        for t in range(R):
            p = tpl["parent"][t]
            assert p < t
            assert tpl["depth"][t] == (1 if p < 0 else tpl["depth"][p] + 1)
            assert (tpl["rank"][t] == 0) or p < 0


def test_retrieve_closed_form_successor_table():
    V = 1000
    table = ((np.arange(V)[:, None] + np.arange(8)[None, :] + 1) % V).astype(np.int32)
    tpl = O.template(8, 8, 52)
    roots = np.array([3, 990], np.int32)
    ret = O.retrieve_tree(table, roots, np.array([8, 40], np.int32), 60, tpl)
    assert list(ret["n_ret"]) == [52, 20]
    # node (rank j, depth d) = root + j + d (mod V)
    head = {}
    for b in range(2):
        for t in range(ret["n_ret"][b]):
            p = tpl["parent"][t]
            head[t] = tpl["rank"][t] if p < 0 else head[p]
            want = (roots[b] + head[t] + tpl["depth"][t]) % V
            assert ret["ret_tok"][b, t] == want
        assert (ret["ret_tok"][b, ret["n_ret"][b]:] == -1).all()


def test_retrieve_tail_chain_closed_form():
    V = 50
    table = ((np.arange(V)[:, None] * 3 + np.arange(8)[None, :] + 1) % V).astype(np.int32)
    d_tok = np.tile(np.arange(16, dtype=np.int32) + 10, (3, 1))
    n_keep = np.array([0, 5, 16], np.int32)
    ret = O.retrieve_tail(table, [7, 7, 7], d_tok, n_keep)
    assert list(ret["n_ret"]) == [16, 11, 0]
    x = 7
    for t in range(16):
        x = (3 * x + 1) % V
        assert ret["ret_tok"][0, t] == x
    x = 14
    for t in range(11):
        x = (3 * x + 1) % V
        assert ret["ret_tok"][1, t] == x


# ----------------------------------------------------------------------------- flatten

def _closure(parent):
    """Ancestor-or-self relation by boolean matrix powers of the parent relation."""
    n = len(parent)
    A = np.zeros((n, n), bool)
    for f, p in enumerate(parent):
        if p >= 0:
            A[f, p] = True
    R = np.eye(n, dtype=bool)
    P = np.eye(n, dtype=bool)
    for _ in range(n):
        P = (P.astype(np.int64) @ A.astype(np.int64)) > 0
        R |= P
    return R


def _build(layout, stages_logp, seed=0):
    rng = np.random.default_rng(seed)
    V = 500
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    par_b, lay_b, lp = _tree_batch(stages_logp)
    B = len(stages_logp)
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    base = rng.integers(0, 1000, size=B).astype(np.int32)
    pr = O.prune_tree(par_b, lay_b, lp)
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, O.template(8, 8, 52))
    fl = O.flatten(layout, 61, roots, base, d_tok, par_b, pr["keep"], pr["n_keep"], ret)
    return dict(pr=pr, ret=ret, fl=fl, d_tok=d_tok, roots=roots, base=base, par=par_b)


def _stage_logps():
    par, lay, _ = TOPO
    ln = math.log
    s2 = np.full(60, ln(0.7))
    s2[lay == 5] = ln(0.1)
    return [np.where(lay == 0, ln(0.25), ln(0.9)), np.where(lay == 0, ln(0.5), ln(0.35)), s2, np.zeros(60)]


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_flatten_mask_is_transitive_closure(layout):
    r = _build(layout, _stage_logps())
    fl = r["fl"]
    for b in range(4):
        par = fl["parent"][b]
        assert par[0] == -1 and (par[1:] >= 0).all() and (par[1:] < np.arange(1, 61)).all()
        R = _closure(par)
        for f in range(61):
            bits = [(int(fl["anc"][b, f]) >> g) & 1 for g in range(61)]
            np.testing.assert_array_equal(bits, R[f].astype(int))
            assert bin(int(fl["anc"][b, f])).count("1") == fl["depth"][b, f] + 1
        np.testing.assert_array_equal(fl["pos_id"][b], r["base"][b] + fl["depth"][b])
        assert fl["tok"][b, 0] == r["roots"][b]


def test_flatten_layouts_place_nodes():
    r_c = _build("compact", _stage_logps(), seed=1)
    r_i = _build("in_place", _stage_logps(), seed=1)
    for b in range(4):
        keep = r_c["pr"]["keep"][b].astype(bool)
        nk = int(keep.sum())
        R = int(r_c["ret"]["n_ret"][b])
        kept = np.nonzero(keep)[0]
        # compact: kept draft ascending, then retrieval in template order
        np.testing.assert_array_equal(r_c["fl"]["tok"][b, 1:1 + nk], r_c["d_tok"][b, kept])
        np.testing.assert_array_equal(r_c["fl"]["tok"][b, 1 + nk:], r_c["ret"]["ret_tok"][b, :R])
        # in-place: draft slot i -> row i+1; vacated rows ascending take retrieval nodes
        np.testing.assert_array_equal(r_i["fl"]["tok"][b, 1 + kept], r_i["d_tok"][b, kept])
        vac = np.nonzero(~keep)[0] + 1
        np.testing.assert_array_equal(r_i["fl"]["tok"][b, vac], r_i["ret"]["ret_tok"][b, :R])
        # both describe the same tree: same multiset of (depth, token) pairs
        a = sorted(zip(r_c["fl"]["depth"][b].tolist(), r_c["fl"]["tok"][b].tolist()))
        c = sorted(zip(r_i["fl"]["depth"][b].tolist(), r_i["fl"]["tok"][b].tolist()))
        assert a == c


# ----------------------------------------------------------------------------- acceptance

def _dfs_accept(tok, parent, g):
    """Independent search: depth-first from the root along edges with
    tok[child] == g[parent]; deepest node, ties by lowest index."""
    T1 = len(tok)
    kids = [[] for _ in range(T1)]
    for f in range(1, T1):
        kids[parent[f]].append(f)
    best = (0, 0)
    stack = [(0, 0)]
    while stack:
        f, d = stack.pop()
        if d > best[0] or (d == best[0] and f < best[1]):
            best = (d, f)
        for c in kids[f]:
            if tok[c] == g[f]:
                stack.append((c, d + 1))
    return best


def _random_tree(rng, T1, V):
    parent = np.array([-1] + [int(rng.integers(0, f)) for f in range(1, T1)], np.int32)
    tok = rng.integers(0, V, size=T1).astype(np.int32)
    return tok, parent


def test_accept_matches_dfs():
    rng = np.random.default_rng(11)
    for trial in range(300):
        T1 = int(rng.integers(1, 30))
        V = int(rng.integers(2, 6))
        tok, parent = _random_tree(rng, T1, V)
        g = rng.integers(0, V, size=T1).astype(np.int32)
        r = O.accept(tok[None], parent[None], g[None], Dmax=T1)
        d, f = _dfs_accept(tok, parent, g)
        assert r["accept_len"][0] == d
        assert r["bonus"][0] == g[f]
        path = r["accept_idx"][0][:d]
        if d:
            assert path[-1] == f
            assert parent[path[0]] == 0
            for a, b2 in zip(path[:-1], path[1:]):
                assert parent[b2] == a
        assert (r["accept_idx"][0][d:] == -1).all()


def test_superset_and_monotonicity_exhaustive_tiny_vocab():
    """Accept length of the hybrid tree >= the pruned-only tree (superset), and the
    dense tree >= the pruned-only tree (monotonicity), for every greedy target
    g: V -> V over a bigram context, V <= 4."""
    rng = np.random.default_rng(12)
    for V in (3, 4):
        for trial in range(6):
            T1 = 10
            tok, parent = _random_tree(rng, T1, V)
            keep_rows = np.array([True] * T1)
            # prune = drop a random subtree set while staying ancestor-closed
            for f in range(1, T1):
                if rng.random() < 0.35 or not keep_rows[parent[f]]:
                    keep_rows[f] = False
            pruned_idx = np.nonzero(keep_rows)[0]
            remap = {int(o): n for n, o in enumerate(pruned_idx)}
            p_tok = tok[pruned_idx]
            p_par = np.array([-1] + [remap[int(parent[o])] for o in pruned_idx[1:]], np.int32)
            # hybrid = pruned + a retrieval chain of extra nodes hung under the root
            extra = int(T1 - len(pruned_idx))
            h_tok = np.concatenate([p_tok, rng.integers(0, V, size=extra).astype(np.int32)])
            h_par = np.concatenate([p_par, np.array([0] + list(range(len(p_tok), len(p_tok) + extra - 1))
                                                    if extra else [], np.int32)]).astype(np.int32)
            for gmap in itertools.product(range(V), repeat=V):
                gm = np.array(gmap, np.int32)
                la = O.accept(tok[None], parent[None], gm[tok][None], T1)["accept_len"][0]
                lp = O.accept(p_tok[None], p_par[None], gm[p_tok][None], T1)["accept_len"][0]
                lh = O.accept(h_tok[None], h_par[None], gm[h_tok][None], T1)["accept_len"][0]
                assert lh >= lp
                assert la >= lp


# ----------------------------------------------------------------------------- update

def test_update_last_writer_wins():
    rng = np.random.default_rng(13)
    V, k = 40, 8
    table = rng.integers(0, V, size=(V, k)).astype(np.int32)
    before = table.copy()
    row_tok = rng.integers(0, 10, size=200).astype(np.int32)
    tk = rng.integers(0, V, size=(200, k)).astype(np.int32)
    O.update(table, row_tok, tk)
    last = {}
    for P, x in enumerate(row_tok):
        last[int(x)] = P
    for x in range(V):
        if x in last:
            np.testing.assert_array_equal(table[x], tk[last[x]])
        else:
            np.testing.assert_array_equal(table[x], before[x])


# ----------------------------------------------------------------------------- grafted subtree

def _placement(layout, keep, n_ret):
    """Rows of the kept draft nodes and of the template nodes under each layout's
    placement rule, derived here from the rule alone: compact puts the kept draft
    nodes first (ascending), then the template nodes in order; in place, draft slot
    i is row i+1 and the vacated slots, ascending, take the template nodes."""
    keep = keep.astype(bool)
    kept = np.nonzero(keep)[0]
    if layout == "compact":
        drow = {int(i): 1 + n for n, i in enumerate(kept)}
        trow = [1 + len(kept) + t for t in range(n_ret)]
    else:
        drow = {int(i): int(i) + 1 for i in kept}
        trow = (np.nonzero(~keep)[0] + 1).tolist()[:n_ret]
    return drow, trow


def _random_logps(rng, n):
    """Draft log-probabilities: log-softmax over each node's 8 siblings of N(0, 1.5)
    logits (the toy workload's recipe), so the stage varies between requests."""
    par, lay, _ = TOPO
    out = []
    for _ in range(n):
        z = rng.normal(0.0, 1.5, size=60)
        lp = np.zeros(60)
        for p in np.unique(par):
            sib = np.nonzero(par == p)[0]
            zs = z[sib]
            lp[sib] = zs - (zs.max() + np.log(np.exp(zs - zs.max()).sum()))
        out.append(lp)
    return out


@pytest.mark.parametrize("layout", ["compact", "in_place"])
@pytest.mark.parametrize("tpl_kind", ["chain", "branching"])
def test_grafted_subtree_follows_template(layout, tpl_kind):
    """Gear 2 of the write-up expands the retrieval tree from the current token: each
    node is the rank-r successor, in the continuation matrix, of its parent node's
    token.  So every row holding template node t must sit at depth tpl_depth[t],
    hang under the row holding tpl_parent[t] (the root at depth 1), and carry
    M[token of that row][tpl_rank[t]].  Kept draft nodes keep their own shape:
    depth = layer + 1 under the row of their draft parent."""
    rng = np.random.default_rng(21 if tpl_kind == "chain" else 22)
    V = 500
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    tpl = O.template(8, 8, 52) if tpl_kind == "chain" else O.template_branching(4, 6, (1, 1), 52)
    logps = _stage_logps() + _random_logps(rng, 12)
    par_b, lay_b, lp = _tree_batch(logps)
    par, lay, _ = TOPO
    B = len(logps)
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    base = rng.integers(0, 1000, size=B).astype(np.int32)
    pr = O.prune_tree(par_b, lay_b, lp)
    assert set(pr["stage"].tolist()) == {0, 1, 2, 3}
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, tpl)
    fl = O.flatten(layout, 61, roots, base, d_tok, par_b, pr["keep"], pr["n_keep"], ret)
    for b in range(B):
        R = int(ret["n_ret"][b])
        assert R == min(60 - int(pr["n_keep"][b]), len(tpl["parent"]))
        drow, trow = _placement(layout, pr["keep"][b], R)
        tk, pa, dp, src = fl["tok"][b], fl["parent"][b], fl["depth"][b], fl["row_src"][b]
        assert (src == O.ROW_RETRIEVED).sum() == R
        for t, f in enumerate(trow):
            pt = int(tpl["parent"][t])
            assert src[f] == O.ROW_RETRIEVED
            assert dp[f] == tpl["depth"][t]
            assert pa[f] == (0 if pt < 0 else trow[pt])
            assert tk[f] == table[tk[pa[f]], tpl["rank"][t]]
        for i, f in drow.items():
            assert src[f] == O.ROW_DRAFT and tk[f] == d_tok[b, i]
            assert dp[f] == lay[i] + 1
            assert pa[f] == (0 if par[i] < 0 else drow[int(par[i])])


@pytest.mark.parametrize("layout", ["compact", "in_place"])
@pytest.mark.parametrize("V,W", [(4, 4), (8, 8)])
def test_superset_through_oracle_pipeline(layout, V, W):
    """Section 三 of the write-up: the hybrid tree contains the pruned draft tree, so
    strict greedy verification accepts at least as much on it.  Through the oracle's
    own prune -> retrieve -> flatten -> accept chain, on the same drafts and matrix,
    the rank-chain template against the empty one (no retrieval), for every greedy
    target g: V -> V at V = 4 (k = 4, width 4) and 600 seeded ones at V = 8."""
    rng = np.random.default_rng(100 * V + (layout == "compact"))
    k = W
    table = rng.integers(0, V, size=(V, k)).astype(np.int32)
    tpl = O.template(W, 8, 52)
    empty = {key: np.zeros(0, np.int32) for key in ("parent", "rank", "depth")}
    logps = _stage_logps() + _random_logps(rng, 4)
    par_b, lay_b, lp = _tree_batch(logps)
    B = len(logps)
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    base = np.zeros(B, np.int32)
    pr = O.prune_tree(par_b, lay_b, lp)
    trees = {}
    for name, tp in (("hybrid", tpl), ("pruned", empty)):
        ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, tp, Rmax_out=52)
        trees[name] = O.flatten(layout, 61, roots, base, d_tok, par_b, pr["keep"], pr["n_keep"], ret)
    ph, pp = trees["hybrid"], trees["pruned"]
    assert (pp["row_src"] != O.ROW_RETRIEVED).all()
    maps = (itertools.product(range(V), repeat=V) if V <= 4
            else (tuple(rng.integers(0, V, size=V)) for _ in range(600)))
    gains = 0
    for gmap in maps:
        gm = np.array(gmap + (0,), np.int32)   # index -1 (an empty row) reads the pad
        lh = O.accept(ph["tok"], ph["parent"], gm[ph["tok"]], 60)["accept_len"]
        lq = O.accept(pp["tok"], pp["parent"], gm[pp["tok"]], 60)["accept_len"]
        assert (lh >= lq).all()
        gains += int((lh > lq).sum())
    assert gains > 0   # retrieval does add accepted tokens on some targets
