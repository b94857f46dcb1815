"""Pins of the oracle's row provenance, softmax statistics and coverage gain
(news write-up, section 三: the gain is the target probability mass that the
grafted candidates add where pruning cut, positive as soon as one of them has
nonzero probability).  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from synth import generators as G
from tests.test_oracle_pins import _build, _stage_logps

D, R_, ROOT = O.ROW_DRAFT, O.ROW_RETRIEVED, O.ROW_ROOT


def _tree(rows):
    """rows: list of (token, parent row, source); row 0 is the root."""
    tok = np.array([[r[0] for r in rows]], np.int32)
    par = np.array([[r[1] for r in rows]], np.int32)
    src = np.array([[r[2] for r in rows]], np.uint8)
    return tok, par, src


# root; draft child 5; retrieved 5 (same token as the draft sibling: not new);
# retrieved 7 (new at the root); retrieved 9 under row 3 (new there);
# retrieved 7 again under the root (counted once)
HAND = [(100, -1, ROOT), (5, 0, D), (5, 0, R_), (7, 0, R_), (9, 3, R_), (7, 0, R_)]


def test_all_equal_rows_give_one_over_v_per_new_token():
    V = 37
    tok, par, src = _tree(HAND)
    logits = np.zeros((1, len(HAND), V), np.float32) + np.float32(1.25)
    g = O.coverage_gain(logits, tok, par, src, "f32")
    assert g[0] == pytest.approx(2.0 / V, rel=1e-14)


def test_one_raised_entry_closed_form():
    V, a = 50, 3.0
    tok, par, src = _tree(HAND)
    logits = np.zeros((1, len(HAND), V), np.float32)
    logits[0, 0, 7] = a                      # root row: token 7 raised
    g = O.coverage_gain(logits, tok, par, src, "f32")
    p7 = math.exp(a) / (math.exp(a) + V - 1)  # new token 7 at the root
    p9 = 1.0 / V                              # new token 9 at row 3 (all-zero row)
    assert g[0] == pytest.approx(p7 + p9, rel=1e-13)


def test_zero_without_new_tokens():
    V = 40
    rng = np.random.default_rng(0)
    logits = rng.standard_normal((1, 4, V)).astype(np.float32)
    # no retrieval rows
    tok, par, src = _tree([(1, -1, ROOT), (2, 0, D), (3, 1, D), (4, 0, D)])
    assert O.coverage_gain(logits, tok, par, src, "f32")[0] == 0.0
    # every retrieved token repeats a kept draft sibling
    tok, par, src = _tree([(1, -1, ROOT), (2, 0, D), (2, 0, R_), (3, 1, D)])
    assert O.coverage_gain(logits, tok, par, src, "f32")[0] == 0.0
    # out-of-range retrieved tokens add nothing
    tok, par, src = _tree([(1, -1, ROOT), (2, 0, D), (V, 0, R_), (-1, 0, R_)])
    assert O.coverage_gain(logits, tok, par, src, "f32")[0] == 0.0


def test_positive_with_one_new_token_and_duplicates_do_not_count():
    V = 64
    rng = np.random.default_rng(1)
    logits = (rng.standard_normal((1, 3, V)) * 4).astype(np.float32)
    tok, par, src = _tree([(1, -1, ROOT), (2, 0, D), (3, 0, R_)])
    g1 = O.coverage_gain(logits, tok, par, src, "f32")[0]
    assert g1 > 0.0
    tok, par, src = _tree([(1, -1, ROOT), (2, 0, D), (3, 0, R_), (3, 0, R_)])
    logits2 = np.concatenate([logits, logits[:, :1]], axis=1)
    assert O.coverage_gain(logits2, tok, par, src, "f32")[0] == g1


def _brute(logits, tok, par, src):
    """Sets of new tokens per parent row and a full-row log-sum-exp softmax."""
    B, T1, V = logits.shape
    out = np.zeros(B)
    for b in range(B):
        for v in range(T1):
            draft = {int(tok[b, c]) for c in range(T1) if par[b, c] == v and src[b, c] == D}
            new = {int(tok[b, c]) for c in range(T1)
                   if par[b, c] == v and src[b, c] == R_ and 0 <= tok[b, c] < V} - draft
            if new:
                row = logits[b, v].astype(np.float64)
                lse = np.logaddexp.reduce(row)
                out[b] += sum(math.exp(row[x] - lse) for x in new)
    return out


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_gain_on_built_trees_matches_brute_force(layout):
    r = _build(layout, _stage_logps(), seed=3)
    fl = r["fl"]
    B, T1 = fl["tok"].shape
    V = 500
    rng = np.random.default_rng(7)
    z = (rng.standard_normal((B, T1, V)) * 2).astype(np.float32)
    logits = G.f32_to_bf16_bits(z).reshape(B, T1, V)
    g = O.coverage_gain(logits, fl["tok"], fl["parent"], fl["row_src"], "bf16")
    widened = (logits.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_allclose(g, _brute(widened, fl["tok"], fl["parent"], fl["row_src"]), rtol=1e-12)
    # stage "none" keeps every draft node: no retrieval, no gain
    assert g[3] == 0.0 and r["pr"]["stage"][3] == 3
    assert (g[:3] > 0).all()


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_row_sources_count_kept_and_retrieved(layout):
    r = _build(layout, _stage_logps())
    src = r["fl"]["row_src"]
    assert (src[:, 0] == ROOT).all()
    np.testing.assert_array_equal((src == D).sum(1), r["pr"]["n_keep"])
    np.testing.assert_array_equal((src == R_).sum(1), r["ret"]["n_ret"])
    assert not (src == O.ROW_EMPTY).any()
    if layout == "in_place":
        # draft node i stays in row i + 1 when kept
        np.testing.assert_array_equal(src[:, 1:] == D, r["pr"]["keep"].astype(bool))


def test_row_stats_closed_forms_and_numpy():
    V = 1000
    eq = np.full((1, V), np.float32(-2.5))
    st = O.row_stats(eq, "f32")
    assert st[0, 0] == -2.5 and st[0, 1] == pytest.approx(V, rel=1e-15)
    rng = np.random.default_rng(2)
    z = (rng.standard_normal((5, V)) * 3).astype(np.float32)
    st = O.row_stats(z, "f32")
    np.testing.assert_array_equal(st[:, 0], z.max(1).astype(np.float64))
    ref = np.exp(z.astype(np.float64) - z.max(1, keepdims=True).astype(np.float64)).sum(1)
    np.testing.assert_allclose(st[:, 1], ref, rtol=1e-12)

