"""GPU parity of each C-ABI entry point against the CPU oracle, element by
element, on seeded inputs plus adversarial ones (ties, signed zeros, all-equal
rows, negative-only rows, ragged and tiny vocabularies, every prune stage,
maximal update collisions).  Integers and indices must match bit for bit;
probabilities within 1e-5 relative of the fp64 oracle."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hybrid_draft_tree_amd import _lib as L  # noqa: E402
from oracle import oracle as O  # noqa: E402
from synth import generators as G  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _s():
    return torch.cuda.current_stream().cuda_stream


def _t(a, dtype=None):
    return torch.as_tensor(np.ascontiguousarray(a)).to(DEV) if dtype is None else \
        torch.as_tensor(np.ascontiguousarray(a)).to(DEV, dtype)


def gpu_topk(rows, k, dtype, want_prob=False):
    """Top-k through graft_update_topk (logits given, topk_out set)."""
    n, V = rows.shape
    if dtype == "bf16":
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)
        dt = L.DTYPE_BF16
    else:
        lg = _t(rows.view(np.float32))
        dt = L.DTYPE_F32
    out = torch.full((n, k), -7, dtype=torch.int32, device=DEV)
    table = torch.zeros(max(V, 1), k, dtype=torch.int32, device=DEV)
    tprob = torch.zeros(max(V, 1), k, dtype=torch.float32, device=DEV) if want_prob else None
    row_tok = torch.arange(n, dtype=torch.int32, device=DEV) % V
    wsb = L.graft_workspace_bytes(n, V, k, dt)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    L.graft_update_topk(n, V, k, dt, lg.data_ptr(), None, None, row_tok.data_ptr(), table.data_ptr(),
                        tprob.data_ptr() if want_prob else None, out.data_ptr(), ws.data_ptr(), wsb, _s())
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if want_prob:
        # the last writer of table row x is the highest row with row_tok == x
        return res, tprob.cpu().numpy(), table.cpu().numpy()
    return res


def _bf16(z):
    return G.f32_to_bf16_bits(np.asarray(z, np.float32)).reshape(np.shape(z))


def _rows_suite(rng, n, V):
    z = rng.standard_normal((n, V)).astype(np.float32)
    suite = {"normal": _bf16(z)}
    suite["quantised_ties"] = _bf16(np.round(z * 2) / 2)
    eq = np.full((n, V), 0x3F80, np.uint16)
    suite["all_equal"] = eq
    neg = _bf16(-np.abs(z) - 0.25)
    suite["negative_only"] = neg
    sz = _bf16(np.round(z))
    zeros = sz == 0
    sz[zeros & (rng.random((n, V)) < 0.5)] = 0x8000
    suite["signed_zeros"] = sz
    asc = _bf16(np.tile(np.linspace(-3, 3, V, dtype=np.float32), (n, 1)))
    suite["ascending"] = asc
    suite["descending"] = asc[:, ::-1].copy()
    bump = _bf16(np.clip(z, -4, 4))
    cols = rng.integers(0, V, size=n)
    bump[np.arange(n), cols] = _bf16(np.full(n, 6.0))
    suite["bump"] = bump
    return suite


@pytest.mark.parametrize("V", [151936, 32000, 1001, 4097, 9, 8, 15, L.GRAFT_MAX_VOCAB, 999_999])
def test_topk_bf16_parity(V):
    rng = np.random.default_rng(V)
    n = 24 if V > 10000 else 40
    for name, rows in _rows_suite(rng, n, V).items():
        got = gpu_topk(rows, 8, "bf16")
        want = O.topk(rows, 8, "bf16")
        assert (got == want).all(), (name, V, np.nonzero((got != want).any(1))[0][:5])


@pytest.mark.parametrize("V,k", [(32000, 8), (1003, 8), (5, 5), (64, 3), (128256, 1), (L.GRAFT_MAX_VOCAB, 8)])
def test_topk_f32_parity(V, k):
    rng = np.random.default_rng(V + k)
    z = rng.standard_normal((20, V)).astype(np.float32)
    z[1] = np.round(z[1])
    z[2] = 0.0
    z[3, ::3] = -0.0
    z[4] = -np.abs(z[4]) - 1
    z[5] = np.float32(1e-40) * np.sign(z[5])        # subnormals
    z[6, :] = -np.inf
    z[6, V // 2] = -3.0
    got = gpu_topk(z, k, "f32")
    want = O.topk(z, k, "f32")
    assert (got == want).all(), np.nonzero((got != want).any(1))[0]


@pytest.mark.parametrize("n,V", [(61, 32000), (61, 128256), (244, 4097), (1100, 1003)])
def test_topk_f32_adversarial(n, V):
    """fp32 rows whose groups all pass the filter (ascending, all equal), heavy
    ties and negative-only rows, on split launches (61 rows: the one-by-one
    inserts, the count over LDS and the full merge of a wave's pending groups)
    and unsplit ones."""
    rng = np.random.default_rng(n + V)
    z = rng.standard_normal((n, V)).astype(np.float32)
    asc = np.tile(np.linspace(-3, 3, V, dtype=np.float32), (n, 1))
    suite = {"normal": z, "quantised_ties": np.round(z * 2) / 2, "all_equal": np.ones((n, V), np.float32),
             "negative_only": -np.abs(z) - 0.25, "ascending": asc, "descending": asc[:, ::-1].copy(),
             "few_values": rng.integers(-3, 4, size=(n, V)).astype(np.float32)}
    for name, rows in suite.items():
        got = gpu_topk(rows, 8, "f32")
        want = O.topk(rows, 8, "f32")
        assert (got == want).all(), (name, n, V, np.nonzero((got != want).any(1))[0][:5])


def test_topk_prob_parity():
    rng = np.random.default_rng(3)
    V = 151936
    z = (rng.standard_normal((12, V)) * 2.0).astype(np.float32)
    z[0] = 0.0
    z[1, :1000] = -np.inf            # masked prefix: the first batches hold only -inf
    z[2] = -np.inf                   # one finite entry: probability 1
    z[2, 77777] = 1.5
    rows = _bf16(z)
    tk, tprob, table = gpu_topk(rows, 8, "bf16", want_prob=True)
    want_tk, want_p = O.topk(rows, 8, "bf16", want_prob=True)
    assert (tk == want_tk).all()
    # rows wrote table rows 0..11 (row_tok = row index)
    np.testing.assert_allclose(tprob[:12], want_p, rtol=1e-5, atol=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_topk_prompt_sized_launch(dtype):
    """1600 rows: one workgroup per row with four blocks per batch (the plan for
    prompt-sized launches), every row compared, tie-heavy and ragged rows included."""
    rng = np.random.default_rng(31)
    n, V = 1600, 4097
    z = rng.standard_normal((n, V)).astype(np.float32)
    z[::7] = np.round(z[::7] * 2) / 2
    z[3::11] = -np.abs(z[3::11]) - 0.5
    rows = _bf16(z) if dtype == "bf16" else z
    got = gpu_topk(rows, 8, dtype)
    want = O.topk(rows, 8, dtype)
    assert (got == want).all(), np.nonzero((got != want).any(1))[0][:5]


# launch plans on both sides of their thresholds: split below 512 rows (at most
# 4 slices) unless 183-256 rows fill the CUs one workgroup each or 436-511 rows
# two workgroups each (8 waves), four
# blocks per batch for unsplit launches and for split rows whose waves stream 6
# or more blocks, two otherwise or when four exceed the LDS
@pytest.mark.parametrize("n,V,dtype,prob", [
    (430, 40000, "bf16", False),    # split into 3 slices, 13 blocks per wave: four
    (511, 40000, "bf16", False),    # whole rows, two on nearly every CU, 8 waves of ~10 blocks: four
    (450, 20000, "f32", True),      # whole fp32 rows, two on nearly every CU, 8 waves of ~10 blocks: four
    (512, 40000, "bf16", True),     # one workgroup per row, 6 waves: four, with probabilities
    (300, 20000, "bf16", False),    # split, 5 blocks per wave: two
    (200, 30000, "bf16", True),     # whole rows, one workgroup per CU, 8 waves of ~7 blocks: four
    (100, 151936, "f32", True),     # split fp32, 30 blocks per wave: four, with probabilities
    (244, 40000, "f32", True),      # whole fp32 rows, one workgroup per CU, 8 waves of ~20 blocks: four
    (2000, 3000, "f32", False),     # unsplit, short rows
    (700, 9, "bf16", False),        # a row shorter than one block
    (5, 151936, "bf16", False),     # split, 16 waves per slice: two
    (1, 999_999, "bf16", False),    # split, four would exceed the LDS: two
])
def test_topk_launch_plans(n, V, dtype, prob):
    rng = np.random.default_rng(n * 7 + V)
    z = rng.standard_normal((n, V)).astype(np.float32)
    z[::5] = np.round(z[::5] * 2) / 2
    rows = _bf16(z) if dtype == "bf16" else z
    if prob:
        tk, tprob, table = gpu_topk(rows, 8, dtype, want_prob=True)
        want_tk, want_p = O.topk(rows, 8, dtype, want_prob=True)
        assert (tk == want_tk).all(), np.nonzero((tk != want_tk).any(1))[0][:5]
        # table row x holds the top-k of the highest row with token x (row_tok = row % V)
        last = {}
        for r in range(n):
            last[r % V] = r
        xs = np.array(sorted(last)[:64])
        rs = np.array([last[x] for x in xs])
        np.testing.assert_allclose(tprob[xs], want_p[rs], rtol=1e-5, atol=0)
    else:
        got = gpu_topk(rows, 8 if V >= 8 else V, dtype)
        want = O.topk(rows, 8 if V >= 8 else V, dtype)
        assert (got == want).all(), np.nonzero((got != want).any(1))[0][:5]


@pytest.mark.parametrize("dtype,V", [("bf16", 30011), ("f32", 16411)])
def test_topk_merge_wave_launch(dtype, V):
    """1024 rows of long streams take the merge-wavefront plan (3 streaming
    waves and one merge wave per row): every adversarial row kind of the suite
    (ties, all-equal rows whose every group passes the filter and fills the
    rings, negative-only rows, signed zeros, ascending and descending rows, a
    bump) with unaligned row starts (odd V), each row compared with the oracle;
    probabilities within 1e-5 relative on the normal rows."""
    n = 1024
    dt = L.DTYPE_BF16 if dtype == "bf16" else L.DTYPE_F32
    plan = L.graft_launch_plan(n, V, dt, 0)
    assert plan["groups_per_row"] == 1 and plan["waves_per_group"] == 4
    rng = np.random.default_rng(V)
    for name, rows in _rows_suite(rng, n, V).items():
        if dtype == "f32":
            rows = G.bf16_bits_to_f32(rows).reshape(rows.shape)
        got = gpu_topk(rows, 8, dtype)
        want = O.topk(rows, 8, dtype)
        assert (got == want).all(), (name, np.nonzero((got != want).any(1))[0][:5])
    z = rng.standard_normal((n, V)).astype(np.float32)
    rows = _bf16(z) if dtype == "bf16" else z
    tk, tprob, table = gpu_topk(rows, 8, dtype, want_prob=True)
    want_tk, want_p = O.topk(rows, 8, dtype, want_prob=True)
    assert (tk == want_tk).all()
    np.testing.assert_allclose(tprob[:n], want_p, rtol=1e-5, atol=0)


def test_topk_max_vocab_unsplit_sampled():
    """512 rows at the largest vocabulary (one workgroup per row, 16 waves per
    row, where four-block batches would need more LDS than a workgroup may
    take, so the launch runs two): logits generated on the device, 16 rows
    compared with the oracle."""
    n, V, k = 512, L.GRAFT_MAX_VOCAB, 8
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    lg = torch.randn(n, V, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.full((n, k), -7, dtype=torch.int32, device=DEV)
    table = torch.zeros(V, k, dtype=torch.int32, device=DEV)
    row_tok = torch.arange(n, dtype=torch.int32, device=DEV)
    wsb = L.graft_workspace_bytes(n, V, k, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    L.graft_update_topk(n, V, k, L.DTYPE_BF16, lg.data_ptr(), None, None, row_tok.data_ptr(), table.data_ptr(),
                        None, out.data_ptr(), ws.data_ptr(), wsb, _s())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = np.random.default_rng(5).choice(n, size=16, replace=False)
    host = lg[torch.as_tensor(rows, device=DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got[rows], O.topk(host, k, "bf16"))
    np.testing.assert_array_equal(table.cpu().numpy()[rows], got[rows])


def test_topk_many_rows_and_ragged_split():
    # many rows, V chosen so the last range of a row is ragged
    rng = np.random.default_rng(4)
    V = 50_003
    rows = _bf16(rng.standard_normal((300, V)).astype(np.float32))
    got = gpu_topk(rows, 8, "bf16")
    assert (got == O.topk(rows, 8, "bf16")).all()


# ----------------------------------------------------------------------------- prune / retrieve / flatten

TOPO = G.static_tree()


def _random_logp(rng, B):
    par, lay, _ = TOPO
    out = []
    for b in range(B):
        mode = b % 5
        lp = np.log(rng.dirichlet(np.ones(8), size=60).max(1)).astype(np.float32)
        if mode == 0:
            lp[lay == 0] -= 1.5
        elif mode == 1:
            lp[lay == 1] -= 1.2
        elif mode == 2:
            lp[lay == 5] -= 3.0
        elif mode == 3:
            lp[:] = 0.0
        out.append(lp)
    return np.array(out, np.float32)


def _log_thr(t):
    return -math.inf if t == 0 else float(np.float32(math.log(t)))


def gpu_prune(parent, layer, score, mode, cfg_t, node_tau=0.0):
    B, Nd = score.shape
    cfg = L.prune_cfg(cfg_t["ckpt"], [_log_thr(t) for t in cfg_t["tau"]], cfg_t["keep"], cfg_t["tail_thr"],
                      _log_thr(node_tau) if node_tau > 0 else None)
    dp, dl, ds = _t(parent, torch.int32), _t(layer, torch.int32), _t(score, torch.float32)
    st = torch.zeros(B, dtype=torch.int32, device=DEV)
    nk = torch.zeros(B, dtype=torch.int32, device=DEV)
    kp = torch.zeros(B, Nd, dtype=torch.uint8, device=DEV)
    cum = torch.zeros(B, Nd, dtype=torch.float32, device=DEV)
    L.graft_prune_select(B, Nd, mode, dp.data_ptr(), dl.data_ptr(), ds.data_ptr(), cfg, st.data_ptr(),
                         nk.data_ptr(), kp.data_ptr(), cum.data_ptr() if mode == L.MODE_TREE else None, _s())
    torch.cuda.synchronize()
    return st.cpu().numpy(), nk.cpu().numpy(), kp.cpu().numpy(), cum.cpu().numpy()


CFG = {"ckpt": (0, 1, 5), "tau": (0.3, 0.2, 0.1), "keep": (8, 24, 40), "tail_thr": 0.5}


def test_prune_tree_parity():
    rng = np.random.default_rng(10)
    B = 67
    par, lay, _ = TOPO
    lp = _random_logp(rng, B)
    # exact ties at the keep boundary and thresholds hit exactly
    lp[5, :] = np.float32(math.log(0.7))
    lp[5, lay == 5] = np.float32(math.log(0.05))
    lp[6, lay == 0] = np.float32(math.log(0.3))
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    st, nk, kp, cum = gpu_prune(P, Ly, lp, L.MODE_TREE, CFG)
    o = O.prune_tree(P, Ly, lp, want_cum=True)
    np.testing.assert_array_equal(st, o["stage"])
    np.testing.assert_array_equal(nk, o["n_keep"])
    np.testing.assert_array_equal(kp, o["keep"])
    np.testing.assert_array_equal(cum.view(np.uint32), o["cum"].view(np.uint32))
    assert set(st.tolist()) == {0, 1, 2, 3}


@pytest.mark.parametrize("node_tau", [0.05, 0.2, 0.3, 0.5])
def test_prune_per_node_parity(node_tau):
    rng = np.random.default_rng(11)
    B = 53
    par, lay, _ = TOPO
    lp = _random_logp(rng, B)
    lp[0, :] = np.float32(math.log(node_tau))        # the threshold hit exactly: kept (>=)
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    st, nk, kp, cum = gpu_prune(P, Ly, lp, L.MODE_TREE, CFG, node_tau=node_tau)
    o = O.prune_tree(P, Ly, lp, want_cum=True, node_tau=node_tau)
    np.testing.assert_array_equal(st, o["stage"])
    np.testing.assert_array_equal(nk, o["n_keep"])
    np.testing.assert_array_equal(kp, o["keep"])
    np.testing.assert_array_equal(cum.view(np.uint32), o["cum"].view(np.uint32))


@pytest.mark.parametrize("tau", [(math.inf, 0, 0), (0, math.inf, 0), (0, 0, math.inf), (0, 0, 0)])
def test_prune_fixed_split_parity(tau):
    rng = np.random.default_rng(12)
    B = 31
    par, lay, _ = TOPO
    lp = _random_logp(rng, B)
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    cfg_t = dict(CFG, tau=tau)
    st, nk, kp, _ = gpu_prune(P, Ly, lp, L.MODE_TREE, cfg_t)
    o = O.prune_tree(P, Ly, lp, tau=tau)
    np.testing.assert_array_equal(st, o["stage"])
    np.testing.assert_array_equal(kp, o["keep"])
    assert len(set(st.tolist())) == 1


def test_prune_small_trees_and_unreached_checkpoints():
    rng = np.random.default_rng(11)
    par = np.array([-1, -1, 0, 0, 1, 2, 2, 3], np.int32)
    lay = np.array([0, 0, 1, 1, 1, 2, 2, 2], np.int32)
    B = 30
    lp = np.log(rng.uniform(0.01, 1.0, size=(B, 8))).astype(np.float32)
    cfg = dict(CFG, keep=(2, 5, 6))
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    st, nk, kp, cum = gpu_prune(P, Ly, lp, L.MODE_TREE, cfg)
    o = O.prune_tree(P, Ly, lp, cfg["ckpt"], cfg["tau"], cfg["keep"], want_cum=True)
    np.testing.assert_array_equal(st, o["stage"])
    np.testing.assert_array_equal(kp, o["keep"])
    np.testing.assert_array_equal(nk, o["n_keep"])


def gpu_ckpt_stats(parent, layer, score, ckpt=(0, 1, 5), keep=(8, 24, 40)):
    B, Nd = score.shape
    cfg = L.prune_cfg(ckpt, [0.0, 0.0, 0.0], keep, 0.5)
    dp, dl, ds = _t(parent, torch.int32), _t(layer, torch.int32), _t(score, torch.float32)
    out = torch.full((B, 3), -7.0, dtype=torch.float32, device=DEV)
    L.graft_checkpoint_stats(B, Nd, dp.data_ptr(), dl.data_ptr(), ds.data_ptr(), cfg, out.data_ptr(), _s())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_checkpoint_stats_parity():
    rng = np.random.default_rng(21)
    B = 67
    par, lay, _ = TOPO
    lp = _random_logp(rng, B)
    lp[3, :] = np.float32(math.log(0.7))              # ties across a whole layer
    lp[4, lay == 1] = -np.inf                          # probability 0 below layer 0
    lp[5, :] = 0.0                                     # probability 1 everywhere
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    got = gpu_ckpt_stats(P, Ly, lp)
    want = O.checkpoint_stats(P, Ly, lp)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert not np.isnan(got).any()
    # unreached checkpoints: layer 5 absent; too few nodes up to layer 1 for keep 9
    par_s = np.array([-1, -1, 0, 0, 1, 2, 2, 3], np.int32)
    lay_s = np.array([0, 0, 1, 1, 1, 2, 2, 2], np.int32)
    Bs = 20
    lps = np.log(rng.uniform(0.01, 1.0, size=(Bs, 8))).astype(np.float32)
    for keep in [(2, 5, 6), (2, 9, 6), (3, 5, 6)]:
        Ps, Ls = np.tile(par_s, (Bs, 1)), np.tile(lay_s, (Bs, 1))
        got = gpu_ckpt_stats(Ps, Ls, lps, keep=keep)
        want = O.checkpoint_stats(Ps, Ls, lps, keep=keep)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
        assert np.isnan(got[:, 2]).all()


def gpu_calibrate(samples, q):
    n = samples.shape[0]
    x = _t(samples if n else np.zeros((1, 3), np.float32), torch.float32)
    out = torch.full((3,), 7.0, dtype=torch.float32, device=DEV)
    L.graft_calibrate_thresholds(n, x.data_ptr(), q, out.data_ptr(), _s())
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n", [0, 1, 5, 80, 1000, 300_000])
def test_calibrate_parity(n):
    rng = np.random.default_rng(100 + n)
    x = (rng.standard_normal((n, 3)) * 3).astype(np.float32)
    x[:, 1] = np.round(x[:, 1] * 4) / 4                 # many ties
    if n >= 5:
        x[: n // 5, 2] = -np.inf
        x[n // 5: n // 5 + 2, 2] = np.inf
        x[-1, 0] = 0.0
    x[rng.random((n, 3)) < 0.2] = np.nan
    for q in [(0.0, 0.2, 1.0), (1e-6, 0.5, 0.3), (0.25, 0.25, 0.25), (1.0, 1.0, 1.0), (0.1, 0.9, 0.05)]:
        got = gpu_calibrate(x, q)
        want = O.calibrate(x, q)
        np.testing.assert_array_equal(got, want, err_msg="n=%d q=%s" % (n, q))


def test_calibrate_all_nan_and_constant_columns():
    x = np.full((50, 3), np.nan, np.float32)
    x[:, 1] = -2.5
    got = gpu_calibrate(x, (0.5, 0.5, 0.0))
    np.testing.assert_array_equal(got, [-np.inf, -2.5, -np.inf])


def test_prune_tail_parity():
    rng = np.random.default_rng(12)
    B = 40
    conf = np.sort(rng.beta(4, 2, size=(B, 16)), axis=1)[:, ::-1].astype(np.float32)
    conf[0] = 0.9
    conf[1] = 0.1
    conf[2] = 0.5
    conf[3, :] = np.float32(0.5) - np.float32(1e-7)
    conf[4] = rng.random(16).astype(np.float32)       # not monotone: prefix rule still applies
    st, nk, kp, _ = gpu_prune(np.zeros((B, 16), np.int32), np.zeros((B, 16), np.int32), conf, L.MODE_TAIL, CFG)
    o = O.prune_tail(conf, 0.5)
    np.testing.assert_array_equal(st, o["stage"])
    np.testing.assert_array_equal(nk, o["n_keep"])
    np.testing.assert_array_equal(kp, o["keep"])


def _tpl_dev(R, kind="chain", W=8, D=8, beta=(1, 1)):
    if kind == "chain":
        par, rk, dp = L.graft_template_master(W, D, R)
    else:
        par, rk, dp = L.graft_template_branching(W, D, beta[0], beta[1], R)
    tp, tr, td = (_t(np.array(x, np.int32)) for x in (par, rk, dp))
    return L.Template(len(par), tp.data_ptr(), tr.data_ptr(), td.data_ptr()), (tp, tr, td), len(par)


def _tpl_host(R, kind="chain", W=8, D=8, beta=(1, 1)):
    return O.template(W, D, R) if kind == "chain" else O.template_branching(W, D, beta, R)


def gpu_retrieve_tree(table, roots, n_keep, slots=60, R=52, V=None, **tk):
    B = len(roots)
    V = table.shape[0] if V is None else V
    tpl, keepalive, r_out = _tpl_dev(R, **tk)
    cfg = L.prune_cfg(CFG["ckpt"], [-1.0] * 3, CFG["keep"], 0.5)
    tb, rt, nk = _t(table, torch.int32), _t(roots, torch.int32), _t(n_keep, torch.int32)
    ret_tok = torch.zeros(B, r_out, dtype=torch.int32, device=DEV)
    ret_par = torch.zeros(B, r_out, dtype=torch.int32, device=DEV)
    n_ret = torch.zeros(B, dtype=torch.int32, device=DEV)
    L.graft_retrieve_expand(B, V, table.shape[1], L.MODE_TREE, slots, tb.data_ptr(), rt.data_ptr(),
                            nk.data_ptr(), None, 60, tpl, cfg, ret_tok.data_ptr(), ret_par.data_ptr(),
                            n_ret.data_ptr(), r_out, _s())
    torch.cuda.synchronize()
    return ret_tok.cpu().numpy(), ret_par.cpu().numpy(), n_ret.cpu().numpy()


def test_retrieve_tree_parity():
    rng = np.random.default_rng(13)
    V = 151936
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    B = 37
    roots = rng.integers(0, V, size=B).astype(np.int32)
    n_keep = rng.choice([8, 24, 40, 60], size=B).astype(np.int32)
    rt, rp, nr = gpu_retrieve_tree(table, roots, n_keep)
    o = O.retrieve_tree(table, roots, n_keep, 60, O.template(8, 8, 52))
    np.testing.assert_array_equal(nr, o["n_ret"])
    np.testing.assert_array_equal(rt, o["ret_tok"])
    np.testing.assert_array_equal(rp, o["ret_parent"])


@pytest.mark.parametrize("kind,W,D,beta,R", [
    ("branching", 8, 8, (1, 1), 52),     # branching: several ranks at every depth
    ("branching", 8, 12, (0, 1), 64),    # breadth-first: depth 2 only within 64 nodes
    ("branching", 2, 30, (100, 1), 52),  # a depth-30 rank-0 chain: the level-by-level path
    ("chain", 8, 2, (1, 1), 52),         # 16 nodes: less than most budgets (empty slots)
    ("branching", 4, 3, (1, 2), 20),
    ("chain", 4, 16, (1, 1), 52),        # rank chains to depth 16: a 16-level path walk
    ("chain", 8, 1, (1, 1), 52),         # root children only: every node reads the root's row
])
def test_retrieve_tree_parity_templates(kind, W, D, beta, R):
    rng = np.random.default_rng(14)
    V = 20011
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    B = 29
    roots = rng.integers(0, V, size=B).astype(np.int32)
    roots[:2] = [0, V - 1]                # the first and the last matrix row
    n_keep = rng.choice([8, 24, 40, 60], size=B).astype(np.int32)
    tpl = _tpl_host(R, kind, W, D, beta)
    o = O.retrieve_tree(table, roots, n_keep, 60, tpl)
    rt, rp, nr = gpu_retrieve_tree(table, roots, n_keep, R=R, kind=kind, W=W, D=D, beta=beta)
    np.testing.assert_array_equal(nr, o["n_ret"])
    np.testing.assert_array_equal(rp, o["ret_parent"])
    np.testing.assert_array_equal(rt, o["ret_tok"])


def test_retrieve_tail_parity():
    rng = np.random.default_rng(14)
    V = 151936
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    B = 33
    roots = rng.integers(0, V, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, 16)).astype(np.int32)
    n_keep = rng.integers(0, 17, size=B).astype(np.int32)
    n_keep[:3] = [0, 16, 1]
    tb, r, nk, dt = (_t(x, torch.int32) for x in (table, roots, n_keep, d_tok))
    ret_tok = torch.zeros(B, 16, dtype=torch.int32, device=DEV)
    ret_par = torch.zeros(B, 16, dtype=torch.int32, device=DEV)
    n_ret = torch.zeros(B, dtype=torch.int32, device=DEV)
    L.graft_retrieve_expand(B, V, 8, L.MODE_TAIL, 16, tb.data_ptr(), r.data_ptr(), nk.data_ptr(), dt.data_ptr(),
                            16, None, None, ret_tok.data_ptr(), ret_par.data_ptr(), n_ret.data_ptr(), 16, _s())
    torch.cuda.synchronize()
    o = O.retrieve_tail(table, roots, d_tok, n_keep)
    np.testing.assert_array_equal(n_ret.cpu().numpy(), o["n_ret"])
    np.testing.assert_array_equal(ret_tok.cpu().numpy(), o["ret_tok"])
    np.testing.assert_array_equal(ret_par.cpu().numpy(), o["ret_parent"])


def gpu_flatten(layout, T1, roots, base, d_tok, d_parent, keep, n_keep, ret):
    B, Nd = d_tok.shape
    r_out = ret["ret_tok"].shape[1]
    args = [_t(x, torch.int32) for x in (roots, base, d_tok, d_parent)]
    kp = _t(keep, torch.uint8)
    nk = _t(n_keep, torch.int32)
    rt, rp, nr = (_t(ret[k], torch.int32) for k in ("ret_tok", "ret_parent", "n_ret"))
    outs = [torch.zeros(B, T1, dtype=torch.int32, device=DEV) for _ in range(4)]
    anc = torch.zeros(B, T1, dtype=torch.int64, device=DEV)
    src = torch.full((B, T1), 99, dtype=torch.uint8, device=DEV)
    L.graft_build_tree_mask(B, Nd, T1, L.LAYOUT[layout], args[0].data_ptr(), args[1].data_ptr(),
                            args[2].data_ptr(), args[3].data_ptr(), kp.data_ptr(), nk.data_ptr(),
                            rt.data_ptr(), rp.data_ptr(), nr.data_ptr(), r_out,
                            *[o.data_ptr() for o in outs], anc.data_ptr(), src.data_ptr(), _s())
    torch.cuda.synchronize()
    res = [o.cpu().numpy() for o in outs]
    return {"tok": res[0], "parent": res[1], "depth": res[2], "pos_id": res[3],
            "anc": anc.cpu().numpy().view(np.uint64), "row_src": src.cpu().numpy()}


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_flatten_tree_parity(layout):
    rng = np.random.default_rng(15)
    B = 45
    V = 5000
    par, lay, _ = TOPO
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    lp = _random_logp(rng, B)
    pr = O.prune_tree(P, Ly, lp)
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, O.template(8, 8, 52))
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    base = rng.integers(0, 100000, size=B).astype(np.int32)
    got = gpu_flatten(layout, 61, roots, base, d_tok, P, pr["keep"], pr["n_keep"], ret)
    want = O.flatten(layout, 61, roots, base, d_tok, P, pr["keep"], pr["n_keep"], ret)
    for key in ("tok", "parent", "depth", "pos_id", "anc", "row_src"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)


def test_flatten_chain_parity():
    rng = np.random.default_rng(16)
    B = 30
    V = 1000
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, 16)).astype(np.int32)
    conf = rng.random((B, 16)).astype(np.float32)
    conf[0] = 0.9
    conf[1] = 0.1
    pr = O.prune_tail(conf, 0.5)
    ret = O.retrieve_tail(table, roots, d_tok, pr["n_keep"])
    base = rng.integers(0, 1000, size=B).astype(np.int32)
    dpar = np.tile(np.arange(-1, 15, dtype=np.int32), (B, 1))
    got = gpu_flatten("chain", 17, roots, base, d_tok, dpar, pr["keep"], pr["n_keep"], ret)
    want = O.flatten("chain", 17, roots, base, d_tok, dpar, pr["keep"], pr["n_keep"], ret)
    for key in ("tok", "parent", "depth", "pos_id", "anc", "row_src"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)


# ----------------------------------------------------------------------------- verify / update

def gpu_verify(rows, tok, parent, depth, k=8, dtype="bf16", want_prob=False, base=None):
    B, T1 = tok.shape
    V = rows.shape[-1]
    lg = _t(rows.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else _t(rows.view(np.float32))
    dt = L.DTYPE_BF16 if dtype == "bf16" else L.DTYPE_F32
    tk = torch.zeros(B, T1, k, dtype=torch.int32, device=DEV)
    pr = torch.zeros(B, T1, k, dtype=torch.float32, device=DEV) if want_prob else None
    al = torch.zeros(B, dtype=torch.int32, device=DEV)
    ai = torch.zeros(B, T1 - 1, dtype=torch.int32, device=DEV)
    bo = torch.zeros(B, dtype=torch.int32, device=DEV)
    bp = _t(base if base is not None else np.zeros(B, np.int32), torch.int32)
    t_, p_, d_ = (_t(x, torch.int32) for x in (tok, parent, depth))
    wsb = L.graft_workspace_bytes(B * T1, V, k, dt)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    L.graft_verify_accept(B, T1, V, k, dt, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                          tk.data_ptr(), pr.data_ptr() if want_prob else None, None, al.data_ptr(), ai.data_ptr(),
                          T1 - 1, bo.data_ptr(), bp.data_ptr(), ws.data_ptr(), wsb, _s())
    torch.cuda.synchronize()
    out = {"topk": tk.cpu().numpy(), "accept_len": al.cpu().numpy(), "accept_idx": ai.cpu().numpy(),
           "bonus": bo.cpu().numpy(), "base_pos": bp.cpu().numpy()}
    if want_prob:
        out["topk_prob"] = pr.cpu().numpy()
    return out


def _random_flat_trees(rng, B, T1, V):
    tok = rng.integers(0, V, size=(B, T1)).astype(np.int32)
    par = np.zeros((B, T1), np.int32)
    for b in range(B):
        par[b, 0] = -1
        for f in range(1, T1):
            par[b, f] = rng.integers(max(0, f - 6), f)
    dep = np.zeros((B, T1), np.int32)
    for b in range(B):
        for f in range(1, T1):
            dep[b, f] = dep[b, par[b, f]] + 1
    return tok, par, dep


@pytest.mark.parametrize("T1,V", [(61, 5), (61, 3), (17, 4), (64, 2), (1, 7), (2, 3)])
def test_verify_accept_parity(T1, V):
    rng = np.random.default_rng(T1 * 100 + V)
    B = 29
    tok, par, dep = _random_flat_trees(rng, B, T1, V)
    rows = _bf16(rng.standard_normal((B, T1, V)).astype(np.float32))
    base = rng.integers(0, 1000, size=B).astype(np.int32)
    got = gpu_verify(rows, tok, par, dep, k=min(8, V), base=base)
    want_tk = O.topk(rows.reshape(B * T1, V), min(8, V), "bf16").reshape(B, T1, -1)
    np.testing.assert_array_equal(got["topk"], want_tk)
    acc = O.accept(tok, par, want_tk[:, :, 0], max(T1 - 1, 0) if T1 > 1 else 0)
    np.testing.assert_array_equal(got["accept_len"], acc["accept_len"])
    np.testing.assert_array_equal(got["bonus"], acc["bonus"])
    if T1 > 1:
        np.testing.assert_array_equal(got["accept_idx"], acc["accept_idx"])
    np.testing.assert_array_equal(got["base_pos"], base + acc["accept_len"] + 1)
    if T1 > 1:
        assert got["accept_len"].max() > 0


def test_verify_with_probabilities():
    rng = np.random.default_rng(20)
    B, T1, V = 4, 61, 128256
    tok, par, dep = _random_flat_trees(rng, B, T1, 50)
    rows = _bf16((rng.standard_normal((B, T1, V)) * 1.5).astype(np.float32))
    got = gpu_verify(rows, tok, par, dep, want_prob=True)
    tk, p = O.topk(rows.reshape(-1, V), 8, "bf16", want_prob=True)
    np.testing.assert_array_equal(got["topk"].reshape(-1, 8), tk)
    np.testing.assert_allclose(got["topk_prob"].reshape(-1, 8), p, rtol=1e-5, atol=0)


def gpu_update(table, row_tok, topk_rows):
    V, k = table.shape
    tb = _t(table, torch.int32)
    rt = _t(row_tok, torch.int32)
    tk = _t(topk_rows, torch.int32)
    L.graft_update_topk(len(row_tok), V, k, L.DTYPE_BF16, None, tk.data_ptr(), None, rt.data_ptr(),
                        tb.data_ptr(), None, None, None, 0, _s())
    torch.cuda.synchronize()
    return tb.cpu().numpy()


@pytest.mark.parametrize("n,ntok", [(976, 151936), (976, 1), (976, 7), (2048, 300), (9000, 50), (17, 17), (1, 5)])
def test_update_parity_collisions(n, ntok):
    rng = np.random.default_rng(n + ntok)
    V, k = max(ntok, 64), 8
    table = rng.integers(0, V, size=(V, k)).astype(np.int32)
    row_tok = rng.integers(0, ntok, size=n).astype(np.int32)
    tk = rng.integers(0, V, size=(n, k)).astype(np.int32)
    got = gpu_update(table.copy(), row_tok, tk)
    want = table.copy()
    O.update(want, row_tok, tk)
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------------------- fused entry points

@pytest.mark.parametrize("kind,W,D,beta", [("chain", 8, 8, (1, 1)), ("branching", 8, 8, (1, 1)),
                                           ("chain", 8, 2, (1, 1)), ("branching", 2, 30, (100, 1))],
                         ids=["chain8x8", "branching8x8", "chain8x2_empty_rows", "deep_chain30"])
@pytest.mark.parametrize("ahead", [False, True], ids=["one_launch", "retrieval_ahead"])
def test_build_hybrid_tree_matches_oracle_tree(kind, W, D, beta, ahead):
    """graft_build_hybrid_tree, or graft_retrieve_expand without n_keep (the
    whole template before the draft exists) followed by
    graft_build_after_retrieval: the same outputs as the oracle's step."""
    rng = np.random.default_rng(30)
    B, V = 37, 5000
    par, lay, _ = TOPO
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    lp = _random_logp(rng, B)
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    base = rng.integers(0, 100000, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    tpl, keepalive, r_out = _tpl_dev(52, kind, W, D, beta)
    tpl_h = _tpl_host(52, kind, W, D, beta)
    cfg = L.prune_cfg(CFG["ckpt"], [float(np.float32(math.log(t))) for t in CFG["tau"]], CFG["keep"], 0.5)
    for layout in ("compact", "in_place"):
        ins = [_t(x, torch.int32) for x in (table, roots, base, P, Ly)]
        sc, dt = _t(lp, torch.float32), _t(d_tok, torch.int32)
        i32 = dict(dtype=torch.int32, device=DEV)
        st, nk, nr = (torch.zeros(B, **i32) for _ in range(3))
        kp = torch.zeros(B, 60, dtype=torch.uint8, device=DEV)
        cum = torch.zeros(B, 60, dtype=torch.float32, device=DEV)
        rt, rp = torch.zeros(B, r_out, **i32), torch.zeros(B, r_out, **i32)
        tok, par_o, dep, pos = (torch.zeros(B, 61, **i32) for _ in range(4))
        anc = torch.zeros(B, 61, dtype=torch.int64, device=DEV)
        src = torch.full((B, 61), 99, dtype=torch.uint8, device=DEV)
        if not ahead:
            L.graft_build_hybrid_tree(B, 60, 61, L.MODE_TREE, L.LAYOUT[layout], 60, cfg, tpl, V, 8,
                                      ins[0].data_ptr(), ins[1].data_ptr(), ins[2].data_ptr(), ins[3].data_ptr(),
                                      ins[4].data_ptr(), sc.data_ptr(), dt.data_ptr(), st.data_ptr(),
                                      nk.data_ptr(), kp.data_ptr(), cum.data_ptr(), rt.data_ptr(), rp.data_ptr(),
                                      nr.data_ptr(), r_out, tok.data_ptr(), par_o.data_ptr(), dep.data_ptr(),
                                      pos.data_ptr(), anc.data_ptr(), src.data_ptr(), _s())
        else:
            L.graft_retrieve_expand(B, V, 8, L.MODE_TREE, 60, ins[0].data_ptr(), ins[1].data_ptr(), None, None,
                                    60, tpl, cfg, rt.data_ptr(), rp.data_ptr(), nr.data_ptr(), r_out, _s())
            torch.cuda.synchronize()
            full = O.retrieve_tree(table, roots, np.zeros(B, np.int32), 60, tpl_h)
            np.testing.assert_array_equal(nr.cpu().numpy(), full["n_ret"])
            np.testing.assert_array_equal(rt.cpu().numpy()[:, :full["ret_tok"].shape[1]], full["ret_tok"])
            L.graft_build_after_retrieval(B, 60, 61, L.LAYOUT[layout], 60, cfg, ins[1].data_ptr(),
                                          ins[2].data_ptr(), ins[3].data_ptr(), ins[4].data_ptr(), sc.data_ptr(),
                                          dt.data_ptr(), st.data_ptr(), nk.data_ptr(), kp.data_ptr(),
                                          cum.data_ptr(), rt.data_ptr(), rp.data_ptr(), nr.data_ptr(), r_out,
                                          tok.data_ptr(), par_o.data_ptr(), dep.data_ptr(), pos.data_ptr(),
                                          anc.data_ptr(), src.data_ptr(), _s())
        torch.cuda.synchronize()
        pr = O.prune_tree(P, Ly, lp, want_cum=True)
        ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, tpl_h)
        fl = O.flatten(layout, 61, roots, base, d_tok, P, pr["keep"], pr["n_keep"], ret)
        np.testing.assert_array_equal(st.cpu().numpy(), pr["stage"])
        np.testing.assert_array_equal(nk.cpu().numpy(), pr["n_keep"])
        np.testing.assert_array_equal(kp.cpu().numpy(), pr["keep"])
        np.testing.assert_array_equal(cum.cpu().numpy().view(np.uint32), pr["cum"].view(np.uint32))
        np.testing.assert_array_equal(nr.cpu().numpy(), ret["n_ret"])
        np.testing.assert_array_equal(rt.cpu().numpy(), ret["ret_tok"])
        np.testing.assert_array_equal(rp.cpu().numpy(), ret["ret_parent"])
        for name, got in (("tok", tok), ("parent", par_o), ("depth", dep), ("pos_id", pos)):
            np.testing.assert_array_equal(got.cpu().numpy(), fl[name], err_msg=(layout, name))
        np.testing.assert_array_equal(anc.cpu().numpy().view(np.uint64), fl["anc"])
        np.testing.assert_array_equal(src.cpu().numpy(), fl["row_src"])


@pytest.mark.parametrize("B", [1, 33])
def test_build_hybrid_tree_tail_matches_oracle(B):
    """graft_build_hybrid_tree in TAIL mode (one launch: prefix, chain of
    rank-0 successors, chain rows) against the oracle's three TAIL steps, with
    prefixes of every length including none (the chain starts at the root) and
    the whole block (nothing retrieved), and a table with self-loops."""
    rng = np.random.default_rng(41 + B)
    V = 3001
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    loops = rng.choice(V, size=300, replace=False)
    table[loops, 0] = loops                                  # x -> x: the chain repeats a token
    roots = rng.integers(0, V, size=B).astype(np.int32)
    base = rng.integers(0, 100000, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, 16)).astype(np.int32)
    d_tok[:, 3] = loops[0]
    conf = rng.random((B, 16)).astype(np.float32)
    for b in range(B):                                        # prefix length b % 17 (then one below 0.5)
        p = (b * 7) % 17 if B > 1 else 15
        conf[b, :p] = 0.5 + 0.5 * rng.random(p).astype(np.float32)
        if p < 16:
            conf[b, p] = 0.49
    if B > 1:
        conf[0] = 0.1                                         # p = 0: chain from the root
        conf[1] = 1.0                                         # p = 16: nothing retrieved
        conf[2, 0], conf[2, 1] = 0.5, np.float32(0.49999997)  # exactly at the threshold, then just below
    dpar = np.tile(np.arange(-1, 15, dtype=np.int32), (B, 1))
    lay = np.tile(np.arange(16, dtype=np.int32), (B, 1))
    cfg = L.prune_cfg(CFG["ckpt"], [float(np.float32(math.log(t))) for t in CFG["tau"]], CFG["keep"], 0.5)
    i32 = dict(dtype=torch.int32, device=DEV)
    ins = [_t(x, torch.int32) for x in (table, roots, base, dpar, lay, d_tok)]
    sc = _t(conf, torch.float32)
    st, nk, nr = (torch.full((B,), 77, **i32) for _ in range(3))
    kp = torch.full((B, 16), 9, dtype=torch.uint8, device=DEV)
    rt, rp = torch.full((B, 16), 77, **i32), torch.full((B, 16), 77, **i32)
    tok, par_o, dep, pos = (torch.full((B, 17), 77, **i32) for _ in range(4))
    anc = torch.zeros(B, 17, dtype=torch.int64, device=DEV)
    src = torch.full((B, 17), 99, dtype=torch.uint8, device=DEV)
    L.graft_build_hybrid_tree(B, 16, 17, L.MODE_TAIL, L.LAYOUT["chain"], 16, cfg, None, V, 8,
                              ins[0].data_ptr(), ins[1].data_ptr(), ins[2].data_ptr(), ins[3].data_ptr(),
                              ins[4].data_ptr(), sc.data_ptr(), ins[5].data_ptr(), st.data_ptr(), nk.data_ptr(),
                              kp.data_ptr(), None, rt.data_ptr(), rp.data_ptr(), nr.data_ptr(), 16,
                              tok.data_ptr(), par_o.data_ptr(), dep.data_ptr(), pos.data_ptr(), anc.data_ptr(),
                              src.data_ptr(), _s())
    torch.cuda.synchronize()
    pr = O.prune_tail(conf, 0.5)
    ret = O.retrieve_tail(table, roots, d_tok, pr["n_keep"])
    fl = O.flatten("chain", 17, roots, base, d_tok, dpar, pr["keep"], pr["n_keep"], ret)
    if B > 1:
        assert pr["n_keep"][0] == 0 and pr["n_keep"][1] == 16 and pr["n_keep"][2] == 1
        assert len(set(pr["n_keep"].tolist())) == 17            # every prefix length occurs
    np.testing.assert_array_equal(st.cpu().numpy(), pr["stage"])
    np.testing.assert_array_equal(nk.cpu().numpy(), pr["n_keep"])
    np.testing.assert_array_equal(kp.cpu().numpy(), pr["keep"])
    np.testing.assert_array_equal(nr.cpu().numpy(), ret["n_ret"])
    np.testing.assert_array_equal(rt.cpu().numpy(), ret["ret_tok"])
    np.testing.assert_array_equal(rp.cpu().numpy(), ret["ret_parent"])
    for name, got in (("tok", tok), ("parent", par_o), ("depth", dep), ("pos_id", pos)):
        np.testing.assert_array_equal(got.cpu().numpy(), fl[name], err_msg=name)
    np.testing.assert_array_equal(anc.cpu().numpy().view(np.uint64), fl["anc"])
    np.testing.assert_array_equal(src.cpu().numpy(), fl["row_src"])


def test_verify_update_matches_oracle_with_collisions():
    rng = np.random.default_rng(31)
    B, T1, V = 16, 61, 20000
    tok, par, dep = _random_flat_trees(rng, B, T1, 40)     # 40 distinct tokens: many collisions
    tok[3] = 7                                              # a whole request on one token
    rows = _bf16(rng.standard_normal((B, T1, V)).astype(np.float32))
    table0 = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    lg = _t(rows.view(np.int16)).view(torch.bfloat16)
    i32 = dict(dtype=torch.int32, device=DEV)
    tb = _t(table0, torch.int32)
    tk = torch.zeros(B, T1, 8, **i32)
    al, bo, bp = torch.zeros(B, **i32), torch.zeros(B, **i32), torch.zeros(B, **i32)
    ai = torch.zeros(B, T1 - 1, **i32)
    t_, p_, d_ = (_t(x, torch.int32) for x in (tok, par, dep))
    wsb = L.graft_workspace_bytes(B * T1, V, 8, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    want_tab = table0.copy()
    for rep in range(3):        # repeated calls: the workspace must come back zeroed
        L.graft_verify_update(B, T1, V, 8, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                              tb.data_ptr(), None, tk.data_ptr(), None, None, al.data_ptr(), ai.data_ptr(), T1 - 1,
                              bo.data_ptr(), bp.data_ptr(), ws.data_ptr(), wsb, _s())
        torch.cuda.synchronize()
        want_tk = O.topk(rows.reshape(-1, V), 8, "bf16").reshape(B, T1, 8)
        acc = O.accept(tok, par, want_tk[:, :, 0], T1 - 1)
        O.update(want_tab, tok.reshape(-1), want_tk.reshape(-1, 8))
        np.testing.assert_array_equal(tk.cpu().numpy(), want_tk)
        np.testing.assert_array_equal(al.cpu().numpy(), acc["accept_len"])
        np.testing.assert_array_equal(ai.cpu().numpy(), acc["accept_idx"])
        np.testing.assert_array_equal(bo.cpu().numpy(), acc["bonus"])
        np.testing.assert_array_equal(tb.cpu().numpy(), want_tab)
        rows = _bf16(rng.standard_normal((B, T1, V)).astype(np.float32))
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("kind,B,T1", [("verify", 16, 61), ("verify", 25, 41), ("ingest", 1, 0)],
                         ids=["verify_976", "verify_1025", "ingest_1024"])
def test_holder_scan_collisions(kind, B, T1):
    """Merge-wave launches of at most 1025 rows find each token's last holder by
    comparing its token with the later rows' tokens (no registration workgroup;
    at 1025 rows the first row reads all 1024 later ones): with the rows' tokens
    drawn from 37 values (many holders per token), some rows empty (-1) and two
    calls in a row, the matrix and every output match the oracle's sequential
    overwrite."""
    rng = np.random.default_rng(37 + B)
    V, k = 30011, 8
    n = B * T1 if kind == "verify" else 1024
    plan = L.graft_launch_plan(n, V, L.DTYPE_BF16, T1)
    assert plan["merge_wave"] == 1 and plan["holder_scan"] == 1
    vals = rng.choice(V, size=37, replace=False).astype(np.int32)
    table0 = rng.integers(0, V, size=(V, k)).astype(np.int32)
    tb = _t(table0, torch.int32)
    want_tab = table0.copy()
    wsb = L.graft_workspace_bytes(n, V, k, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    for call in range(2):
        tok = vals[rng.integers(0, len(vals), size=n)]
        tok[rng.random(n) < 0.05] = -1
        if kind == "verify":
            tok = tok.reshape(B, T1)
            tok[:, 0] = vals[0]                  # every root holds one token
            _, par, dep = _random_flat_trees(rng, B, T1, V)
        rows = _bf16(rng.standard_normal((n, V)).astype(np.float32))
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)
        t_ = _t(tok.reshape(-1), torch.int32)
        tk = torch.zeros(n, k, **i32)
        print("%s holder scan: %d rows, call %d" % (kind, n, call), flush=True)
        want_tk = O.topk(rows, k, "bf16")
        if kind == "verify":
            al, bo = torch.zeros(B, **i32), torch.zeros(B, **i32)
            ai = torch.zeros(B, T1 - 1, **i32)
            p_, d_ = _t(par, torch.int32), _t(dep, torch.int32)
            L.graft_verify_update(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(),
                                  d_.data_ptr(), tb.data_ptr(), None, tk.data_ptr(), None, None, al.data_ptr(),
                                  ai.data_ptr(), T1 - 1, bo.data_ptr(), None, ws.data_ptr(), wsb, _s())
            torch.cuda.synchronize()
            acc = O.accept(tok, par, want_tk.reshape(B, T1, k)[:, :, 0], T1 - 1)
            np.testing.assert_array_equal(al.cpu().numpy(), acc["accept_len"])
            np.testing.assert_array_equal(ai.cpu().numpy(), acc["accept_idx"])
            np.testing.assert_array_equal(bo.cpu().numpy(), acc["bonus"])
        else:
            L.graft_update_topk(n, V, k, L.DTYPE_BF16, lg.data_ptr(), None, None, t_.data_ptr(), tb.data_ptr(),
                                None, tk.data_ptr(), ws.data_ptr(), wsb, _s())
            torch.cuda.synchronize()
        O.update(want_tab, tok.reshape(-1), want_tk)
        np.testing.assert_array_equal(tk.cpu().numpy(), want_tk)
        np.testing.assert_array_equal(tb.cpu().numpy(), want_tab)
        assert not ws[L.GRAFT_WS_COUNTER_BYTES:].any().item()


def _chain_batch(rng, B, T1, V):
    """Chain trees whose first p_b candidates carry the target's bumped greedy
    token: logits N(0, 1) with +6 at a random column per row."""
    z = rng.standard_normal((B, T1, V)).astype(np.float32)
    col = rng.integers(0, V, size=(B, T1))
    np.put_along_axis(z, col[:, :, None], 6.0, axis=2)
    rows = _bf16(z)
    p = rng.integers(0, T1, size=B)
    tok = rng.integers(0, V, size=(B, T1)).astype(np.int32)
    for b in range(B):
        tok[b, 1:p[b] + 1] = col[b, :p[b]]
    par = np.tile(np.arange(-1, T1 - 1, dtype=np.int32), (B, 1))
    dep = np.tile(np.arange(T1, dtype=np.int32), (B, 1))
    return rows, tok, par, dep


def test_verify_update_batch_above_resident_coordinators():
    """8192 requests of 17 rows at V = 1024: one coordinator wavefront per request
    would need 8192 workgroups ahead of the rows, more than the chip holds at once;
    the launch caps them (each wavefront watches many requests).  Every output and
    the matrix match the oracle on two calls in a row, the second with fewer
    requests on the same workspace."""
    rng = np.random.default_rng(8192)
    V, T1, k = 1024, 17, 8
    plan = L.graft_launch_plan(8192 * T1, V, L.DTYPE_BF16, T1)
    assert plan["coord_groups"] == L.GRAFT_MAX_COORD_GROUPS and plan["waves_per_group"] == 1
    i32 = dict(dtype=torch.int32, device=DEV)
    table0 = rng.integers(0, V, size=(V, k)).astype(np.int32)
    tb = _t(table0, torch.int32)
    want_tab = table0.copy()
    wsb = L.graft_workspace_bytes(8192 * T1, V, k, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    for B in (8192, 3000):
        rows, tok, par, dep = _chain_batch(rng, B, T1, V)
        base = rng.integers(0, 10000, size=B).astype(np.int32)
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)
        tk = torch.zeros(B, T1, k, **i32)
        al, bo = torch.zeros(B, **i32), torch.zeros(B, **i32)
        bp = _t(base, torch.int32)
        ai = torch.zeros(B, T1 - 1, **i32)
        t_, p_, d_ = (_t(x, torch.int32) for x in (tok, par, dep))
        print("verify_update B=%d T1=%d V=%d" % (B, T1, V), flush=True)
        L.graft_verify_update(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                              tb.data_ptr(), None, tk.data_ptr(), None, None, al.data_ptr(), ai.data_ptr(), T1 - 1,
                              bo.data_ptr(), bp.data_ptr(), ws.data_ptr(), wsb, _s())
        torch.cuda.synchronize()
        want_tk = O.topk(rows.reshape(-1, V), k, "bf16").reshape(B, T1, k)
        acc = O.accept(tok, par, want_tk[:, :, 0], T1 - 1)
        O.update(want_tab, tok.reshape(-1), want_tk.reshape(-1, k))
        np.testing.assert_array_equal(tk.cpu().numpy(), want_tk)
        np.testing.assert_array_equal(al.cpu().numpy(), acc["accept_len"])
        np.testing.assert_array_equal(ai.cpu().numpy(), acc["accept_idx"])
        np.testing.assert_array_equal(bo.cpu().numpy(), acc["bonus"])
        np.testing.assert_array_equal(bp.cpu().numpy(), base + acc["accept_len"] + 1)
        np.testing.assert_array_equal(tb.cpu().numpy(), want_tab)
        assert acc["accept_len"].max() >= T1 - 2
    assert not ws[L.GRAFT_WS_COUNTER_BYTES:].any().item()      # left zero-filled past the launch counters


def test_verify_update_launch_counters_wrap():
    """The per-row launch counters are 32-bit and wrap: with both counters of
    every row preset to 2^32 - 2 (and stale completion words of the counter
    before), three calls in a row run through 2^32 - 1, 0 and 1 and each still
    matches the oracle."""
    rng = np.random.default_rng(4242)
    V, k, B, T1 = 30011, 8, 16, 61
    assert L.graft_launch_plan(B * T1, V, L.DTYPE_BF16, T1)["launch_counters"] == 1
    i32 = dict(dtype=torch.int32, device=DEV)
    table0 = rng.integers(0, V, size=(V, k)).astype(np.int32)
    tb = _t(table0, torch.int32)
    want_tab = table0.copy()
    wsb = L.graft_workspace_bytes(B * T1, V, k, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    n_tag = L.GRAFT_WS_COUNTER_BYTES // 12
    start = (1 << 32) - 2
    words = np.full(n_tag, (start << 32) | 1, dtype=np.uint64)  # a stale word of counter 2^32 - 2, greedy 0
    ws[:n_tag * 8] = torch.from_numpy(words.view(np.uint8)).to(DEV)
    ws[n_tag * 8:n_tag * 12] = torch.from_numpy(np.full(n_tag, start, dtype=np.uint32).view(np.uint8)).to(DEV)
    for call in range(3):
        rows, tok, par, dep = _chain_batch(rng, B, T1, V)
        base = rng.integers(0, 10000, size=B).astype(np.int32)
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)
        tk = torch.zeros(B, T1, k, **i32)
        al, bo = torch.zeros(B, **i32), torch.zeros(B, **i32)
        bp = _t(base, torch.int32)
        ai = torch.zeros(B, T1 - 1, **i32)
        t_, p_, d_ = (_t(x, torch.int32) for x in (tok, par, dep))
        print("verify_update call %d, counters at %d" % (call, (start + call + 1) % (1 << 32)), flush=True)
        L.graft_verify_update(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                              tb.data_ptr(), None, tk.data_ptr(), None, None, al.data_ptr(), ai.data_ptr(), T1 - 1,
                              bo.data_ptr(), bp.data_ptr(), ws.data_ptr(), wsb, _s())
        torch.cuda.synchronize()
        want_tk = O.topk(rows.reshape(-1, V), k, "bf16").reshape(B, T1, k)
        acc = O.accept(tok, par, want_tk[:, :, 0], T1 - 1)
        O.update(want_tab, tok.reshape(-1), want_tk.reshape(-1, k))
        np.testing.assert_array_equal(tk.cpu().numpy(), want_tk)
        np.testing.assert_array_equal(al.cpu().numpy(), acc["accept_len"])
        np.testing.assert_array_equal(ai.cpu().numpy(), acc["accept_idx"])
        np.testing.assert_array_equal(bo.cpu().numpy(), acc["bonus"])
        np.testing.assert_array_equal(bp.cpu().numpy(), base + acc["accept_len"] + 1)
        np.testing.assert_array_equal(tb.cpu().numpy(), want_tab)
        ctr = ws[n_tag * 8:n_tag * 12].view(torch.int32).cpu().numpy().view(np.uint32)
        assert (ctr[:B * T1] == (start + call + 1) % (1 << 32)).all()
        assert (ctr[B * T1:] == start).all()


def test_verify_update_merge_wave_past_the_counters():
    """A merge-wave verify launch of more rows than the launch counters cover
    (16385 rows of V = 8192) falls back to completion words that its
    coordinators clear; the next call on the same workspace (15000 rows) uses the
    counters.  Both match the oracle and leave the workspace past the counters
    zero-filled."""
    rng = np.random.default_rng(16385)
    V, k = 8192, 8
    calls = [(3277, 5), (3000, 5)]
    plans = [L.graft_launch_plan(B * T1, V, L.DTYPE_BF16, T1) for B, T1 in calls]
    assert [(p["merge_wave"], p["launch_counters"]) for p in plans] == [(1, 0), (1, 1)]
    i32 = dict(dtype=torch.int32, device=DEV)
    table0 = rng.integers(0, V, size=(V, k)).astype(np.int32)
    tb = _t(table0, torch.int32)
    want_tab = table0.copy()
    wsb = L.graft_workspace_bytes(3277 * 5, V, k, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    for B, T1 in calls:
        rows, tok, par, dep = _chain_batch(rng, B, T1, V)
        base = rng.integers(0, 10000, size=B).astype(np.int32)
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)
        tk = torch.zeros(B, T1, k, **i32)
        al, bo = torch.zeros(B, **i32), torch.zeros(B, **i32)
        bp = _t(base, torch.int32)
        ai = torch.zeros(B, T1 - 1, **i32)
        t_, p_, d_ = (_t(x, torch.int32) for x in (tok, par, dep))
        print("verify_update B=%d T1=%d V=%d" % (B, T1, V), flush=True)
        L.graft_verify_update(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                              tb.data_ptr(), None, tk.data_ptr(), None, None, al.data_ptr(), ai.data_ptr(), T1 - 1,
                              bo.data_ptr(), bp.data_ptr(), ws.data_ptr(), wsb, _s())
        torch.cuda.synchronize()
        want_tk = O.topk(rows.reshape(-1, V), k, "bf16").reshape(B, T1, k)
        acc = O.accept(tok, par, want_tk[:, :, 0], T1 - 1)
        O.update(want_tab, tok.reshape(-1), want_tk.reshape(-1, k))
        np.testing.assert_array_equal(tk.cpu().numpy(), want_tk)
        np.testing.assert_array_equal(al.cpu().numpy(), acc["accept_len"])
        np.testing.assert_array_equal(ai.cpu().numpy(), acc["accept_idx"])
        np.testing.assert_array_equal(bo.cpu().numpy(), acc["bonus"])
        np.testing.assert_array_equal(bp.cpu().numpy(), base + acc["accept_len"] + 1)
        np.testing.assert_array_equal(tb.cpu().numpy(), want_tab)
        assert not ws[L.GRAFT_WS_COUNTER_BYTES:].any().item()


def test_verify_update_launch_counters_across_sizes():
    """Verify launches of at most 16384 rows tag each row's completion word with a
    per-row launch counter instead of clearing it.  One workspace serves launches
    of 1024, 976, 1037 and 2048 rows with a merge wavefront and of 427 rows cut
    into slices, in any order, and a zero fill between calls; every call matches
    the oracle, the workspace past the counters is zero after each, and each
    row's two counters equal the number of launches that held it since the last
    zero fill."""
    rng = np.random.default_rng(16384)
    V, k = 30011, 8
    calls = [(16, 64), (7, 61), (16, 61), (17, 61), (32, 64), (16, 64), None, (16, 61), (16, 61)]
    # every one tagged: 1024, 976, 1037 and 2048 rows with a merge wavefront, 427 rows cut into slices
    plans = [L.graft_launch_plan(B * T1, V, L.DTYPE_BF16, T1) for B, T1 in [c for c in calls if c]]
    assert [(p["merge_wave"], p["groups_per_row"] > 1, p["launch_counters"]) for p in plans] == \
        [(1, False, 1), (0, True, 1)] + [(1, False, 1)] * 6
    i32 = dict(dtype=torch.int32, device=DEV)
    table0 = rng.integers(0, V, size=(V, k)).astype(np.int32)
    tb = _t(table0, torch.int32)
    want_tab = table0.copy()
    wsb = max(L.graft_workspace_bytes(B * T1, V, k, L.DTYPE_BF16) for c in calls if c for B, T1 in [c])
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    n_tag = L.GRAFT_WS_COUNTER_BYTES // 12
    count = np.zeros(n_tag, np.int64)
    for c in calls:
        if c is None:
            ws.zero_()
            count[:] = 0
            continue
        B, T1 = c
        n = B * T1
        plan = L.graft_launch_plan(n, V, L.DTYPE_BF16, T1)
        tagged = bool(plan["launch_counters"])
        rows, tok, par, dep = _chain_batch(rng, B, T1, V)
        base = rng.integers(0, 10000, size=B).astype(np.int32)
        lg = _t(rows.view(np.int16)).view(torch.bfloat16)
        tk = torch.zeros(B, T1, k, **i32)
        al, bo = torch.zeros(B, **i32), torch.zeros(B, **i32)
        bp = _t(base, torch.int32)
        ai = torch.zeros(B, T1 - 1, **i32)
        t_, p_, d_ = (_t(x, torch.int32) for x in (tok, par, dep))
        print("verify_update B=%d T1=%d V=%d tagged=%s plan=%s" % (B, T1, V, tagged, plan), flush=True)
        L.graft_verify_update(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                              tb.data_ptr(), None, tk.data_ptr(), None, None, al.data_ptr(), ai.data_ptr(), T1 - 1,
                              bo.data_ptr(), bp.data_ptr(), ws.data_ptr(), wsb, _s())
        torch.cuda.synchronize()
        want_tk = O.topk(rows.reshape(-1, V), k, "bf16").reshape(B, T1, k)
        acc = O.accept(tok, par, want_tk[:, :, 0], T1 - 1)
        O.update(want_tab, tok.reshape(-1), want_tk.reshape(-1, k))
        np.testing.assert_array_equal(tk.cpu().numpy(), want_tk)
        np.testing.assert_array_equal(al.cpu().numpy(), acc["accept_len"])
        np.testing.assert_array_equal(ai.cpu().numpy(), acc["accept_idx"])
        np.testing.assert_array_equal(bo.cpu().numpy(), acc["bonus"])
        np.testing.assert_array_equal(bp.cpu().numpy(), base + acc["accept_len"] + 1)
        np.testing.assert_array_equal(tb.cpu().numpy(), want_tab)
        assert not ws[L.GRAFT_WS_COUNTER_BYTES:].any().item()
        if tagged:
            count[:n] += 1
        words = ws[:n_tag * 8].view(torch.int64).cpu().numpy().view(np.uint64)
        want_ctr = ws[n_tag * 8:n_tag * 12].view(torch.int32).cpu().numpy().view(np.uint32)
        np.testing.assert_array_equal(want_ctr.astype(np.int64), count)
        np.testing.assert_array_equal((words >> np.uint64(32)).astype(np.int64), count)
        if tagged:  # this launch's words: its counter and the row's greedy token + 1
            np.testing.assert_array_equal((words[:n] & np.uint64(0xffffffff)).astype(np.int64),
                                          want_tk.reshape(-1, k)[:, 0].astype(np.int64) + 1)


@pytest.mark.parametrize("n_rows,row_bytes", [(3, 16 * 13), (5, 16 * (64 * 9 + 5)), (61, 256512), (976, 303872)])
def test_stream_read_xor(n_rows, row_bytes):
    """The streaming-read probe reads every byte: each row's XOR of its 32-bit
    words equals numpy's, for ragged rows (not whole 1 KB blocks), rows of fewer
    blocks than wavefronts and the metric shape (976 rows of 151936 bf16)."""
    rng = np.random.default_rng(n_rows)
    host = rng.integers(0, 2 ** 32, size=(n_rows, row_bytes // 4), dtype=np.uint32)
    d = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros(n_rows, dtype=torch.int32, device=DEV)
    print("stream_read rows=%d bytes=%d" % (n_rows, row_bytes), flush=True)
    L.graft_stream_read(d.data_ptr(), n_rows, row_bytes, sink.data_ptr(), _s())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sink.cpu().numpy().view(np.uint32), np.bitwise_xor.reduce(host, axis=1))


# ----------------------------------------------------------------------------- coverage gain

def _coverage_case(rng, B, T1, V, layout, dtype):
    """Oracle-built hybrid trees (row sources included) and random logits."""
    par, lay, _ = TOPO
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    lp = _random_logp(rng, B)
    pr = O.prune_tree(P, Ly, lp)
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, O.template(8, 8, 52))
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    # make some retrieved tokens repeat a kept draft sibling at the root
    d_tok[:, :8] = np.where(rng.random((B, 8)) < 0.3, table[roots][:, :8], d_tok[:, :8])
    fl = O.flatten(layout, T1, roots, np.zeros(B, np.int32), d_tok, P, pr["keep"], pr["n_keep"], ret)
    z = (rng.standard_normal((B, T1, V)) * 2.5).astype(np.float32)
    rows = _bf16(z) if dtype == "bf16" else z
    return fl, rows, pr


@pytest.mark.parametrize("dtype,layout", [("bf16", "in_place"), ("bf16", "compact"), ("f32", "compact")])
def test_row_stats_and_coverage_gain(dtype, layout):
    """Row softmax statistics from the verify launch (largest value exact, the
    normaliser within 1e-5 relative of fp64) and graft_coverage_gain from them,
    within 1e-5 relative of the fp64 oracle; requests that retrieved nothing
    give exactly 0."""
    rng = np.random.default_rng(40 if dtype == "bf16" else 41)
    B, T1, V = 12, 61, 30011
    fl, rows, pr = _coverage_case(rng, B, T1, V, layout, dtype)
    lg = _t(rows.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else _t(rows)
    dt = L.DTYPE_BF16 if dtype == "bf16" else L.DTYPE_F32
    i32 = dict(dtype=torch.int32, device=DEV)
    tk = torch.zeros(B, T1, 8, **i32)
    stats = torch.zeros(B, T1, 2, dtype=torch.float32, device=DEV)
    al, bo = torch.zeros(B, **i32), torch.zeros(B, **i32)
    ai = torch.zeros(B, T1 - 1, **i32)
    t_, p_, d_ = (_t(fl[x], torch.int32) for x in ("tok", "parent", "depth"))
    src = _t(fl["row_src"], torch.uint8)
    wsb = L.graft_workspace_bytes(B * T1, V, 8, dt)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    L.graft_verify_accept(B, T1, V, 8, dt, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                          tk.data_ptr(), None, stats.data_ptr(), al.data_ptr(), ai.data_ptr(), T1 - 1,
                          bo.data_ptr(), None, ws.data_ptr(), wsb, _s())
    gain = torch.full((B,), -1.0, dtype=torch.float32, device=DEV)
    L.graft_coverage_gain(B, T1, V, dt, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), src.data_ptr(),
                          stats.data_ptr(), gain.data_ptr(), _s())
    torch.cuda.synchronize()
    want_st = O.row_stats(rows, dtype)
    got_st = stats.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got_st[..., 0], want_st[..., 0])
    np.testing.assert_allclose(got_st[..., 1], want_st[..., 1], rtol=1e-5, atol=0)
    want = O.coverage_gain(rows, fl["tok"], fl["parent"], fl["row_src"], dtype)
    got = gain.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=0)
    assert (want[pr["stage"] == 3] == 0).all()
    assert (want[pr["stage"] < 3] > 0).all()
    # the top-k is unchanged by asking for the statistics
    np.testing.assert_array_equal(tk.cpu().numpy(), O.topk(rows.reshape(-1, V), 8, dtype).reshape(B, T1, 8))


def test_coverage_gain_hand_tree_closed_form():
    """All-equal rows: every new token is worth exactly 1/V (fp32 1/V within 1e-6);
    duplicates of a draft sibling or of an earlier retrieved sibling add nothing."""
    V = 4096
    rows_spec = [(100, -1, 0), (5, 0, 1), (5, 0, 2), (7, 0, 2), (9, 3, 2), (7, 0, 2), (V + 3, 0, 2)]
    T1 = len(rows_spec)
    tok = np.array([[r[0] for r in rows_spec]], np.int32)
    par = np.array([[r[1] for r in rows_spec]], np.int32)
    src = np.array([[r[2] for r in rows_spec]], np.uint8)
    rows = np.full((1, T1, V), 0x3F80, np.uint16)       # bf16 1.0 everywhere
    lg = _t(rows.view(np.int16)).view(torch.bfloat16)
    stats = torch.zeros(1, T1, 2, dtype=torch.float32, device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    tk, al, bo = torch.zeros(1, T1, 8, **i32), torch.zeros(1, **i32), torch.zeros(1, **i32)
    ai = torch.zeros(1, T1 - 1, **i32)
    t_, p_ = _t(tok, torch.int32), _t(par, torch.int32)
    d_ = _t(np.array([[0, 1, 1, 1, 2, 1, 1]], np.int32), torch.int32)
    wsb = L.graft_workspace_bytes(T1, V, 8, L.DTYPE_BF16)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    L.graft_verify_accept(1, T1, V, 8, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), d_.data_ptr(),
                          tk.data_ptr(), None, stats.data_ptr(), al.data_ptr(), ai.data_ptr(), T1 - 1,
                          bo.data_ptr(), None, ws.data_ptr(), wsb, _s())
    gain = torch.zeros(1, dtype=torch.float32, device=DEV)
    s_ = _t(src, torch.uint8)
    L.graft_coverage_gain(1, T1, V, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(), s_.data_ptr(),
                          stats.data_ptr(), gain.data_ptr(), _s())
    torch.cuda.synchronize()
    assert abs(float(gain.item()) - 2.0 / V) <= 1e-6 * (2.0 / V)
    assert float(O.coverage_gain(rows, tok, par, src, "bf16")[0]) == pytest.approx(2.0 / V, rel=1e-14)


# ----------------------------------------------------------------------------- input checks

def _draft_flags(par, lay, score, tok, V, mode):
    """The header's conditions, per request."""
    B, Nd = score.shape
    out = np.zeros(B, np.int32)
    for b in range(B):
        f = 0
        for i in range(Nd):
            if not (0 <= tok[b, i] < V):
                f |= L.BAD_TOKEN
            s = score[b, i]
            if mode == L.MODE_TREE and not (s <= 0):
                f |= L.BAD_SCORE
            if mode == L.MODE_TAIL and not (0 <= s <= 1):
                f |= L.BAD_SCORE
            if mode == L.MODE_TREE:
                p = par[b, i]
                if not (-1 <= p < i):
                    f |= L.BAD_PARENT
                elif lay[b, i] != (0 if p < 0 else lay[b, p] + 1):
                    f |= L.BAD_LAYER
        out[b] = f
    return out


def _gpu_check_draft(par, lay, score, tok, V, mode):
    B, Nd = score.shape
    st = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    # keep every input tensor alive until the launch has run
    dp = _t(par, torch.int32) if par is not None else None
    dl = _t(lay, torch.int32) if lay is not None else None
    ds, dt = _t(score, torch.float32), _t(tok, torch.int32)
    L.graft_check_draft(B, Nd, mode, V, dp.data_ptr() if dp is not None else None,
                        dl.data_ptr() if dl is not None else None, ds.data_ptr(), dt.data_ptr(), st.data_ptr(), _s())
    torch.cuda.synchronize()
    return st.cpu().numpy()


def test_check_draft_flags():
    rng = np.random.default_rng(40)
    par, lay, _ = TOPO
    B, V = 24, 1000
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    lp = _random_logp(rng, B)
    tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    np.testing.assert_array_equal(_gpu_check_draft(P, Ly, lp, tok, V, L.MODE_TREE), 0)
    tok[1, 5] = V
    tok[2, 0] = -1
    lp[3, 7] = np.nan
    lp[4, 59] = 0.25                     # a probability above 1
    P[5, 30] = 30                         # own index
    P[6, 10] = -2
    Ly[7, 12] += 1                        # layer not parent's + 1
    P[8, 40], Ly[8, 3] = 41, 4            # two faults in one request
    lp[9, :] = 0.0                        # probability 1 everywhere is fine
    got = _gpu_check_draft(P, Ly, lp, tok, V, L.MODE_TREE)
    np.testing.assert_array_equal(got, _draft_flags(P, Ly, lp, tok, V, L.MODE_TREE))
    assert (got[1:9] != 0).all() and got[9] == 0 and got[8] == L.BAD_PARENT | L.BAD_LAYER
    # TAIL: confidences in [0, 1], tokens in range; parents and layers not read
    conf = rng.uniform(0, 1, size=(B, 16)).astype(np.float32)
    tt = rng.integers(0, V, size=(B, 16)).astype(np.int32)
    conf[0, 3], conf[1, 0], tt[2, 15] = 1.5, -0.1, V + 3
    got = _gpu_check_draft(None, None, conf, tt, V, L.MODE_TAIL)
    np.testing.assert_array_equal(got, _draft_flags(None, None, conf, tt, V, L.MODE_TAIL))
    assert list(got[:4]) == [L.BAD_SCORE, L.BAD_SCORE, L.BAD_TOKEN, 0]


def _gpu_check_tree(tok, par, dep, V):
    B, T1 = tok.shape
    st = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    dt, dp, dd = _t(tok, torch.int32), _t(par, torch.int32), _t(dep, torch.int32)
    L.graft_check_tree(B, T1, V, dt.data_ptr(), dp.data_ptr(), dd.data_ptr(), st.data_ptr(), _s())
    torch.cuda.synchronize()
    return st.cpu().numpy()


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_check_tree_accepts_built_trees_and_flags_faults(layout):
    rng = np.random.default_rng(41)
    par, lay, _ = TOPO
    B, V = 16, 3000
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    lp = _random_logp(rng, B)
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, 60)).astype(np.int32)
    pr = O.prune_tree(P, Ly, lp)
    tpl = O.template_branching(8, 2, (1, 1), 20)          # small template: empty rows too
    ret = O.retrieve_tree(table, roots, pr["n_keep"], 60, tpl)
    fl = O.flatten(layout, 61, roots, np.zeros(B, np.int32), d_tok, P, pr["keep"], pr["n_keep"], ret)
    tok, pa, de = fl["tok"].copy(), fl["parent"].copy(), fl["depth"].copy()
    assert (tok == -1).any()
    np.testing.assert_array_equal(_gpu_check_tree(tok, pa, de, V), 0)
    with_empty = [b for b in range(B) if (tok[b] == -1).any()]
    assert len(with_empty) >= 2
    e0, e1 = with_empty[0], with_empty[1]
    rest = [b for b in range(B) if b not in (e0, e1)]
    r0, r1, r2 = rest[:3]
    tok[r0, 0] = V                                   # root token out of range
    pa[r1, 0] = 0                                    # root with a parent
    f = int(np.nonzero(tok[r2] >= 0)[0][3])
    de[r2, f] += 1                                   # depth not parent's + 1
    e = int(np.nonzero(tok[e0] == -1)[0][0])
    pa[e0, e] = 0                                    # an empty slot with a parent
    ce = int(np.nonzero(tok[e1] == -1)[0][0])
    c = int(np.nonzero((tok[e1] >= 0) & (np.arange(61) > ce))[0][0]) if (tok[e1, ce + 1:] >= 0).any() else None
    if c is not None:
        pa[e1, c] = ce                               # a child of an empty slot
        de[e1, c] = 1
    got = _gpu_check_tree(tok, pa, de, V)
    assert got[r0] & L.BAD_TOKEN and got[r1] & L.BAD_PARENT and got[r2] & L.BAD_DEPTH
    assert got[e0] & L.BAD_PARENT
    if c is not None:
        assert got[e1] & L.BAD_PARENT
    clean = [b for b in range(B) if b not in (r0, r1, r2, e0, e1)]
    assert (got[clean] == 0).all()


def test_pipeline_debug_checks_raise_on_a_bad_draft():
    from hybrid_draft_tree_amd.driver import GraftPipeline
    from synth import WORKLOADS
    from synth import runner as R
    from tests.backends import HipBackend

    cfg = WORKLOADS[3].scaled(V=8000, B=4, noise_pool_rows=8)
    hb = HipBackend(cfg)
    hb.p.debug_checks = True
    wl = R.Workload(cfg)
    R.start(hb, wl)
    R.step(hb, wl, 0)                      # a valid draft passes
    d = wl.draft(1, hb.get_roots())
    d["logp"][2, 5] = np.nan
    with pytest.raises(ValueError, match=r"request\(s\) \[2\].*score"):
        hb.build(d)
    assert isinstance(hb.p, GraftPipeline)


@pytest.mark.parametrize("layout", ["compact", "in_place"])
def test_build_at_the_largest_tree(layout):
    """63 draft nodes, 63 slots, 64 verified rows: the ancestor mask's top bit
    is used and the retrieval fills up to 55 slots."""
    rng = np.random.default_rng(50)
    par, lay, _ = G.static_tree((8, 16, 16, 12, 8, 3))
    Nd, slots, T1 = 63, 63, 64
    B, V = 24, 7000
    P, Ly = np.tile(par, (B, 1)), np.tile(lay, (B, 1))
    lp = np.log(rng.dirichlet(np.ones(8), size=(B, Nd)).max(2)).astype(np.float32)
    lp[0::4, lay == 0] -= 1.5          # stage 0
    lp[1::4, lay == 1] -= 1.2          # stage 1
    lp[2::4, lay == 5] -= 3.0          # stage 2
    lp[3::4] = 0.0                     # no prune
    table = rng.integers(0, V, size=(V, 8)).astype(np.int32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    base = rng.integers(0, 100000, size=B).astype(np.int32)
    d_tok = rng.integers(0, V, size=(B, Nd)).astype(np.int32)
    R = slots - 8
    tpl, keepalive, r_out = _tpl_dev(R)
    tpl_h = _tpl_host(R)
    cfg = L.prune_cfg(CFG["ckpt"], [float(np.float32(math.log(t))) for t in CFG["tau"]], CFG["keep"], 0.5)
    i32 = dict(dtype=torch.int32, device=DEV)
    ins = [_t(x, torch.int32) for x in (table, roots, base, P, Ly)]
    sc, dt = _t(lp, torch.float32), _t(d_tok, torch.int32)
    st, nk, nr = (torch.zeros(B, **i32) for _ in range(3))
    kp = torch.zeros(B, Nd, dtype=torch.uint8, device=DEV)
    cum = torch.zeros(B, Nd, dtype=torch.float32, device=DEV)
    rt, rp = torch.zeros(B, r_out, **i32), torch.zeros(B, r_out, **i32)
    tok, par_o, dep, pos = (torch.zeros(B, T1, **i32) for _ in range(4))
    anc = torch.zeros(B, T1, dtype=torch.int64, device=DEV)
    src = torch.full((B, T1), 99, dtype=torch.uint8, device=DEV)
    L.graft_build_hybrid_tree(B, Nd, T1, L.MODE_TREE, L.LAYOUT[layout], slots, cfg, tpl, V, 8, ins[0].data_ptr(),
                              ins[1].data_ptr(), ins[2].data_ptr(), ins[3].data_ptr(), ins[4].data_ptr(),
                              sc.data_ptr(), dt.data_ptr(), st.data_ptr(), nk.data_ptr(), kp.data_ptr(),
                              cum.data_ptr(), rt.data_ptr(), rp.data_ptr(), nr.data_ptr(), r_out, tok.data_ptr(),
                              par_o.data_ptr(), dep.data_ptr(), pos.data_ptr(), anc.data_ptr(), src.data_ptr(), _s())
    torch.cuda.synchronize()
    pr = O.prune_tree(P, Ly, lp, want_cum=True)
    ret = O.retrieve_tree(table, roots, pr["n_keep"], slots, tpl_h)
    fl = O.flatten(layout, T1, roots, base, d_tok, P, pr["keep"], pr["n_keep"], ret)
    assert set(pr["stage"].tolist()) == {0, 1, 2, 3}
    np.testing.assert_array_equal(st.cpu().numpy(), pr["stage"])
    np.testing.assert_array_equal(kp.cpu().numpy(), pr["keep"])
    np.testing.assert_array_equal(nr.cpu().numpy(), ret["n_ret"])
    for name, got in (("tok", tok), ("parent", par_o), ("depth", dep), ("pos_id", pos)):
        np.testing.assert_array_equal(got.cpu().numpy(), fl[name], err_msg=(layout, name))
    a = anc.cpu().numpy().view(np.uint64)
    np.testing.assert_array_equal(a, fl["anc"])
    np.testing.assert_array_equal(src.cpu().numpy(), fl["row_src"])
    assert ((a >> np.uint64(63)) & np.uint64(1)).any()     # row 63 exists and is its own ancestor
