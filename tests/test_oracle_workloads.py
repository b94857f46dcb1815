"""The oracle driven through the five synthetic workloads at reduced sizes:
structural invariants that hold at any size (slot budget, ancestor-closed keep
sets, valid accepted paths, table rows equal to the last writer's top-k)."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import WORKLOADS
from synth import generators as G
from synth import runner as R
from synth.device import DeviceRows
from tests.backends import OracleBackend


def _small(cfg_id):
    cfg = WORKLOADS[cfg_id]
    kw = dict(V=997 if cfg.dtype == "f32" else 1000, noise_pool_rows=8)
    if cfg_id == 4:
        kw.update(prompt_len=600, ingest_chunk=256, ident_vocab=64, span_len=16)
    if cfg.B > 4:
        kw["B"] = 3
    return cfg.scaled(**kw)


def test_device_rows_equal_host_rows_on_cpu():
    cfg = _small(3)
    pool = G.NoisePool(cfg)
    rng = G.rng_for(3, 0, 0, G.STREAM_LOGITS)
    desc = G.row_descriptors(pool, rng, rng.integers(0, cfg.V, size=20))
    host = G.materialize_rows_np(pool, desc)
    dev = DeviceRows(pool, "cpu").materialize(desc)
    np.testing.assert_array_equal(dev.view(__import__("torch").int16).numpy().view(np.uint16), host)
    assert (host[np.arange(20), desc["col"]] == desc["bits"]).all()


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_workload_invariants(cfg_id):
    cfg = _small(cfg_id)
    be = OracleBackend(cfg)
    wl = R.Workload(cfg)
    T1 = cfg.rows_per_request
    seen_stages = set()

    def check(s, flat, res):
        for b in range(cfg.B):
            if cfg.mode == "tree":
                st, nk, nr = int(flat["stage"][b]), int(flat["n_keep"][b]), int(flat["n_ret"][b])
                seen_stages.add(st)
                assert nk + nr == cfg.slots
                assert (nr == 0) == (st == 3)
                par = G.static_tree()[0]
                kp = flat["keep"][b].astype(bool)
                assert all(kp[par[i]] for i in range(len(par)) if kp[i] and par[i] >= 0)
            else:
                assert int(flat["n_keep"][b]) + int(flat["n_ret"][b]) == cfg.tail_block
            n = int(res["accept_len"][b])
            path = res["accept_idx"][b][:n]
            prev = 0
            for f in path:
                assert flat["parent"][b][f] == prev
                prev = f
            assert (res["accept_idx"][b][n:] == -1).all()
        tk = res["topk"].reshape(-1, cfg.k)
        last = {}
        for P, x in enumerate(flat["tok"].reshape(-1)):
            last[int(x)] = P
        tab = be.get_table()
        for x, P in last.items():
            np.testing.assert_array_equal(tab[x], tk[P])

    R.run(be, wl, n_steps=6, warmup=2, on_step=check)
    if cfg.mode == "tree":
        assert len(seen_stages) >= 2


def test_ingest_table_rows_are_last_occurrence_topk():
    cfg = _small(4)
    be = OracleBackend(cfg)
    wl = R.Workload(cfg)
    R.start(be, wl)
    tab = be.get_table()
    prompt = wl.prompt
    last = {}
    for p, x in enumerate(prompt):
        last[int(x)] = p
    descs = list(wl.ingest_descs())
    rows_by_p = {}
    for c0, c1, desc in descs:
        rows = G.materialize_rows_np(wl.pool, desc)
        for i in range(c1 - c0):
            rows_by_p[c0 + i] = rows[i]
    for x, p in list(last.items())[:50]:
        want = O.topk(rows_by_p[p][None], cfg.k, cfg.dtype)[0]
        np.testing.assert_array_equal(tab[x], want)
    # every request starts from the greedy token of the last prompt row
    g_last = O.topk(rows_by_p[len(prompt) - 1][None], 1, cfg.dtype)[0, 0]
    assert (be.get_roots() == g_last).all()
