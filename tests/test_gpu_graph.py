"""Whole steps captured in a HIP graph replay to the same results as the same
steps enqueued eagerly.

The verify launch keeps state in device memory from call to call: the launch
counters that tag every row's completion word, and (for launches of up to
1025 rows) nothing else, since each row decides from the later rows' tokens
whether it writes its matrix row.  A replayed graph passes the same pointers
every time, so its launches must read and advance that state exactly as eager
launches do, also when eager launches on the same workspace come between two
replays.  Two pipelines start from the same state; one replays a captured
graph of three steps, the other runs the same three steps eagerly, and every
output and the whole continuation matrix must agree bit for bit after each
replay.
"""
import pytest
import torch

import bench
from hybrid_draft_tree_amd import _lib as L
from synth import WORKLOADS

pytestmark = pytest.mark.gpu

STATE = ("table", "roots", "base_pos", "stage", "n_keep", "tok", "parent", "depth", "pos_id", "anc", "topk",
         "accept_len", "accept_idx")

# (workload, vocabulary, extra settings, expected plan): the B=16 tree step
# takes the merge-wave plan with launch counters and the holder scan; the TAIL
# step (272 rows) and the B=1 step (61 rows cut into 4 slices of 8 waves) split
# rows with launch counters and the registration hand-off; the B=4 decode step
# (244 whole rows of 8 waves, after a shortened prompt ingest) whole rows with
# the registration hand-off.
CASES = [(3, 30011, {}, (1, 1, 1)), (5, 30011, {}, (0, 1, 0)), (2, 128256, {}, (0, 1, 0)),
         (4, 151936, {"prompt_len": 4096}, (0, 1, 0))]


def _state(pipe):
    return {n: getattr(pipe, n).cpu().clone() for n in STATE}


def _assert_same(a, b, where):
    for n in STATE:
        assert torch.equal(a[n], b[n]), "%s differs %s" % (n, where)


def _steps(pipe, drafts, logits, order):
    for i in order:
        pipe.build_device(drafts[i])
        pipe.verify_update_device(logits[i])


@pytest.mark.parametrize("cfg_id,V,extra,plan", CASES, ids=["tree_b16", "tail_b16", "tree_b1", "decode_b4"])
def test_graph_replay_matches_eager(cfg_id, V, extra, plan):
    cfg = WORKLOADS[cfg_id].scaled(V=V, noise_pool_rows=16, **extra)
    dev = torch.device("cuda", 0)
    P = 3
    pipe_g, drafts_g, logits_g, acc_g = bench.setup_pool(cfg, P, dev, torch)
    pipe_e, drafts_e, logits_e, acc_e = bench.setup_pool(cfg, P, dev, torch)
    assert acc_g == acc_e
    n_rows = cfg.B * cfg.rows_per_request
    p = L.graft_launch_plan(n_rows, V, pipe_g.dtype, pipe_g.T1)
    assert (p["merge_wave"], p["launch_counters"], p["holder_scan"]) == plan
    _assert_same(_state(pipe_g), _state(pipe_e), "after set-up")
    for i in range(P):
        assert torch.equal(logits_g[i], logits_e[i])

    order = (2, 0, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _steps(pipe_g, drafts_g, logits_g, order)
    torch.cuda.synchronize()
    # capture enqueues nothing: both pipelines still stand at the same state
    _assert_same(_state(pipe_g), _state(pipe_e), "after capture")

    for rep in range(3):
        g.replay()
        _steps(pipe_e, drafts_e, logits_e, order)
        torch.cuda.synchronize()
        _assert_same(_state(pipe_g), _state(pipe_e), "after replay %d" % rep)
        assert int(pipe_g.accept_len.min()) >= 0
        # eager launches on the graph pipeline's own workspace between replays
        extra = rep % P
        _steps(pipe_g, drafts_g, logits_g, (extra,))
        _steps(pipe_e, drafts_e, logits_e, (extra,))
        torch.cuda.synchronize()
        _assert_same(_state(pipe_g), _state(pipe_e), "after the eager step following replay %d" % rep)
    # every call leaves the workspace past the counters zero-filled
    assert int(pipe_g.ws[L.GRAFT_WS_COUNTER_BYTES:].count_nonzero()) == 0
    assert int(pipe_e.ws[L.GRAFT_WS_COUNTER_BYTES:].count_nonzero()) == 0
