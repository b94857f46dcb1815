"""graft_verify_update_noalloc (no workspace argument: the library's static
per-GPU scratch) against graft_verify_update with a caller workspace, through
the C ABI, element by element: top-k, acceptance outputs, position bases and the
whole matrix, plus the oracle.  Two calls in a row on the same scratch, the
second with a smaller input (and rows split over workgroups), then a third
with probabilities."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from hybrid_draft_tree_amd import _lib as L  # noqa: E402
from oracle import oracle as O  # noqa: E402
from synth import generators as G  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(a, dtype):
    return torch.as_tensor(np.ascontiguousarray(a)).to(DEV, dtype)


def _case(rng, B, T1, V):
    """Chain-and-branch trees whose rows often carry the target's greedy token
    (N(0, 1) logits with +6 at a random column per row)."""
    z = rng.standard_normal((B, T1, V)).astype(np.float32)
    col = rng.integers(0, V, size=(B, T1))
    np.put_along_axis(z, col[:, :, None], 6.0, axis=2)
    rows = G.f32_to_bf16_bits(z).reshape(z.shape)
    par = np.zeros((B, T1), np.int32)
    tok = rng.integers(0, V, size=(B, T1)).astype(np.int32)
    tok[:, 1:] = np.where(rng.random((B, T1 - 1)) < 0.5, tok[:, 1:], rng.integers(0, 40, size=(B, T1 - 1)))
    for b in range(B):
        par[b, 0] = -1
        for f in range(1, T1):
            par[b, f] = rng.integers(max(0, f - 4), f)
            if rng.random() < 0.7:
                tok[b, f] = col[b, par[b, f]]
    dep = np.zeros((B, T1), np.int32)
    for b in range(B):
        for f in range(1, T1):
            dep[b, f] = dep[b, par[b, f]] + 1
    return rows, tok, par, dep


class _Side:
    """One side's device outputs and matrix."""

    def __init__(self, B, T1, V, k, table0, base, prob):
        i32 = dict(dtype=torch.int32, device=DEV)
        self.table = _t(table0, torch.int32)
        self.table_prob = torch.zeros(V, k, dtype=torch.float32, device=DEV) if prob else None
        self.topk = torch.full((B, T1, k), -5, **i32)
        self.topk_prob = torch.zeros(B, T1, k, dtype=torch.float32, device=DEV) if prob else None
        self.stats = torch.zeros(B, T1, 2, dtype=torch.float32, device=DEV) if prob else None
        self.al, self.bo = torch.full((B,), -5, **i32), torch.full((B,), -5, **i32)
        self.ai = torch.full((B, T1 - 1), -5, **i32)
        self.bp = _t(base, torch.int32)

    def args(self):
        p = lambda x: x.data_ptr() if x is not None else None  # noqa: E731
        return (p(self.table), p(self.table_prob), p(self.topk), p(self.topk_prob), p(self.stats), p(self.al),
                p(self.ai))

    def host(self):
        out = {"topk": self.topk, "accept_len": self.al, "accept_idx": self.ai, "bonus": self.bo,
               "base_pos": self.bp, "table": self.table}
        if self.table_prob is not None:
            out.update(table_prob=self.table_prob, topk_prob=self.topk_prob, stats=self.stats)
        return {k: v.cpu().numpy() for k, v in out.items()}


def test_noalloc_matches_workspace_call():
    rng = np.random.default_rng(2024)
    k, V = 8, 151936
    table0 = rng.integers(0, V, size=(V, k)).astype(np.int32)
    want_tab = table0.copy()
    ref = wsp = None
    s = torch.cuda.current_stream().cuda_stream
    for B, T1, prob in ((16, 61, False), (2, 17, False), (4, 61, True)):
        rows, tok, par, dep = _case(rng, B, T1, V)
        base = rng.integers(0, 5000, size=B).astype(np.int32)
        lg = _t(rows.view(np.int16), torch.int16).view(torch.bfloat16)
        t_, p_, d_ = (_t(x, torch.int32) for x in (tok, par, dep))
        # each side carries its own matrix forward from the previous call
        a_tab = ref.table.cpu().numpy() if ref is not None else table0
        b_tab = wsp.table.cpu().numpy() if wsp is not None else table0
        ref, wsp = _Side(B, T1, V, k, a_tab, base, prob), _Side(B, T1, V, k, b_tab, base, prob)
        wsb = L.graft_workspace_bytes(B * T1, V, k, L.DTYPE_BF16)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        plan = L.graft_launch_plan(B * T1, V, L.DTYPE_BF16, T1)
        print("noalloc B=%d T1=%d V=%d prob=%s groups_per_row=%d" % (B, T1, V, prob, plan["groups_per_row"]),
              flush=True)
        tb, tp, tk, tkp, st, al, ai = wsp.args()
        L.graft_verify_update(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(),
                              d_.data_ptr(), tb, tp, tk, tkp, st, al, ai, T1 - 1, wsp.bo.data_ptr(),
                              wsp.bp.data_ptr(), ws.data_ptr(), wsb, s)
        tb, tp, tk, tkp, st, al, ai = ref.args()
        L.graft_verify_update_noalloc(B, T1, V, k, L.DTYPE_BF16, lg.data_ptr(), t_.data_ptr(), p_.data_ptr(),
                                      d_.data_ptr(), tb, tp, tk, tkp, st, al, ai, T1 - 1, ref.bo.data_ptr(),
                                      ref.bp.data_ptr(), s)
        torch.cuda.synchronize()
        got, want = ref.host(), wsp.host()
        for key in want:
            if key in ("topk_prob", "stats", "table_prob"):
                np.testing.assert_array_equal(got[key].view(np.uint32), want[key].view(np.uint32), err_msg=key)
            else:
                np.testing.assert_array_equal(got[key], want[key], err_msg=key)
        # and the oracle
        want_tk, want_p = O.topk(rows.reshape(-1, V), k, "bf16", want_prob=True)
        want_tk = want_tk.reshape(B, T1, k)
        acc = O.accept(tok, par, want_tk[:, :, 0], T1 - 1)
        O.update(want_tab, tok.reshape(-1), want_tk.reshape(-1, k))
        np.testing.assert_array_equal(got["topk"], want_tk)
        np.testing.assert_array_equal(got["accept_len"], acc["accept_len"])
        np.testing.assert_array_equal(got["accept_idx"], acc["accept_idx"])
        np.testing.assert_array_equal(got["bonus"], acc["bonus"])
        np.testing.assert_array_equal(got["base_pos"], base + acc["accept_len"] + 1)
        np.testing.assert_array_equal(got["table"], want_tab)
        if prob:
            np.testing.assert_allclose(got["topk_prob"].reshape(-1, k), want_p, rtol=1e-5, atol=0)
        assert acc["accept_len"].max() > 0
        assert not ws[L.GRAFT_WS_COUNTER_BYTES:].any().item()
