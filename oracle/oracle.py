"""ctypes front-end of the CPU oracle (oracle/graft_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Arrays are numpy;
every function allocates its outputs and raises on a nonzero status.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

DT_F32 = 0
DT_BF16 = 1
LAYOUTS = {"compact": 0, "in_place": 1, "chain": 2}
ROW_ROOT, ROW_DRAFT, ROW_RETRIEVED, ROW_EMPTY = 0, 1, 2, 3


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        L = C.CDLL(path)
        P = C.c_void_p
        L.oracle_prune_tree.argtypes = [C.c_int, C.c_int, P, P, P, P, P, P, C.c_double, P, P, P, P]
        L.oracle_prune_tail.argtypes = [C.c_int, C.c_int, P, C.c_float, P, P, P]
        L.oracle_checkpoint_stats.argtypes = [C.c_int, C.c_int, P, P, P, P, P, P]
        L.oracle_calibrate.argtypes = [C.c_int64, P, P, P]
        L.oracle_template.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P]
        L.oracle_template_branching.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P]
        L.oracle_retrieve_tree.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, C.c_int, C.c_int, P, P,
                                           C.c_int, P, P, P]
        L.oracle_retrieve_tail.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, C.c_int, P, P, P]
        L.oracle_flatten.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P, P, P, C.c_int,
                                     P, P, P, P, P, P, P, P, P]
        L.oracle_row_stats.argtypes = [C.c_int64, C.c_int, C.c_int, P, P]
        L.oracle_coverage_gain.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P, P]
        L.oracle_topk.argtypes = [C.c_int64, C.c_int, C.c_int, C.c_int, P, P, P]
        L.oracle_accept.argtypes = [C.c_int, C.c_int, P, P, P, C.c_int, P, P, P]
        L.oracle_update.argtypes = [C.c_int64, C.c_int, C.c_int, P, P, P, P, P]
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_num_threads.restype = C.c_int
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with status %d" % (what, rc))


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def prune_tree(parent, layer, logp, ckpt_layers=(0, 1, 5), tau=(0.3, 0.2, 0.1), keep=(8, 24, 40),
               want_cum=False, node_tau=0.0, log_thr=None):
    """Checkpoint pruning; with node_tau > 0 the per-node variant instead (stage 4 when it cuts).
    log_thr (fp32 [3]), when given, replaces (float) ln tau, e.g. calibrated thresholds."""
    parent, layer = _i32(parent), _i32(layer)
    logp = np.ascontiguousarray(logp, dtype=np.float32)
    B, Nd = parent.shape
    stage = np.zeros(B, np.int32)
    n_keep = np.zeros(B, np.int32)
    keepm = np.zeros((B, Nd), np.uint8)
    cum = np.zeros((B, Nd), np.float32) if want_cum else None
    ck = _i32(ckpt_layers)
    lt = log_thresholds(tau) if log_thr is None else np.ascontiguousarray(log_thr, dtype=np.float32)
    kn = _i32(keep)
    rc = lib().oracle_prune_tree(B, Nd, _p(parent), _p(layer), _p(logp), _p(ck), _p(lt), _p(kn),
                                 float(node_tau), _p(stage), _p(n_keep), _p(keepm), _p(cum))
    _check(rc, "prune_tree")
    out = {"stage": stage, "n_keep": n_keep, "keep": keepm}
    if want_cum:
        out["cum"] = cum
    return out


def checkpoint_stats(parent, layer, logp, ckpt_layers=(0, 1, 5), keep=(8, 24, 40)):
    """Per request, the statistic each checkpoint compares (fp32 [B, 3], NaN where not reached)."""
    parent, layer = _i32(parent), _i32(layer)
    logp = np.ascontiguousarray(logp, dtype=np.float32)
    B, Nd = parent.shape
    out = np.zeros((B, 3), np.float32)
    _check(lib().oracle_checkpoint_stats(B, Nd, _p(parent), _p(layer), _p(logp), _p(_i32(ckpt_layers)),
                                         _p(_i32(keep)), _p(out)), "checkpoint_stats")
    return out


def calibrate(samples, q):
    """fp32 log-thresholds [3] from warm-up statistics [n, 3] at quantile levels q [3]."""
    samples = np.ascontiguousarray(samples, dtype=np.float32).reshape(-1, 3)
    qa = np.ascontiguousarray(q, dtype=np.float32)
    out = np.zeros(3, np.float32)
    _check(lib().oracle_calibrate(samples.shape[0], _p(samples), _p(qa), _p(out)), "calibrate")
    return out


def log_thresholds(tau):
    """(float) ln tau per checkpoint: tau 0 -> -inf (never fires), +inf -> +inf (always)."""
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(tau, np.float64)).astype(np.float32)


def prune_tail(conf, thr=0.5):
    conf = np.ascontiguousarray(conf, dtype=np.float32)
    B, L = conf.shape
    stage = np.zeros(B, np.int32)
    n_keep = np.zeros(B, np.int32)
    keepm = np.zeros((B, L), np.uint8)
    _check(lib().oracle_prune_tail(B, L, _p(conf), float(thr), _p(stage), _p(n_keep), _p(keepm)),
           "prune_tail")
    return {"stage": stage, "n_keep": n_keep, "keep": keepm}


def template(W=8, D=8, Rmax=52):
    par = np.zeros(max(Rmax, 1), np.int32)
    rank = np.zeros(max(Rmax, 1), np.int32)
    dep = np.zeros(max(Rmax, 1), np.int32)
    n = lib().oracle_template(W, D, Rmax, _p(par), _p(rank), _p(dep))
    if n < 0:
        raise RuntimeError("oracle template failed")
    return {"parent": par[:n], "rank": rank[:n], "depth": dep[:n]}


def template_branching(W=8, D=8, beta=(1, 1), Rmax=52):
    """Branching template: rank paths ordered by d*den + num*sum(ranks), beta = num/den."""
    num, den = beta
    par = np.zeros(max(Rmax, 1), np.int32)
    rank = np.zeros(max(Rmax, 1), np.int32)
    dep = np.zeros(max(Rmax, 1), np.int32)
    n = lib().oracle_template_branching(W, D, num, den, Rmax, _p(par), _p(rank), _p(dep))
    if n < 0:
        raise RuntimeError("oracle branching template failed")
    return {"parent": par[:n], "rank": rank[:n], "depth": dep[:n]}


def retrieve_tree(table, root_tok, n_keep, slots, tpl, Rmax_out=None):
    table = _i32(table)
    V, k = table.shape
    root_tok, n_keep = _i32(root_tok), _i32(n_keep)
    B = len(root_tok)
    Rt = len(tpl["parent"])
    Rmax_out = Rt if Rmax_out is None else Rmax_out
    ret_tok = np.zeros((B, max(Rmax_out, 1)), np.int32)
    ret_par = np.zeros((B, max(Rmax_out, 1)), np.int32)
    n_ret = np.zeros(B, np.int32)
    tp, tr = _i32(tpl["parent"]), _i32(tpl["rank"])
    rc = lib().oracle_retrieve_tree(B, V, k, _p(table), _p(root_tok), _p(n_keep), slots, Rt, _p(tp),
                                    _p(tr), max(Rmax_out, 1), _p(ret_tok), _p(ret_par), _p(n_ret))
    _check(rc, "retrieve_tree")
    return {"ret_tok": ret_tok, "ret_parent": ret_par, "n_ret": n_ret}


def retrieve_tail(table, root_tok, d_tok, n_keep):
    table = _i32(table)
    V, k = table.shape
    d_tok = _i32(d_tok)
    B, L = d_tok.shape
    ret_tok = np.zeros((B, L), np.int32)
    ret_par = np.zeros((B, L), np.int32)
    n_ret = np.zeros(B, np.int32)
    rc = lib().oracle_retrieve_tail(B, V, k, _p(table), _p(_i32(root_tok)), _p(d_tok), _p(_i32(n_keep)),
                                    L, _p(ret_tok), _p(ret_par), _p(n_ret))
    _check(rc, "retrieve_tail")
    return {"ret_tok": ret_tok, "ret_parent": ret_par, "n_ret": n_ret}


def flatten(layout, T1, root_tok, base_pos, d_tok, d_parent, keep, n_keep, ret):
    d_tok = _i32(d_tok)
    B, Nd = d_tok.shape
    d_parent = _i32(d_parent)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    rt, rp = _i32(ret["ret_tok"]), _i32(ret["ret_parent"])
    Rmax = rt.shape[1]
    tok = np.zeros((B, T1), np.int32)
    par = np.zeros((B, T1), np.int32)
    dep = np.zeros((B, T1), np.int32)
    pos = np.zeros((B, T1), np.int32)
    anc = np.zeros((B, T1), np.uint64)
    src = np.zeros((B, T1), np.uint8)
    rc = lib().oracle_flatten(B, Nd, T1, LAYOUTS[layout], _p(_i32(root_tok)), _p(_i32(base_pos)),
                              _p(d_tok), _p(d_parent), _p(keep), _p(_i32(n_keep)), Rmax, _p(rt), _p(rp),
                              _p(_i32(ret["n_ret"])), _p(tok), _p(par), _p(dep), _p(pos), _p(anc), _p(src))
    _check(rc, "flatten")
    return {"tok": tok, "parent": par, "depth": dep, "pos_id": pos, "anc": anc, "row_src": src}


def _logits(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return a.view(np.uint16), DT_BF16
    return a.view(np.float32), DT_F32


def row_stats(logits, dtype="bf16"):
    """fp64 softmax statistics per row: [..., 2] = (max value, sum of exp(value - max))."""
    a, dt = _logits(logits, dtype)
    V = a.shape[-1]
    n = a.size // V
    out = np.zeros((n, 2), np.float64)
    _check(lib().oracle_row_stats(n, V, dt, _p(a), _p(out)), "row_stats")
    return out.reshape(a.shape[:-1] + (2,))


def coverage_gain(logits, tok, parent, row_src, dtype="bf16"):
    """fp64 coverage gain per request; logits [B, T1, V], tree arrays [B, T1]."""
    a, dt = _logits(logits, dtype)
    tok, parent = _i32(tok), _i32(parent)
    B, T1 = tok.shape
    V = a.shape[-1]
    assert a.size == B * T1 * V
    src = np.ascontiguousarray(row_src, np.uint8)
    out = np.zeros(B, np.float64)
    _check(lib().oracle_coverage_gain(B, T1, V, dt, _p(a), _p(tok), _p(parent), _p(src), _p(out)),
           "coverage_gain")
    return out


def topk(logits, k=8, dtype="bf16", want_prob=False):
    """logits: [..., V] uint16 (bf16 bit patterns) or float32."""
    a = np.ascontiguousarray(logits)
    V = a.shape[-1]
    n = a.size // V
    if dtype == "bf16":
        a = a.view(np.uint16)
        dt = DT_BF16
    else:
        a = a.view(np.float32)
        dt = DT_F32
    out = np.zeros((n, k), np.int32)
    prob = np.zeros((n, k), np.float64) if want_prob else None
    _check(lib().oracle_topk(n, V, k, dt, _p(a), _p(out), _p(prob)), "topk")
    shp = a.shape[:-1] + (k,)
    return (out.reshape(shp), prob.reshape(shp)) if want_prob else out.reshape(shp)


def accept(tok, parent, g, Dmax):
    tok, parent, g = _i32(tok), _i32(parent), _i32(g)
    B, T1 = tok.shape
    alen = np.zeros(B, np.int32)
    aidx = np.zeros((B, Dmax), np.int32)
    bonus = np.zeros(B, np.int32)
    _check(lib().oracle_accept(B, T1, _p(tok), _p(parent), _p(g), Dmax, _p(alen), _p(aidx), _p(bonus)),
           "accept")
    return {"accept_len": alen, "accept_idx": aidx, "bonus": bonus}


def update(table, row_tok, topk_rows, prob=None, table_prob=None):
    """In place on ``table`` (int32 [V, k]); rows applied in increasing order."""
    assert table.dtype == np.int32 and table.flags.c_contiguous
    V, k = table.shape
    row_tok = _i32(row_tok).reshape(-1)
    tk = _i32(topk_rows).reshape(-1, k)
    pr = None if prob is None else np.ascontiguousarray(prob, np.float64).reshape(-1, k)
    if table_prob is not None:
        assert table_prob.dtype == np.float32 and table_prob.flags.c_contiguous
    _check(lib().oracle_update(len(row_tok), V, k, _p(row_tok), _p(tk), _p(table), _p(pr), _p(table_prob)),
           "update")
    return table
