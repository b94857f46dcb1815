"""Thin ctypes binding of libgraft.so (include/graft.h).  Argument marshalling
only: every function forwards to the C entry point of the same name and raises
on a nonzero status.  Pointers are plain integers (device addresses, e.g.
``tensor.data_ptr()``) or None; ``stream`` is a raw hipStream_t handle.

There is no fallback: if the HIP library has not been built this module fails
loudly at load time.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgraft.so")

GRAFT_OK = 0
GRAFT_EINVAL = -1
GRAFT_EUNSUPPORTED = -2
GRAFT_EDEVICE = -3
GRAFT_ESCRATCH = -4
GRAFT_NOALLOC_SCRATCH_BYTES = 8 << 20  # static scratch of graft_verify_update_noalloc per GPU
GRAFT_WS_COUNTER_BYTES = 196608  # leading workspace bytes kept between calls (per-row launch counters)
GRAFT_MAX_ROWS = 64
GRAFT_MAX_K = 8
GRAFT_MAX_VOCAB = 1000000   # logits per row accepted by the top-k calls
GRAFT_MAX_BATCH = 1 << 24   # requests per call
GRAFT_MAX_COORD_GROUPS = 128  # coordinator workgroups of a verify launch at most
DTYPE_F32 = 0
DTYPE_BF16 = 1
MODE_TREE = 0
MODE_TAIL = 1
LAYOUT = {"compact": 0, "in_place": 1, "chain": 2}
ROW_ROOT, ROW_DRAFT, ROW_RETRIEVED, ROW_EMPTY = 0, 1, 2, 3
MAX_ROWS = 64
MAX_K = 8

EXPORTS = (
    "graft_prune_select", "graft_check_draft", "graft_check_tree", "graft_checkpoint_stats", "graft_calibrate_thresholds", "graft_template_master", "graft_template_branching", "graft_retrieve_expand",
    "graft_build_tree_mask", "graft_verify_accept", "graft_update_topk",
    "graft_build_hybrid_tree", "graft_build_after_retrieval", "graft_verify_update",
    "graft_verify_update_noalloc", "graft_coverage_gain", "graft_stream_read",
    "graft_launch_plan", "graft_workspace_bytes", "graft_status_string",
)


class GraftError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _LIB.graft_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__("%s failed: %d (%s)" % (fn, status, msg))


class PruneCfg(C.Structure):
    _fields_ = [("ckpt_layer", C.c_int32 * 3), ("log_thr", C.c_float * 3),
                ("keep", C.c_int32 * 3), ("tail_thr", C.c_float), ("node_mode", C.c_int32),
                ("node_log_thr", C.c_float)]


class Template(C.Structure):
    _fields_ = [("size", C.c_int32), ("parent", C.c_void_p), ("rank", C.c_void_p),
                ("depth", C.c_void_p)]


class Plan(C.Structure):
    _fields_ = [("waves_per_group", C.c_int32), ("groups_per_row", C.c_int32),
                ("blocks_per_batch", C.c_int32), ("coord_groups", C.c_int32), ("workgroups", C.c_int64),
                ("merge_wave", C.c_int32), ("launch_counters", C.c_int32), ("holder_scan", C.c_int32)]


_LIB = None


def load():
    """Load libgraft.so (raises if it was not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError("libgraft.so not found at %s: build it with "
                          "`python -m hybrid_draft_tree_amd.build` (there is no CPU fallback)" % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    P, I, I64, S = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    L.graft_prune_select.argtypes = [I, I, I, P, P, P, C.POINTER(PruneCfg), P, P, P, P, P]
    L.graft_check_draft.argtypes = [I, I, I, I, P, P, P, P, P, P]
    L.graft_check_tree.argtypes = [I, I, I, P, P, P, P, P]
    L.graft_checkpoint_stats.argtypes = [I, I, P, P, P, C.POINTER(PruneCfg), P, P]
    L.graft_calibrate_thresholds.argtypes = [I64, P, C.POINTER(C.c_float * 3), P, P]
    L.graft_template_master.argtypes = [I, I, I, P, P, P]
    L.graft_template_branching.argtypes = [I, I, I, I, I, P, P, P]
    L.graft_retrieve_expand.argtypes = [I, I, I, I, I, P, P, P, P, I, C.POINTER(Template),
                                        C.POINTER(PruneCfg), P, P, P, I, P]
    L.graft_build_tree_mask.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, P]
    L.graft_verify_accept.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, I, P, P, P, S, P]
    L.graft_update_topk.argtypes = [I64, I, I, I, P, P, P, P, P, P, P, P, S, P]
    L.graft_build_hybrid_tree.argtypes = [I, I, I, I, I, I, C.POINTER(PruneCfg), C.POINTER(Template), I, I,
                                          P, P, P, P, P, P, P, P, P, P, P, P, P, P, I, P, P, P, P, P, P, P]
    L.graft_build_after_retrieval.argtypes = [I, I, I, I, I, C.POINTER(PruneCfg), P, P, P, P, P, P, P, P, P, P,
                                              P, P, P, I, P, P, P, P, P, P, P]
    L.graft_verify_update.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, I, P, P, P, S, P]
    L.graft_verify_update_noalloc.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, I, P, P, P]
    L.graft_coverage_gain.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
    L.graft_stream_read.argtypes = [P, I64, I64, P, P]
    L.graft_launch_plan.argtypes = [I64, I, I, I, C.POINTER(Plan)]
    L.graft_workspace_bytes.argtypes = [I64, I, I, I]
    L.graft_workspace_bytes.restype = S
    L.graft_status_string.argtypes = [I]
    L.graft_status_string.restype = C.c_char_p
    for name in EXPORTS:
        if name not in ("graft_workspace_bytes", "graft_status_string"):
            getattr(L, name).restype = C.c_int
    _LIB = L
    return L


def _chk(fn, rc):
    if rc < 0:
        raise GraftError(fn, rc)
    return rc


def prune_cfg(ckpt_layers, log_thr, keep, tail_thr, node_log_thr=None) -> PruneCfg:
    """node_log_thr (fp32 log-confidence) switches TREE pruning to the per-node variant."""
    c = PruneCfg()
    for i in range(3):
        c.ckpt_layer[i] = int(ckpt_layers[i])
        c.log_thr[i] = float(log_thr[i])
        c.keep[i] = int(keep[i])
    c.tail_thr = float(tail_thr)
    c.node_mode = 0 if node_log_thr is None else 1
    c.node_log_thr = 0.0 if node_log_thr is None else float(node_log_thr)
    return c


def graft_prune_select(B, Nd, mode, d_parent, d_layer, d_score, cfg, stage, n_keep, keep, cum_out, stream):
    return _chk("graft_prune_select", load().graft_prune_select(
        B, Nd, mode, d_parent, d_layer, d_score, C.byref(cfg), stage, n_keep, keep, cum_out, stream))


BAD_PARENT, BAD_LAYER, BAD_SCORE, BAD_TOKEN, BAD_DEPTH = 1, 2, 4, 8, 16


def graft_check_draft(B, Nd, mode, V, d_parent, d_layer, d_score, d_tok, status, stream):
    return _chk("graft_check_draft", load().graft_check_draft(
        B, Nd, mode, V, d_parent, d_layer, d_score, d_tok, status, stream))


def graft_check_tree(B, T1, V, tok, parent, depth, status, stream):
    return _chk("graft_check_tree", load().graft_check_tree(B, T1, V, tok, parent, depth, status, stream))


def graft_checkpoint_stats(B, Nd, d_parent, d_layer, d_score, cfg, out, stream):
    return _chk("graft_checkpoint_stats", load().graft_checkpoint_stats(
        B, Nd, d_parent, d_layer, d_score, C.byref(cfg), out, stream))


def graft_calibrate_thresholds(n, samples, q, log_thr, stream):
    qa = (C.c_float * 3)(*[float(x) for x in q])
    return _chk("graft_calibrate_thresholds", load().graft_calibrate_thresholds(
        n, samples, C.byref(qa), log_thr, stream))


def graft_template_master(width, depth, cap):
    """Returns (parent, rank, depth) host lists of the master template order."""
    par = (C.c_int32 * max(cap, 1))()
    rk = (C.c_int32 * max(cap, 1))()
    dp = (C.c_int32 * max(cap, 1))()
    n = _chk("graft_template_master", load().graft_template_master(width, depth, cap, par, rk, dp))
    return list(par[:n]), list(rk[:n]), list(dp[:n])


def graft_template_branching(width, depth, beta_num, beta_den, cap):
    """Returns (parent, rank, depth) host lists of the branching template's master order."""
    par = (C.c_int32 * max(cap, 1))()
    rk = (C.c_int32 * max(cap, 1))()
    dp = (C.c_int32 * max(cap, 1))()
    n = _chk("graft_template_branching",
             load().graft_template_branching(width, depth, beta_num, beta_den, cap, par, rk, dp))
    return list(par[:n]), list(rk[:n]), list(dp[:n])


def graft_retrieve_expand(B, V, k, mode, slots, table, root_tok, n_keep, d_tok, Nd, tpl, cfg,
                          ret_tok, ret_parent, n_ret, r_out, stream):
    return _chk("graft_retrieve_expand", load().graft_retrieve_expand(
        B, V, k, mode, slots, table, root_tok, n_keep, d_tok, Nd,
        C.byref(tpl) if tpl is not None else None, C.byref(cfg) if cfg is not None else None,
        ret_tok, ret_parent, n_ret, r_out, stream))


def graft_build_tree_mask(B, Nd, T1, layout, root_tok, base_pos, d_tok, d_parent, keep, n_keep,
                          ret_tok, ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc, row_src,
                          stream):
    return _chk("graft_build_tree_mask", load().graft_build_tree_mask(
        B, Nd, T1, layout, root_tok, base_pos, d_tok, d_parent, keep, n_keep, ret_tok, ret_parent,
        n_ret, r_out, tok, parent, depth, pos_id, anc, row_src, stream))


def graft_verify_accept(B, T1, V, k, dtype, logits, tok, parent, depth, topk, topk_prob, row_stats,
                        accept_len, accept_idx, dmax, bonus, base_pos_io, ws, ws_bytes, stream):
    return _chk("graft_verify_accept", load().graft_verify_accept(
        B, T1, V, k, dtype, logits, tok, parent, depth, topk, topk_prob, row_stats, accept_len,
        accept_idx, dmax, bonus, base_pos_io, ws, ws_bytes, stream))


def graft_update_topk(n_rows, V, k, dtype, logits, topk_in, prob_in, row_tok, table, table_prob,
                      topk_out, ws, ws_bytes, stream):
    return _chk("graft_update_topk", load().graft_update_topk(
        n_rows, V, k, dtype, logits, topk_in, prob_in, row_tok, table, table_prob, topk_out,
        ws, ws_bytes, stream))


def graft_build_hybrid_tree(B, Nd, T1, mode, layout, slots, cfg, tpl, V, k, table, root_tok, base_pos,
                            d_parent, d_layer, d_score, d_tok, stage, n_keep, keep, cum_out, ret_tok,
                            ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc, row_src, stream):
    return _chk("graft_build_hybrid_tree", load().graft_build_hybrid_tree(
        B, Nd, T1, mode, layout, slots, C.byref(cfg), C.byref(tpl) if tpl is not None else None, V, k,
        table, root_tok, base_pos, d_parent, d_layer, d_score, d_tok, stage, n_keep, keep, cum_out,
        ret_tok, ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc, row_src, stream))


def graft_build_after_retrieval(B, Nd, T1, layout, slots, cfg, root_tok, base_pos, d_parent, d_layer, d_score,
                                d_tok, stage, n_keep, keep, cum_out, ret_tok, ret_parent, n_ret, r_out, tok, parent,
                                depth, pos_id, anc, row_src, stream):
    return _chk("graft_build_after_retrieval", load().graft_build_after_retrieval(
        B, Nd, T1, layout, slots, C.byref(cfg), root_tok, base_pos, d_parent, d_layer, d_score, d_tok, stage,
        n_keep, keep, cum_out, ret_tok, ret_parent, n_ret, r_out, tok, parent, depth, pos_id, anc, row_src,
        stream))


def graft_verify_update(B, T1, V, k, dtype, logits, tok, parent, depth, table, table_prob, topk, topk_prob,
                        row_stats, accept_len, accept_idx, dmax, bonus, base_pos_io, ws, ws_bytes, stream):
    return _chk("graft_verify_update", load().graft_verify_update(
        B, T1, V, k, dtype, logits, tok, parent, depth, table, table_prob, topk, topk_prob, row_stats,
        accept_len, accept_idx, dmax, bonus, base_pos_io, ws, ws_bytes, stream))


def graft_verify_update_noalloc(B, T1, V, k, dtype, logits, tok, parent, depth, table, table_prob, topk,
                                topk_prob, row_stats, accept_len, accept_idx, dmax, bonus, base_pos_io, stream):
    return _chk("graft_verify_update_noalloc", load().graft_verify_update_noalloc(
        B, T1, V, k, dtype, logits, tok, parent, depth, table, table_prob, topk, topk_prob, row_stats,
        accept_len, accept_idx, dmax, bonus, base_pos_io, stream))


def graft_coverage_gain(B, T1, V, dtype, logits, tok, parent, row_src, row_stats, gain, stream):
    return _chk("graft_coverage_gain", load().graft_coverage_gain(
        B, T1, V, dtype, logits, tok, parent, row_src, row_stats, gain, stream))


def graft_stream_read(data, n_rows, row_bytes, sink, stream):
    """Read ceiling of the verify launch's geometry (measurement aid): one XOR word per row into sink."""
    return _chk("graft_stream_read", load().graft_stream_read(data, n_rows, row_bytes, sink, stream))


def graft_launch_plan(n_rows, V, dtype, T1):
    """The top-k launch's plan as a dict (host only; nothing is enqueued)."""
    p = Plan()
    _chk("graft_launch_plan", load().graft_launch_plan(n_rows, V, dtype, T1, C.byref(p)))
    return {f: int(getattr(p, f)) for f, _ in Plan._fields_}


def graft_workspace_bytes(n_rows, V, k, dtype):
    return int(load().graft_workspace_bytes(n_rows, V, k, dtype))


def graft_status_string(status):
    return load().graft_status_string(status).decode()
