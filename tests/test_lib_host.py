"""Host-side checks of libgraft.so that need no GPU: the library loads, exports
every entry point include/graft.h declares, validates arguments before
launching anything, and its host-built retrieval template equals the oracle's
independently written one."""
import ctypes
import os
import re

import numpy as np
import pytest

from hybrid_draft_tree_amd import _lib as L
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "graft.h")).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char \*)\s*\**\s*(graft_\w+)\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = _declared()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_product_package_has_no_oracle_dependency():
    pkg = os.path.join(ROOT, "hybrid_draft_tree_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_status_strings():
    assert L.graft_status_string(0) == "ok"
    assert "invalid" in L.graft_status_string(-1)
    assert "unsupported" in L.graft_status_string(-2)


def test_workspace_bytes():
    assert L.graft_workspace_bytes(976, 151936, 8, L.DTYPE_BF16) > 976 * 8 * 8
    assert L.graft_workspace_bytes(10, 100, 9, L.DTYPE_BF16) == 0      # k > 8
    assert L.graft_workspace_bytes(10, 4, 8, L.DTYPE_BF16) == 0        # k > V
    assert L.graft_workspace_bytes(10, 100, 8, 7) == 0                 # bad dtype
    assert L.graft_workspace_bytes(0, 100, 8, L.DTYPE_F32) >= 0


def test_launch_size_limits():
    """Row counts that do not fit one top-k launch (32-bit thread count, 32-bit
    row positions) get no workspace size and are rejected before any launch."""
    bf = L.DTYPE_BF16
    # small vocabulary: one wavefront per row, (rows + 128 coordinators) x 64 < 2^32
    assert L.graft_workspace_bytes(67_108_735, 100, 8, bf) > 0
    assert L.graft_workspace_bytes(67_108_736, 100, 8, bf) == 0
    assert L.graft_workspace_bytes((1 << 31) - 1, 100, 8, bf) == 0
    # V = 10^6 bf16 needs 16 wavefronts per row (127 blocks of 512 elements per wavefront at most)
    assert L.graft_workspace_bytes(4_194_175, 10 ** 6, 8, bf) > 0
    assert L.graft_workspace_bytes(4_194_176, 10 ** 6, 8, bf) == 0
    lib = L.load()
    P = 0x1000  # never dereferenced
    huge = 1 << 62
    assert lib.graft_update_topk(67_108_736, 100, 8, bf, P, None, None, P, P, None, None, P, huge, None) == \
        L.GRAFT_EINVAL
    assert lib.graft_update_topk(1 << 40, 100, 8, bf, P, None, None, P, P, None, None, P, huge, None) == \
        L.GRAFT_EINVAL
    assert lib.graft_verify_accept(1_100_200, 61, 100, 8, bf, *([P] * 9), 60, P, None, P, huge, None) == \
        L.GRAFT_EINVAL
    assert lib.graft_verify_update(1_100_200, 61, 100, 8, bf, *([P] * 11), 60, P, None, P, huge, None) == \
        L.GRAFT_EINVAL
    # the call without a workspace: sizes beyond its static scratch are refused before anything runs
    assert lib.graft_verify_update_noalloc(20000, 61, 10 ** 6, 8, bf, *([P] * 11), 60, P, None, None) == \
        L.GRAFT_ESCRATCH
    assert lib.graft_verify_update_noalloc(20000, 61, 100, 8, bf, *([P] * 11), 60, P, None, None) == \
        L.GRAFT_ESCRATCH
    assert lib.graft_verify_update_noalloc(1_100_200, 61, 100, 8, bf, *([P] * 11), 60, P, None, None) == \
        L.GRAFT_EINVAL
    assert "static scratch" in L.graft_status_string(L.GRAFT_ESCRATCH)
    # per-request calls: at most 2^24 requests
    cfg = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 40), 0.5)
    assert lib.graft_prune_select(L.GRAFT_MAX_BATCH + 1, 60, 0, P, P, P, ctypes.byref(cfg), P, P, P, None, None) == \
        L.GRAFT_EINVAL
    assert lib.graft_build_tree_mask(L.GRAFT_MAX_BATCH + 1, 60, 61, 0, *([P] * 9), 52, *([P] * 5), None, None) == \
        L.GRAFT_EINVAL
    assert lib.graft_coverage_gain(L.GRAFT_MAX_BATCH + 1, 61, 100, 1, *([P] * 6), None) == L.GRAFT_EINVAL
    assert lib.graft_check_tree(L.GRAFT_MAX_BATCH + 1, 61, 100, P, P, P, P, None) == L.GRAFT_EINVAL


@pytest.mark.parametrize("W,D,R", [(8, 8, 52), (8, 8, 64), (8, 8, 20), (4, 6, 24), (1, 3, 3), (5, 1, 5)])
def test_template_matches_oracle(W, D, R):
    par, rk, dp = L.graft_template_master(W, D, R)
    o = O.template(W, D, R)
    assert par == o["parent"].tolist()
    assert rk == o["rank"].tolist()
    assert dp == o["depth"].tolist()


def test_calibration_validation_rejects_without_launch():
    cfg = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 40), 0.5)
    lib = L.load()
    P = 0x1000  # never dereferenced
    q = (ctypes.c_float * 3)
    ok = q(0.2, 0.2, 0.2)
    assert lib.graft_checkpoint_stats(1, 65, P, P, P, ctypes.byref(cfg), P, None) == L.GRAFT_EINVAL
    assert lib.graft_checkpoint_stats(1, 0, P, P, P, ctypes.byref(cfg), P, None) == L.GRAFT_EINVAL
    assert lib.graft_checkpoint_stats(1, 60, P, P, P, None, P, None) == L.GRAFT_EINVAL
    assert lib.graft_checkpoint_stats(1, 60, P, None, P, ctypes.byref(cfg), P, None) == L.GRAFT_EINVAL
    assert lib.graft_checkpoint_stats(0, 60, None, None, None, ctypes.byref(cfg), None, None) == L.GRAFT_OK
    for bad in [q(1.5, 0.2, 0.2), q(0.2, -0.1, 0.2), q(0.2, 0.2, float("nan"))]:
        assert lib.graft_calibrate_thresholds(10, P, ctypes.byref(bad), P, None) == L.GRAFT_EINVAL
    assert lib.graft_calibrate_thresholds(-1, P, ctypes.byref(ok), P, None) == L.GRAFT_EINVAL
    assert lib.graft_calibrate_thresholds((1 << 26) + 1, P, ctypes.byref(ok), P, None) == L.GRAFT_EINVAL
    assert lib.graft_calibrate_thresholds(10, None, ctypes.byref(ok), P, None) == L.GRAFT_EINVAL
    assert lib.graft_calibrate_thresholds(10, P, ctypes.byref(ok), None, None) == L.GRAFT_EINVAL


def test_retrieval_ahead_validation_rejects_without_launch():
    cfg = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 40), 0.5)
    lib = L.load()
    P = 0x1000  # never dereferenced
    cb = ctypes.byref(cfg)
    # TAIL retrieval needs the kept prefix: no n_keep is invalid there
    assert lib.graft_retrieve_expand(1, 100, 8, 1, 16, P, P, None, P, 16, None, None, P, P, P, 16, None) == L.GRAFT_EINVAL
    # the chain layout (TAIL) cannot take a retrieval done ahead
    args = [P] * 14
    assert lib.graft_build_after_retrieval(1, 60, 61, 2, 60, cb, *args[:13], 52, *args[:6], None) == \
        L.GRAFT_EUNSUPPORTED
    assert lib.graft_build_after_retrieval(1, 60, 62, 0, 60, cb, *args[:13], 52, *args[:6], None) == L.GRAFT_EINVAL
    assert lib.graft_build_after_retrieval(1, 60, 61, 0, 60, None, *args[:13], 52, *args[:6], None) == L.GRAFT_EINVAL
    assert lib.graft_build_after_retrieval(1, 60, 61, 0, 60, cb, None, *args[:12], 52, *args[:6], None) == \
        L.GRAFT_EINVAL
    assert lib.graft_build_after_retrieval(1, 60, 61, 0, 60, cb, *args[:13], 65, *args[:6], None) == L.GRAFT_EINVAL


def test_host_validation_rejects_without_launch():
    cfg = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 40), 0.5)
    lib = L.load()
    P = 0x1000  # never dereferenced: every call below fails validation first
    # unsupported mode / layout / dtype
    assert lib.graft_prune_select(1, 60, 7, P, P, P, ctypes.byref(cfg), P, P, P, None, None) == L.GRAFT_EUNSUPPORTED
    assert lib.graft_build_tree_mask(1, 60, 61, 9, *([P] * 9), 52, *([P] * 5), None, None) == L.GRAFT_EUNSUPPORTED
    assert lib.graft_verify_accept(1, 61, 100, 8, 5, *([P] * 9), 60, P, None, P, 1 << 20, None) == L.GRAFT_EUNSUPPORTED
    # bad sizes
    assert lib.graft_prune_select(1, 65, 0, P, P, P, ctypes.byref(cfg), P, P, P, None, None) == L.GRAFT_EINVAL
    assert lib.graft_prune_select(1, 0, 0, P, P, P, ctypes.byref(cfg), P, P, P, None, None) == L.GRAFT_EINVAL
    bad = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 70), 0.5)
    assert lib.graft_prune_select(1, 60, 0, P, P, P, ctypes.byref(bad), P, P, P, None, None) == L.GRAFT_EINVAL
    assert lib.graft_build_tree_mask(1, 60, 65, 0, *([P] * 9), 52, *([P] * 5), None, None) == L.GRAFT_EINVAL
    assert lib.graft_build_tree_mask(1, 60, 60, 1, *([P] * 9), 52, *([P] * 5), None, None) == L.GRAFT_EINVAL  # in-place needs T1 = Nd + 1
    assert lib.graft_verify_accept(1, 61, 100, 9, 1, *([P] * 9), 60, P, None, P, 1 << 20, None) == L.GRAFT_EINVAL
    assert lib.graft_verify_accept(1, 61, 100, 8, 1, P + 2, *([P] * 8), 60, P, None, P, 1 << 20, None) == L.GRAFT_EINVAL  # misaligned logits
    assert lib.graft_verify_accept(1, 61, 100, 8, 1, *([P] * 9), 60, P, None, P, 16, None) == L.GRAFT_EINVAL  # workspace too small
    assert lib.graft_verify_accept(1, 61, 100, 8, 1, *([P] * 6), P + 4, P, P, 60, P, None, P, 1 << 20,
                                   None) == L.GRAFT_EINVAL  # misaligned row_stats
    assert lib.graft_coverage_gain(1, 65, 100, 1, *([P] * 6), None) == L.GRAFT_EINVAL
    assert lib.graft_coverage_gain(1, 61, 100, 7, *([P] * 6), None) == L.GRAFT_EUNSUPPORTED
    assert lib.graft_coverage_gain(1, 61, 100, 1, P, P, P, P, P + 4, P, None) == L.GRAFT_EINVAL
    assert lib.graft_coverage_gain(1, 61, 100, 1, P, P, P, None, P, P, None) == L.GRAFT_EINVAL
    assert lib.graft_coverage_gain(0, 61, 100, 1, *([None] * 6), None) == 0
    # null pointers
    assert lib.graft_prune_select(1, 60, 0, None, P, P, ctypes.byref(cfg), P, P, P, None, None) == L.GRAFT_EINVAL
    assert lib.graft_update_topk(10, 100, 8, 1, None, None, None, P, P, None, None, P, 1 << 20, None) == L.GRAFT_EINVAL
    # template checks: the output rows must hold the template; a stage may not keep more than the slots
    tpl = L.Template(60, P, P, P)
    assert lib.graft_retrieve_expand(1, 100, 8, 0, 60, P, P, P, None, 60, ctypes.byref(tpl),
                                     ctypes.byref(cfg), P, P, P, 52, None) == L.GRAFT_EINVAL
    tpl = L.Template(20, P, P, P)
    over = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 61), 0.5)
    assert lib.graft_retrieve_expand(1, 100, 8, 0, 60, P, P, P, None, 60, ctypes.byref(tpl),
                                     ctypes.byref(over), P, P, P, 52, None) == L.GRAFT_EINVAL
    assert lib.graft_template_branching(8, 8, -1, 1, 52, P, P, P) == L.GRAFT_EINVAL
    assert lib.graft_template_branching(8, 8, 1, 0, 52, P, P, P) == L.GRAFT_EINVAL
    # empty batches enqueue nothing and succeed
    assert lib.graft_prune_select(0, 60, 0, None, None, None, ctypes.byref(cfg), None, None, None, None, None) == 0
    assert lib.graft_update_topk(0, 100, 8, 1, None, None, None, None, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("W,D,beta,cap", [(8, 8, (1, 1), 52), (8, 12, (3, 2), 64), (4, 6, (0, 1), 64),
                                          (6, 10, (5, 1), 52), (2, 3, (1, 1), 64), (8, 2, (1, 1), 64)])
def test_branching_template_matches_oracle(W, D, beta, cap):
    par, rk, dp = L.graft_template_branching(W, D, beta[0], beta[1], cap)
    o = O.template_branching(W, D, beta, cap)
    assert par == o["parent"].tolist() and rk == o["rank"].tolist() and dp == o["depth"].tolist()


def test_input_check_validation_rejects_without_launch():
    lib = L.load()
    P = 0x1000  # never dereferenced
    assert lib.graft_check_draft(1, 60, 9, 100, P, P, P, P, P, None) == L.GRAFT_EUNSUPPORTED
    assert lib.graft_check_draft(1, 65, 0, 100, P, P, P, P, P, None) == L.GRAFT_EINVAL
    assert lib.graft_check_draft(1, 60, 0, 0, P, P, P, P, P, None) == L.GRAFT_EINVAL
    assert lib.graft_check_draft(1, 60, 0, 100, None, P, P, P, P, None) == L.GRAFT_EINVAL
    assert lib.graft_check_draft(1, 16, 1, 100, None, None, P, P, None, None) == L.GRAFT_EINVAL
    assert lib.graft_check_draft(0, 60, 0, 100, None, None, None, None, None, None) == L.GRAFT_OK
    assert lib.graft_check_tree(1, 65, 100, P, P, P, P, None) == L.GRAFT_EINVAL
    assert lib.graft_check_tree(1, 61, 100, P, None, P, P, None) == L.GRAFT_EINVAL
    assert lib.graft_check_tree(0, 61, 100, None, None, None, None, None) == L.GRAFT_OK


def test_vocabulary_limit_rejects_without_launch():
    """Top-k calls take at most GRAFT_MAX_VOCAB logits per row (16 wavefronts
    per row, 16-bit local offsets); the header's value is the binding's."""
    src = open(os.path.join(ROOT, "include", "graft.h")).read()
    assert re.search(r"#define GRAFT_MAX_VOCAB (\d+)", src).group(1) == str(L.GRAFT_MAX_VOCAB)
    lib = L.load()
    P = 0x1000  # never dereferenced
    big = L.GRAFT_MAX_VOCAB + 1
    assert L.graft_workspace_bytes(976, big, 8, L.DTYPE_BF16) == 0
    assert L.graft_workspace_bytes(976, L.GRAFT_MAX_VOCAB, 8, L.DTYPE_BF16) > 0
    assert lib.graft_verify_accept(1, 61, big, 8, 1, *([P] * 9), 60, P, None, P, 1 << 30, None) == L.GRAFT_EINVAL
    assert lib.graft_verify_update(1, 61, big, 8, 1, *([P] * 11), 60, P, None, P, 1 << 30, None) == L.GRAFT_EINVAL
    assert lib.graft_update_topk(4, big, 8, 1, P, None, None, P, P, None, P, P, 1 << 30, None) == L.GRAFT_EINVAL
    assert lib.graft_coverage_gain(1, 61, big, 1, P, P, P, P, P, P, None) == L.GRAFT_EINVAL


def test_empty_batches_enqueue_nothing():
    """B == 0 (or n_rows == 0) returns GRAFT_OK before any pointer is looked at."""
    cfg = L.prune_cfg((0, 1, 5), (-1.2, -1.6, -2.3), (8, 24, 40), 0.5)
    lib = L.load()
    cb = ctypes.byref(cfg)
    assert lib.graft_prune_select(0, 60, 0, None, None, None, cb, None, None, None, None, None) == L.GRAFT_OK
    assert lib.graft_build_tree_mask(0, 60, 61, 0, *([None] * 9), 52, *([None] * 6), None) == L.GRAFT_OK
    assert lib.graft_build_hybrid_tree(0, 60, 61, 0, 1, 60, cb, None, 100, 8, *([None] * 14), 52,
                                       *([None] * 6), None) == L.GRAFT_OK
    assert lib.graft_verify_accept(0, 61, 100, 8, 1, *([None] * 9), 60, None, None, None, 0, None) == L.GRAFT_OK
    assert lib.graft_verify_update(0, 61, 100, 8, 1, *([None] * 11), 60, None, None, None, 0, None) == L.GRAFT_OK
    assert lib.graft_update_topk(0, 100, 8, 1, *([None] * 7), None, 0, None) == L.GRAFT_OK
    assert lib.graft_coverage_gain(0, 61, 100, 1, *([None] * 6), None) == L.GRAFT_OK
    assert lib.graft_checkpoint_stats(0, 60, None, None, None, cb, None, None) == L.GRAFT_OK
    assert lib.graft_stream_read(None, 0, 16, None, None) == L.GRAFT_OK


def test_stream_read_rejects_bad_arguments_on_the_host():
    """graft_stream_read checks its sizes and pointers before it enqueues
    anything: rows of a positive multiple of 16 bytes, 0 <= n_rows < 2^31,
    non-null 16-byte-aligned data and a non-null sink."""
    lib = L.load()
    bad = [(None, 1, 16, None), (None, -1, 16, None), (None, 1, 0, None), (None, 1, 24, None),
           (None, 1 << 31, 16, None), (ctypes.c_void_p(8), 1, 16, ctypes.c_void_p(64)),
           (ctypes.c_void_p(64), 1, 16, None)]
    for data, n, rb, sink in bad:
        assert lib.graft_stream_read(data, n, rb, sink, None) == L.GRAFT_EINVAL, (data, n, rb, sink)


def test_coordinators_are_bounded_whatever_the_batch():
    """A verify launch's coordinator workgroups wait for rows dispatched after them,
    so their number must stay far below what the chip holds at once (256 CUs,
    32 wavefronts and 160 KB of LDS each): at most GRAFT_MAX_COORD_GROUPS
    workgroups, one wavefront per request below that, for every batch the calls
    accept."""
    bf, f32 = L.DTYPE_BF16, L.DTYPE_F32
    seen_cap = False
    for T1 in (1, 2, 17, 61, 64):
        for V in (8, 100, 1024, 16000, 32000, 151936, L.GRAFT_MAX_VOCAB):
            for B in (1, 3, 4, 16, 33, 64, 127, 384, 1000, 8192, 20000, 100_000, 1_000_000, L.GRAFT_MAX_BATCH):
                for dt in (bf, f32):
                    n = B * T1
                    if L.graft_workspace_bytes(n, V, min(8, V), dt) == 0:
                        continue
                    p = L.graft_launch_plan(n, V, dt, T1)
                    S = p["waves_per_group"]
                    assert 1 <= S <= 16
                    assert p["coord_groups"] == min(-(-B // S), L.GRAFT_MAX_COORD_GROUPS)
                    # a quarter of the chip's 8192 wavefront slots at most
                    assert p["coord_groups"] * S <= 2048
                    assert p["workgroups"] == n * p["groups_per_row"] + p["coord_groups"]
                    assert p["workgroups"] * S * 64 < 2 ** 32
                    seen_cap |= p["coord_groups"] == L.GRAFT_MAX_COORD_GROUPS
    assert seen_cap
    # the case found by reading the old code: 8192 one-wavefront coordinators
    p = L.graft_launch_plan(8192 * 17, 16000, bf, 17)
    assert p["waves_per_group"] <= 2 and p["coord_groups"] == L.GRAFT_MAX_COORD_GROUPS
    # the prompt ingest has no requests: an update-only launch needs a registration
    # workgroup unless its rows find their token's last holder themselves (merge-wave
    # rows, at most 1025 of them: 16 x 64 later rows held in registers)
    q = L.graft_launch_plan(2048, 151936, bf, 0)
    assert q["merge_wave"] == 1 and q["holder_scan"] == 0 and q["coord_groups"] == 1
    q = L.graft_launch_plan(1024, 151936, bf, 0)
    assert q["merge_wave"] == 1 and q["holder_scan"] == 1 and q["coord_groups"] == 0
    assert L.graft_launch_plan(1025, 151936, bf, 1)["holder_scan"] == 1
    assert L.graft_launch_plan(1026, 151936, bf, 1)["holder_scan"] == 0
    assert L.graft_launch_plan(16 * 17, 151936, bf, 17)["holder_scan"] == 0      # rows cut into slices
    assert L.graft_launch_plan(0, 151936, bf, 0)["workgroups"] == 0
    # the metric shape keeps one coordinator wavefront per request
    p = L.graft_launch_plan(16 * 61, 151936, bf, 61)
    assert (p["waves_per_group"], p["groups_per_row"], p["blocks_per_batch"], p["coord_groups"]) == (4, 1, 2, 4)
    # ... with a merge wavefront per row and the per-row launch counters
    assert (p["merge_wave"], p["launch_counters"]) == (1, 1)
    # few-row launches: 61 rows cut into 4 slices of 8 waves, four blocks per
    # batch from 6 blocks per wave (128256 bf16: ~7.8), two below (32000 fp32:
    # ~3.9); 183-256 rows whole, 8 waves each; TAIL rows in 4 slices of 2 waves
    shape = lambda q: (q["waves_per_group"], q["groups_per_row"], q["blocks_per_batch"], q["merge_wave"])
    assert shape(L.graft_launch_plan(61, 128256, bf, 61)) == (8, 4, 4, 0)
    assert shape(L.graft_launch_plan(61, 32000, L.DTYPE_F32, 61)) == (8, 4, 2, 0)
    assert shape(L.graft_launch_plan(4 * 61, 151936, bf, 61)) == (8, 1, 4, 0)
    assert shape(L.graft_launch_plan(183, 151936, bf, 61)) == (8, 1, 4, 0)
    assert shape(L.graft_launch_plan(244, 40000, L.DTYPE_F32, 0)) == (8, 1, 4, 0)
    # 436-511 rows: two whole rows on nearly every CU, 8 waves; 427 rows stay in slices
    assert shape(L.graft_launch_plan(8 * 61, 151936, bf, 61)) == (8, 1, 4, 0)
    assert shape(L.graft_launch_plan(436, 151936, bf, 0)) == (8, 1, 4, 0)
    assert shape(L.graft_launch_plan(7 * 61, 151936, bf, 61))[1] > 1
    assert shape(L.graft_launch_plan(488, 10 ** 6, bf, 0))[1] > 1           # 8 waves would exceed the cap
    # split bf16 rows: 8 waves per slice from 68 blocks per slice (122 rows at 151936), 4 below (128256); fp32 unchanged
    assert shape(L.graft_launch_plan(2 * 61, 151936, bf, 61)) == (8, 4, 4, 0)
    assert shape(L.graft_launch_plan(2 * 61, 128256, bf, 61)) == (4, 4, 4, 0)
    assert shape(L.graft_launch_plan(2 * 61, 151936, L.DTYPE_F32, 61))[0] == 4
    assert shape(L.graft_launch_plan(256, 10 ** 6, bf, 0)) == (16, 1, 2, 0)   # 8 waves would exceed 127 blocks each
    assert shape(L.graft_launch_plan(16 * 17, 151936, bf, 17)) == (2, 4, 4, 0)
    # the counters cover verify launches of up to 16384 rows (rows cut into slices
    # too); an update-only launch has no completion words
    n_ctr = L.GRAFT_WS_COUNTER_BYTES // 12
    assert n_ctr == 16384
    assert L.graft_launch_plan(n_ctr, 151936, bf, 1)["launch_counters"] == 1
    assert L.graft_launch_plan(n_ctr + 1, 151936, bf, 1)["launch_counters"] == 0
    assert L.graft_launch_plan(2048, 151936, bf, 0)["launch_counters"] == 0
    q = L.graft_launch_plan(16 * 17, 151936, bf, 17)
    assert q["groups_per_row"] > 1 and (q["merge_wave"], q["launch_counters"]) == (0, 1)
    # every workspace starts with the counters
    assert L.graft_workspace_bytes(1, 100, 8, bf) > L.GRAFT_WS_COUNTER_BYTES
    with pytest.raises(L.GraftError):
        L.graft_launch_plan(100, 1000, bf, 61)   # T1 does not divide the rows


def test_launch_plans_keep_the_per_wave_block_cap():
    """Over many shapes, every plan keeps each wavefront of a row (or slice) within
    the blocks its local offsets can address (bf16: 127 blocks of 512 elements;
    fp32: 1023 blocks of 256 — past that, wave-local ranks would collide), uses
    the merge wavefront only for whole rows of at most 4 streaming waves, and
    never more than 16 wavefronts per workgroup."""
    rng = np.random.default_rng(11)
    shapes = [(n, V) for n in (1, 5, 61, 100, 182, 183, 244, 256, 272, 300, 488, 511, 512, 976, 1024, 1600, 2048,
                               4096, 16384) for V in (9, 1001, 4097, 16000, 32000, 128256, 151936, 999_999)]
    shapes += [(int(rng.integers(1, 20000)), int(rng.integers(8, 1_000_001))) for _ in range(300)]
    for n, V in shapes:
        for dt, epg, cap in ((L.DTYPE_BF16, 8, 127), (L.DTYPE_F32, 4, 1023)):
            if L.graft_workspace_bytes(n, V, min(8, V), dt) == 0:
                continue
            p = L.graft_launch_plan(n, V, dt, 0)
            S = p["waves_per_group"] - p["merge_wave"]
            G = p["groups_per_row"]
            assert 1 <= S and p["waves_per_group"] <= 16, (n, V, dt, p)
            assert p["blocks_per_batch"] in (2, 4)
            if p["merge_wave"]:
                assert G == 1 and S <= 4, (n, V, dt, p)
            nblk = -(-(-(-V // epg)) // 64)          # 1 KB blocks of a row, at most
            per_wave = -(-(-(-nblk // G)) // S)      # blocks of one wavefront, at most
            assert per_wave <= cap, (n, V, dt, p, per_wave)
