"""Chunk -> rank planner (host code of the library, no GPU): valid plans,
optimal with two chunks per rank (against exhaustive search), never worse
than the dual-chunk / snake assignment, and the argument checks."""
import ctypes as C

import numpy as np
import pytest

from oracle import masks as OM
from synth import masks as SM
import masked_tiled_attention_amd as fm
from masked_tiled_attention_amd import _lib as L


def _snake(c, r):
    return [(i % r) if (i // r) % 2 == 0 else r - 1 - (i % r) for i in range(c)]


def _check_valid(work, r, plan, mx):
    c = len(work)
    assert sorted(plan) == sorted(list(range(r)) * (c // r))
    assert mx == int(OM.plan_loads(work, plan, r).max())


@pytest.mark.parametrize("c,r", [(4, 2), (6, 3), (8, 4), (10, 5)])
def test_two_per_rank_is_optimal(c, r):
    rng = np.random.default_rng(c * 10 + r)
    for _ in range(12):
        work = rng.integers(0, 1000, c)
        plan, mx = fm.fm_cp_plan(work, r)
        _check_valid(work, r, plan, mx)
        assert mx == OM.best_plan_max(work, r)


@pytest.mark.parametrize("c,r", [(6, 2), (9, 3), (8, 2), (12, 4)])
def test_more_per_rank_valid_and_not_worse_than_snake(c, r):
    rng = np.random.default_rng(c * 7 + r)
    gaps = []
    for _ in range(10):
        work = rng.integers(0, 1000, c)
        plan, mx = fm.fm_cp_plan(work, r)
        _check_valid(work, r, plan, mx)
        assert mx <= int(OM.plan_loads(work, _snake(c, r), r).max())
        best = OM.best_plan_max(work, r)
        assert best <= mx <= 1.15 * best
        gaps.append(mx / max(best, 1))
    assert np.mean(gaps) < 1.05


def test_document_mask_plan_beats_dual_chunk():
    """Document-causal work of 16 chunks on 8 ranks (the rank-share layout at
    a reduced size): the plan's largest load is at most dual-chunk's."""
    n, deg = 8192, 8
    docs = SM.lognormal_doc_lengths(np.random.default_rng(5), n, 512, 1.0, 16, 4096)
    vec = tuple(np.asarray(x)[None, None] for x in SM.document_causal(docs))
    cl = n // (2 * deg)
    starts = [i * cl for i in range(2 * deg)]
    work = OM.chunk_work(vec, n, starts, [cl] * (2 * deg))[0]
    plan, mx = fm.fm_cp_plan(work, deg)
    _check_valid(work, deg, plan, mx)
    dual = [min(i, 2 * deg - 1 - i) for i in range(2 * deg)]
    assert mx <= int(OM.plan_loads(work, dual, deg).max())


def test_plan_rejects_bad_arguments():
    lib = L.load()
    w = (C.c_int64 * 6)(1, 2, 3, 4, 5, 6)
    out = (C.c_int32 * 6)()
    assert lib.fm_cp_plan(w, 6, 4, out, None) == L.FM_ERR_INVALID_ARGUMENT   # 6 chunks on 4 ranks
    assert lib.fm_cp_plan(w, 6, 0, out, None) == L.FM_ERR_INVALID_ARGUMENT
    neg = (C.c_int64 * 2)(5, -1)
    assert lib.fm_cp_plan(neg, 2, 1, out, None) == L.FM_ERR_INVALID_ARGUMENT
    assert lib.fm_cp_plan(w, 6, 3, out, None) == L.FM_OK
