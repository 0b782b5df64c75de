"""GPU integer steps vs the oracle, bit-exact: tile summaries, tile classes
(both orders, kernel tiles and others, broadcast masks, ragged edges,
non-canonical bounds) and mask localization (hand-worked cases, random
chunk lists, the dual-chunk rank share at full size)."""
import numpy as np
import pytest
import torch

from gpu_util import dev_mask, log
from oracle import masks as OM
from synth import configs as SC
from synth import masks as SM

pytestmark = pytest.mark.gpu


def _family_vectors(n, rng):
    docs = SM.uniform_doc_lengths(rng, n, 16, 200)
    return {
        "causal": SM.causal(n),
        "document": SM.document_causal(docs),
        "window": SM.sliding_window_causal(n, 97),
        "prefix": SM.prefix_lm(n, n // 3),
        "share_question": SM.share_question(n // 5, SM.answer_lengths(rng, n - n // 5, 4)),
        "none": SM.no_mask(n, n),
    }


def _check_classes(vec, sq, sk, bq, bk, fm):
    mask = dev_mask(vec)
    bm, hm = vec[0].shape[:2] if vec[0] is not None else vec[2].shape[:2]
    for transposed in (False, True):
        summ, cls = fm.fm_tile_classify(mask, sq, sk, bq, bk, transposed)
        torch.cuda.synchronize()
        summ, cls = summ.cpu().numpy(), cls.cpu().numpy()
        for b in range(bm):
            for h in range(hm):
                ref_s = OM.tile_summary(vec, sq, sk, bk, b, h)
                ref_c = OM.tile_classes(vec, sq, sk, bq, bk, b, h)
                assert np.array_equal(summ[b, h], ref_s), "summary"
                got = cls[b, h].T if transposed else cls[b, h]
                assert np.array_equal(got, ref_c), f"classes transposed={transposed}"


@pytest.mark.parametrize("n", [700, 1000, 64, 1])
def test_classes_mask_families(gpu_lib, n):
    fm = gpu_lib
    rng = np.random.default_rng(n)
    for name, v in _family_vectors(n, rng).items() if n > 8 else [("causal", SM.causal(n))]:
        vec = tuple(x[None, None] for x in v)
        for bq, bk in (fm.fm_kernel_tile(128, False), fm.fm_kernel_tile(128, True), (16, 48), (100, 7)):
            log(f"classes {name} n={n} tiles=({bq},{bk})")
            _check_classes(vec, n, n, bq, bk, fm)


def test_classes_random_and_broadcast(gpu_lib):
    fm = gpu_lib
    rng = np.random.default_rng(7)
    for trial in range(6):
        sq, sk = int(rng.integers(1, 900)), int(rng.integers(1, 900))
        bm, hm = int(rng.choice([1, 2])), int(rng.choice([1, 3]))
        vec = tuple(rng.integers(-50, sq + 50, (bm, hm, sk)).astype(np.int32) for _ in range(4))
        if trial == 4:
            vec = (None, None) + vec[2:]
        if trial == 5:
            vec = vec[:2] + (None, None)
        log(f"classes random trial={trial} sq={sq} sk={sk} bm={bm} hm={hm}")
        for bq, bk in ((128, 64), (64, 128), (33, 17)):
            _check_classes(vec, sq, sk, bq, bk, fm)


def test_classes_extreme_bounds(gpu_lib):
    """Bounds at the int32 limits are legal and classified by the same rule."""
    fm = gpu_lib
    sk, sq = 300, 257
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    rng = np.random.default_rng(3)
    vec = tuple(rng.choice(np.array([lo, hi, 0, 5, sq, sq + 1, -1], np.int32), (1, 1, sk)) for _ in range(4))
    _check_classes(vec, sq, sk, 128, 64, fm)


def test_localize_golden(gpu_lib):
    import json
    import os
    fm = gpu_lib
    with open(os.path.join(os.path.dirname(__file__), "golden", "localize_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.asarray(c["global"], dtype=np.int32)[None, None]
        loc = fm.fm_mask_localize(dev_mask((x, x, x, x)), c["seq_q_global"], c["chunk_start"], c["chunk_len"])
        got = loc.lts.cpu().numpy()[0, 0].tolist()
        log(f"localize golden: {c['note']}")
        assert got == c["local"]


def test_localize_random_vs_counting(gpu_lib):
    fm = gpu_lib
    rng = np.random.default_rng(17)
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    for trial in range(20):
        sq = int(rng.integers(1, 5000))
        sk = int(rng.integers(1, 3000))
        bm, hm = int(rng.choice([1, 2])), int(rng.choice([1, 4]))
        k = int(rng.integers(1, 9))
        cuts = np.sort(rng.choice(np.arange(sq + 1), size=2 * k, replace=True))
        starts, lens = cuts[0::2], cuts[1::2] - cuts[0::2]
        keep = lens > 0
        if not keep.any():
            starts, lens = np.array([0]), np.array([sq])
        else:
            starts, lens = starts[keep], lens[keep]
        s2, l2, end = [], [], 0
        for s, l in zip(starts, lens):
            if s >= end:
                s2.append(int(s))
                l2.append(int(l))
                end = s + l
        vec = [rng.integers(-100, sq + 100, (bm, hm, sk)).astype(np.int32) for _ in range(4)]
        vec[0][..., :3] = [lo, hi, 0]
        vec = tuple(vec)
        if trial % 5 == 4:
            vec = (None, None) + vec[2:]
        log(f"localize trial={trial} sq={sq} sk={sk} chunks={len(s2)}")
        got = fm.fm_mask_localize(dev_mask(vec), sq, s2, l2)
        ref = OM.localize(vec, s2, l2)
        for i, (g, r) in enumerate(zip((got.lts, got.lte, got.uts, got.ute), ref)):
            if r is None:
                assert g is None
            else:
                assert np.array_equal(g.cpu().numpy(), r), f"vector {i}"


def test_localize_dual_chunk_full_size(gpu_lib):
    """The context-parallel rank share (rank 3 of 8, dual-chunk, global 65536)
    at full size: bit-exact localized vectors, dense slice equality on sampled
    rows, and exact classes of the localized mask with the kernels' tiles."""
    fm = gpu_lib
    from oracle import attention as OA
    w = SC.build("c5_cp_rank3_of_8", 0, tensors=False)
    got = fm.fm_mask_localize(dev_mask(w.global_vectors), w.seq_q_global, w.chunk_start, w.chunk_len)
    ref = OM.localize(w.global_vectors, w.chunk_start, w.chunk_len)
    gv = tuple(x.cpu().numpy() for x in (got.lts, got.lte, got.uts, got.ute))
    for g, r in zip(gv, ref):
        assert np.array_equal(g, r)
    rng = np.random.default_rng(0)
    rows = rng.choice(w.seq_q, 64, replace=False)
    dl = OA.dense_mask(*[x[0, 0].astype(np.int64) for x in gv], rows)
    dg = OA.dense_mask(*[x[0, 0].astype(np.int64) for x in w.global_vectors], w.local_rows[rows])
    assert np.array_equal(dl, dg)
    for bwd in (False, True):
        bq, bk = fm.fm_kernel_tile(128, bwd)
        _, cls = fm.fm_tile_classify(got, w.seq_q, w.seq_k, bq, bk)
        dense = OM.tile_classes_dense(ref, w.seq_q, w.seq_k, bq, bk)
        assert np.array_equal(cls.cpu().numpy()[0, 0], dense), "classes exact on the localized mask"


def _check_transfer(vec, sq, sk, bk, fm, tag):
    log(f"transfer set {tag} sq={sq} sk={sk} block_k={bk}")
    need, count = fm.fm_kv_transfer_set(dev_mask(vec), sq, bk)
    torch.cuda.synchronize()
    ref = OM.transfer_set(vec, sq, sk, bk)
    assert np.array_equal(need.cpu().numpy(), ref), f"need {tag}"
    assert np.array_equal(count.cpu().numpy(), ref.sum(axis=2).astype(np.int32)), f"count {tag}"
    return ref


@pytest.mark.parametrize("n", [700, 64, 1])
def test_transfer_set_mask_families(gpu_lib, n):
    """Bit-exact need flags and counts on every mask family, for all rows and
    for localized dual-chunk ranks, with kernel and odd key tiles."""
    fm = gpu_lib
    rng = np.random.default_rng(n + 1)
    fams = _family_vectors(n, rng) if n > 8 else {"causal": SM.causal(n)}
    for name, v in fams.items():
        vec = tuple(x[None, None] for x in v)
        for bk in sorted({fm.fm_kernel_tile(128, False)[1], fm.fm_kernel_tile(128, True)[1], 1, 7, 200}):
            if bk > n:
                continue
            _check_transfer(vec, n, n, bk, fm, f"{name} all rows")
        if n % 8 == 0:
            for degree, rank in ((2, 1), (4, 0), (4, 3)):
                cs, cl = SM.dual_chunk(n, degree, rank)
                loc = OM.localize(vec, cs, cl)
                _check_transfer(loc, int(sum(cl)), n, 16, fm, f"{name} rank {rank}/{degree}")


def test_transfer_set_random_and_extreme(gpu_lib):
    """Random and int32-limit bounds, broadcast shapes, a missing pair, one
    key per tile and a single tile."""
    fm = gpu_lib
    rng = np.random.default_rng(29)
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    for trial in range(8):
        sq, sk = int(rng.integers(1, 600)), int(rng.integers(1, 900))
        bm, hm = int(rng.choice([1, 2])), int(rng.choice([1, 3]))
        vec = [rng.integers(-50, sq + 50, (bm, hm, sk)).astype(np.int32) for _ in range(4)]
        if trial % 2:
            pick = np.array([lo, hi, 0, 1, sq - 1, sq, sq + 1, -1], np.int32)
            vec = [rng.choice(pick, (bm, hm, sk)) for _ in range(4)]
        if trial == 4:
            vec[0] = vec[1] = None
        if trial == 5:
            vec[2] = vec[3] = None
        for bk in (1, 64, sk):
            _check_transfer(tuple(vec), sq, sk, bk, fm, f"random trial={trial}")


def test_transfer_set_rank_share_full_size(gpu_lib):
    """The context-parallel rank share (rank 3 of 8, dual-chunk, global 65536,
    document-causal) at full size with the kernels' key tiles: bit-exact
    against the dense truth, and equal to the OR of the exact tile classes."""
    fm = gpu_lib
    w = SC.build("c5_cp_rank3_of_8", 0, tensors=False)
    loc = fm.fm_mask_localize(dev_mask(w.global_vectors), w.seq_q_global, w.chunk_start, w.chunk_len)
    ref_loc = OM.localize(w.global_vectors, w.chunk_start, w.chunk_len)
    for bwd in (False, True):
        bq, bk = fm.fm_kernel_tile(128, bwd)
        need, count = fm.fm_kv_transfer_set(loc, w.seq_q, bk)
        ref = OM.transfer_set(ref_loc, w.seq_q, w.seq_k, bk)
        assert np.array_equal(need.cpu().numpy(), ref)
        assert int(count.cpu()[0, 0]) == int(ref.sum())
        _, cls = fm.fm_tile_classify(loc, w.seq_q, w.seq_k, bq, bk)
        assert np.array_equal(ref[0, 0], (cls.cpu().numpy()[0, 0] != 0).any(axis=0).astype(np.uint8))
        log(f"rank share: {int(ref.sum())} of {ref.shape[2]} key tiles of {bk} keys needed")


def _check_chunk_work(vec, sq, sk, starts, lens, fm, tag):
    log(f"chunk work {tag} sq={sq} sk={sk} chunks={len(starts)}")
    got = fm.fm_chunk_work(dev_mask(vec), sq, starts, lens).cpu().numpy()
    ref = OM.chunk_work(vec, sk, starts, lens)
    assert np.array_equal(got, ref), tag


def test_chunk_work_families_and_random(gpu_lib):
    """Bit-exact open-pair counts per chunk: every mask family under
    dual-chunk layouts and random chunk lists, random and int32-limit bounds,
    broadcast shapes and a missing pair."""
    fm = gpu_lib
    rng = np.random.default_rng(37)
    n = 640
    for name, v in _family_vectors(n, rng).items():
        vec = tuple(x[None, None] for x in v)
        for degree, rank in ((2, 0), (4, 3), (8, 5)):
            cs, cl = SM.dual_chunk(n, degree, rank)
            _check_chunk_work(vec, n, n, list(cs), list(cl), fm, f"{name} rank {rank}/{degree}")
        _check_chunk_work(vec, n, n, [i * 40 for i in range(16)], [40] * 16, fm, f"{name} 16 chunks")
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    for trial in range(6):
        sq, sk = int(rng.integers(2, 700)), int(rng.integers(1, 900))
        bm, hm = int(rng.choice([1, 2])), int(rng.choice([1, 3]))
        vec = [rng.integers(-50, sq + 50, (bm, hm, sk)).astype(np.int32) for _ in range(4)]
        if trial % 2:
            pick = np.array([lo, hi, 0, 1, sq - 1, sq, sq + 1, -1], np.int32)
            vec = [rng.choice(pick, (bm, hm, sk)) for _ in range(4)]
        if trial == 4:
            vec[0] = vec[1] = None
        cuts = np.unique(np.concatenate([[0, sq], rng.integers(0, sq + 1, int(rng.integers(1, 12)))]))
        _check_chunk_work(tuple(vec), sq, sk, list(cuts[:-1]), list(np.diff(cuts)), fm, f"random trial={trial}")


def test_chunk_work_and_plan_full_size(gpu_lib):
    """The global 64K document-causal mask in 16 chunks of 4096 (the rank-share
    layout): the chunks add up to the closed-form pair count, two chunks match
    the dense truth, and the plan for 8 ranks is no worse than dual-chunk."""
    fm = gpu_lib
    from oracle import attention as OA
    w = SC.build("c5_cp_rank3_of_8", 0, tensors=False)
    n = w.seq_q_global
    starts, lens = [i * 4096 for i in range(16)], [4096] * 16
    got = fm.fm_chunk_work(dev_mask(w.global_vectors), n, starts, lens).cpu().numpy()[0]
    assert int(got.sum()) == OA.nnz_closed_form(w.global_vectors, n)
    for c in (3, 12):
        assert got[c] == OM.chunk_work(w.global_vectors, w.seq_k, [starts[c]], [lens[c]])[0, 0]
    plan, mx = fm.fm_cp_plan(got, 8)
    dual = [min(i, 15 - i) for i in range(16)]
    dual_max = int(OM.plan_loads(got, dual, 8).max())
    assert mx <= dual_max
    log(f"rank loads: mean {got.sum() / 8:.4g}, dual-chunk max {dual_max:.4g}, planned max {mx:.4g}")
