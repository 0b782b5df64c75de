"""Backward parity: dQ, dK, dV from the HIP kernels (through the C ABI, fed
with the HIP forward's O and LSE as in training) vs the float64 oracle's exact
gradients, element by element, plus edge cases and the gradient invariants."""
import math

import numpy as np
import pytest
import torch

from gpu_util import BF16_ROUND, assert_close, dev_mask, log, np64
from oracle import attention as OA
from synth import masks as SM
from synth import tensors as ST

pytestmark = pytest.mark.gpu


def _families(n, rng):
    return {
        "causal": SM.causal(n),
        "document": SM.document_causal(SM.uniform_doc_lengths(rng, n, 40, 300)),
        "window": SM.sliding_window_causal(n, 150),
        "prefix_lm": SM.prefix_lm(n, n // 4),
        "share_question": SM.share_question(n // 6, SM.answer_lengths(rng, n - n // 6, 5)),
        "none": SM.no_mask(n, n),
    }


def _run(fm, q, k, v, do, vec, scale):
    q, k, v, do = (t.cuda() for t in (q, k, v, do))
    m = dev_mask(vec)
    o, lse = fm.fm_attn_fwd(q, k, v, m, scale)
    dq, dk, dv = fm.fm_attn_bwd(q, k, v, o, lse, do, m, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _compare(fm, q, k, v, do, vec, scale, tag, out_round=0.0):
    log(f"bwd {tag} q={tuple(q.shape)} k={tuple(k.shape)} dtype={q.dtype}")
    dq, dk, dv = _run(fm, q, k, v, do, vec, scale)
    rq, rk, rv = OA.backward(np64(q), np64(k), np64(v), np64(do), vec, scale)
    assert_close(np64(dq), rq, f"{tag} dQ", out_round=out_round)
    assert_close(np64(dk), rk, f"{tag} dK", out_round=out_round)
    assert_close(np64(dv), rv, f"{tag} dV", out_round=out_round)
    return dq, dk, dv


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_mask_families(gpu_lib, d):
    rng = np.random.default_rng(100 + d)
    n = 700
    for name, v in _families(n, rng).items():
        q, k, vv, do = ST.qkv(2, n, n, 3, d, seed=d + len(name), with_do=True)
        _compare(gpu_lib, q, k, vv, do, tuple(x[None, None] for x in v), 1 / math.sqrt(d), f"{name} d={d}")


def test_bwd_per_batch_and_head_masks(gpu_lib):
    rng = np.random.default_rng(11)
    n, B, H, d = 520, 2, 3, 128
    per = [[list(_families(n, rng).values())[(b * H + h) % 6] for h in range(H)] for b in range(B)]
    vec = SM.stack(per)
    q, k, v, do = ST.qkv(B, n, n, H, d, seed=15, with_do=True)
    _compare(gpu_lib, q, k, v, do, vec, 0.09, "per-(b,h) masks")


def test_bwd_random_vectors_rectangular(gpu_lib):
    rng = np.random.default_rng(12)
    for sq, sk in ((300, 900), (900, 300), (129, 65)):
        vec = tuple(rng.integers(-20, sq + 20, (1, 1, sk)).astype(np.int32) for _ in range(4))
        q, k, v, do = ST.qkv(1, sq, sk, 2, 128, seed=sq + 1, with_do=True)
        dq, dk, dv = _compare(gpu_lib, q, k, v, do, vec, 0.1, f"random {sq}x{sk}")
        allowed = ~OA.dense_mask(*[x[0, 0].astype(np.int64) for x in vec], np.arange(sq), sk)
        empty = torch.from_numpy(~allowed.any(axis=1))
        assert torch.all(dq[:, empty] == 0)


@pytest.mark.parametrize("sq,sk", [(1, 1), (1, 1000), (1000, 1), (64, 128), (65, 129)])
def test_bwd_tiny_and_edge_shapes(gpu_lib, sq, sk):
    rng = np.random.default_rng(sq * 5 + sk)
    vec = tuple(rng.integers(-2, sq + 2, (1, 1, sk)).astype(np.int32) for _ in range(2)) + \
        (np.zeros((1, 1, sk), np.int32), np.zeros((1, 1, sk), np.int32))
    q, k, v, do = ST.qkv(1, sq, sk, 1, 64, seed=sq + 2 * sk, with_do=True)
    # with one key, dV sums dO over up to 1000 rows (|dV| ~ 90): a bf16 output
    # cannot hold that within 2e-2, so for that shape alone the bar adds the
    # output's own rounding
    rnd = BF16_ROUND if (sq, sk) == (1000, 1) else 0.0
    _compare(gpu_lib, q, k, v, do, vec, 0.125, f"edge {sq}x{sk}", out_round=rnd)


def test_bwd_float32_inputs(gpu_lib):
    n = 300
    vec = tuple(x[None, None] for x in SM.causal(n))
    q, k, v, do = ST.qkv(1, n, n, 2, 64, seed=3, dtype=torch.float32, with_do=True)
    _compare(gpu_lib, q, k, v, do, vec, 0.125, "fp32 causal")


def test_bwd_invariants(gpu_lib):
    """sum_j dK_j = 0 and sum_j dV_j = sum over rows with an open key of dO_i
    (softmax shift invariance), on the GPU's own gradients."""
    n = 800
    rng = np.random.default_rng(5)
    vec = tuple(x[None, None] for x in SM.share_question(100, SM.answer_lengths(rng, n - 100, 5)))
    q, k, v, do = ST.qkv(1, n, n, 2, 128, seed=21, with_do=True)
    dq, dk, dv = _run(gpu_lib, q, k, v, do, vec, 0.1)
    sdk = np64(dk).sum(axis=1)
    sdv = np64(dv).sum(axis=1)
    ref = np64(do).sum(axis=1)
    scale_ref = np.abs(np64(dk)).sum(axis=1).max()
    assert np.abs(sdk).max() <= 1e-2 * scale_ref, np.abs(sdk).max()
    assert_close(sdv, ref, "sum dV = sum dO", max_abs=0.25, rel_l2=1e-2)


# ---------------------------------------------------------------- stored dS
def _run_ds(fm, q, k, v, do, vec, scale, short=0):
    """Backward with the workspace that lets it store dS (minus `short` bytes)."""
    q, k, v, do = (t.cuda() for t in (q, k, v, do))
    m = dev_mask(vec)
    o, lse = fm.fm_attn_fwd(q, k, v, m, scale)
    nbytes = fm.fm_bwd_workspace_size_ds(q, k, v, m, scale) - short
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = fm.fm_attn_bwd(q, k, v, o, lse, do, m, scale, workspace=ws)
    dq0, dk0, dv0 = fm.fm_attn_bwd(q, k, v, o, lse, do, m, scale)   # minimum workspace: recompute
    torch.cuda.synchronize()
    return [t.cpu() for t in (dq, dk, dv, dq0, dk0, dv0)]


def _compare_ds(fm, q, k, v, do, vec, scale, tag, short=0, out_round=0.0):
    log(f"bwd stored-dS {tag} q={tuple(q.shape)} k={tuple(k.shape)} dtype={q.dtype} short={short}")
    dq, dk, dv, dq0, dk0, dv0 = _run_ds(fm, q, k, v, do, vec, scale, short)
    rq, rk, rv = OA.backward(np64(q), np64(k), np64(v), np64(do), vec, scale)
    assert_close(np64(dq), rq, f"{tag} dQ", out_round=out_round)
    assert_close(np64(dk), rk, f"{tag} dK", out_round=out_round)
    assert_close(np64(dv), rv, f"{tag} dV", out_round=out_round)
    # dK and dV do not depend on the dQ path
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
    return dq, dq0


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_stored_ds_mask_families(gpu_lib, d):
    rng = np.random.default_rng(300 + d)
    n = 700
    for name, v in _families(n, rng).items():
        q, k, vv, do = ST.qkv(2, n, n, 3, d, seed=d + 7 * len(name), with_do=True)
        _compare_ds(gpu_lib, q, k, vv, do, tuple(x[None, None] for x in v), 1 / math.sqrt(d), f"{name} d={d}")


def test_bwd_stored_ds_per_batch_and_head_masks(gpu_lib):
    rng = np.random.default_rng(21)
    n, B, H, d = 520, 2, 3, 128
    per = [[list(_families(n, rng).values())[(b * H + h + 1) % 6] for h in range(H)] for b in range(B)]
    vec = SM.stack(per)
    q, k, v, do = ST.qkv(B, n, n, H, d, seed=25, with_do=True)
    _compare_ds(gpu_lib, q, k, v, do, vec, 0.09, "per-(b,h) masks")


def test_bwd_stored_ds_random_vectors_rectangular(gpu_lib):
    rng = np.random.default_rng(22)
    for sq, sk in ((300, 900), (900, 300), (129, 65)):
        vec = tuple(rng.integers(-20, sq + 20, (1, 1, sk)).astype(np.int32) for _ in range(4))
        q, k, v, do = ST.qkv(1, sq, sk, 2, 128, seed=sq + 3, with_do=True)
        _compare_ds(gpu_lib, q, k, v, do, vec, 0.1, f"random {sq}x{sk}")


def test_bwd_key_tiles_masked_for_every_row(gpu_lib):
    """Keys [128, 384) are masked for every row, so two whole 128-key tiles
    have no non-SKIP query tile: their dK / dV are exactly 0 and the key tiles
    around them match the oracle, with the minimum and the stored-dS
    workspace."""
    n, d = 700, 128
    lts, lte, uts, ute = (np.array(x) for x in SM.causal(n))
    lts[128:384], lte[128:384] = 0, n
    vec = tuple(x[None, None] for x in (lts, lte, uts, ute))
    q, k, v, do = ST.qkv(1, n, n, 2, d, seed=41, with_do=True)
    _, dk, dv = _compare(gpu_lib, q, k, v, do, vec, 1 / math.sqrt(d), "dead key tiles")
    assert torch.all(dk[:, 128:384] == 0) and torch.all(dv[:, 128:384] == 0)
    _compare_ds(gpu_lib, q, k, v, do, vec, 1 / math.sqrt(d), "dead key tiles, stored dS")


@pytest.mark.parametrize("hkv", [2, 1])
def test_bwd_mostly_dead_key_tiles(gpu_lib, hkv):
    """Only keys [0, 200) are open (causal among them), so 30 of the 32
    key tiles of 128 keys have no non-SKIP tile. The workgroups with work
    write the zeros of up to four empty key tiles each and the remaining
    empty ones write their own, so both kinds run. 2 query heads on hkv K/V
    heads (one K/V head: float32 partials per query head, summed afterwards);
    both workspaces."""
    sq, sk, H, d = 256, 4096, 2, 128
    j = np.arange(sk)
    vec = tuple(np.ascontiguousarray(x.astype(np.int32)[None, None]) for x in (
        np.where(j < 200, sq, 0), np.full(sk, sq), np.zeros(sk), np.where(j < 200, j, 0)))
    q, k, v, do = ST.qkv(1, sq, sk, H, d, seed=43, with_do=True)
    k, v = k[:, :, :hkv].contiguous(), v[:, :, :hkv].contiguous()
    _, dk, dv = _compare(gpu_lib, q, k, v, do, vec, 1 / math.sqrt(d), f"dead key tiles, {hkv} K/V heads")
    assert torch.all(dk[:, 200:] == 0) and torch.all(dv[:, 200:] == 0)
    # (dK, dV of the stored-dS backward equal those of the recompute one, bit for bit)
    _compare_ds(gpu_lib, q, k, v, do, vec, 1 / math.sqrt(d), f"dead key tiles, {hkv} K/V heads, stored dS")


def test_bwd_stored_ds_more_key_tiles_than_one_list(gpu_lib):
    """140,000 keys: 1094 key tiles, more than one compacted list of the dQ
    kernel, which then walks its key tiles in two passes. With so few query
    tiles the lists are also split into parts (8 here, 4 for the random mask
    over 16,384 keys) whose partial dQ a second kernel sums."""
    sq, sk = 200, 140000
    vec = tuple(x[None, None] for x in SM.no_mask(sk, sq))
    q, k, v, do = ST.qkv(1, sq, sk, 1, 128, seed=43, with_do=True)
    _compare_ds(gpu_lib, q, k, v, do, vec, 0.088, "140k keys")
    rng = np.random.default_rng(44)
    sq, sk = 300, 16384
    vec = tuple(rng.integers(-20, sq + 20, (1, 1, sk)).astype(np.int32) for _ in range(4))
    q, k, v, do = ST.qkv(1, sq, sk, 2, 128, seed=45, with_do=True)
    _compare_ds(gpu_lib, q, k, v, do, vec, 0.088, "random 300x16384")
    # float32 inputs, head_dim 64: the same split with float32 partials and output
    q, k, v, do = ST.qkv(1, 200, 16384, 1, 64, seed=46, dtype=torch.float32, with_do=True)
    _compare_ds(gpu_lib, q, k, v, do, tuple(x[None, None] for x in SM.no_mask(16384, 200)), 0.125,
                "float32 200x16384", out_round=0.0)


def test_bwd_stored_ds_float32_inputs(gpu_lib):
    n = 300
    vec = tuple(x[None, None] for x in SM.causal(n))
    q, k, v, do = ST.qkv(1, n, n, 2, 64, seed=4, dtype=torch.float32, with_do=True)
    _compare_ds(gpu_lib, q, k, v, do, vec, 0.125, "fp32 causal")


def test_bwd_stored_ds_path_is_taken(gpu_lib):
    """With the stored-dS workspace the plan selects the stored-dS dQ kernel;
    one byte short, and with the minimum workspace, the recompute one. The
    library reports its choice (fm_bwd_dq_path); both paths give the oracle's
    gradients."""
    n, H, d = 1024, 2, 128
    vec = tuple(x[None, None] for x in SM.causal(n))
    q, k, v, do = ST.qkv(1, n, n, H, d, seed=31, with_do=True)
    qc, kc, vc, dc = (t.cuda() for t in (q, k, v, do))
    m = dev_mask(vec)
    o, lse = gpu_lib.fm_attn_fwd(qc, kc, vc, m, 0.088)
    full = gpu_lib.fm_bwd_workspace_size_ds(qc, kc, vc, m, 0.088)
    minimum = gpu_lib.fm_workspace_size(qc, kc, vc, m, True, 0.088)
    rq, _, _ = OA.backward(np64(q), np64(k), np64(v), np64(do), vec, 0.088)
    for nbytes, expect in ((full, True), (full - 1, False), (minimum, False)):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dq, _, _ = gpu_lib.fm_attn_bwd(qc, kc, vc, o, lse, dc, m, 0.088, workspace=ws)
        used = gpu_lib.fm_bwd_dq_path(qc, kc, vc, m, ws, 0.088)
        log(f"workspace {nbytes} bytes (stored-dS size {full}): dQ from stored dS = {used}")
        assert used == expect
        assert_close(np64(dq.cpu()), rq, f"dQ, workspace {nbytes} bytes")


def test_bwd_stored_ds_short_workspace_falls_back(gpu_lib):
    """One byte short of the stored-dS size: the plan keeps the recompute path,
    bit for bit the result of the minimum workspace."""
    rng = np.random.default_rng(23)
    n = 600
    vec = tuple(x[None, None] for x in SM.document_causal(SM.uniform_doc_lengths(rng, n, 40, 300)))
    q, k, v, do = ST.qkv(1, n, n, 2, 128, seed=9, with_do=True)
    dq, dq0 = _compare_ds(gpu_lib, q, k, v, do, vec, 0.088, "short workspace", short=1)
    assert torch.equal(dq, dq0)
