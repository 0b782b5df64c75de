"""Backward parity on long key-tile lists, element by element.

Tall, narrow problems (70,000 query rows against 256-384 keys): every key
tile of the dK/dV kernel then lists 1,094 query tiles of 64 rows, more than
one compacted list holds (1,024), so the kernel walks them in two passes.
All of dQ, dK and dV are compared with the float64 oracle
("FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr), section
"Block processing keeps the global normalization": outputs and gradients are
those of exact attention, checked with tolerances), with both dQ paths
(stored dS and recompute), no mask, causal bounds, random bounds and
per-head masks, bf16 and float32 inputs, head_dim 64 and 128.

dK and dV sum over all 70,000 rows, so at unit scale they reach |x| ~ 8.
There the absolute bar of 2e-2 is a relative one of 0.25%, about what
rounding the matrix operands to bf16 (relative 2^-9 per term, float32
inputs included) and, for bf16 outputs, half an ulp of the output (2^-6)
already cost. These cases therefore draw dO at a quarter of unit scale (an
exact power-of-two scaling): gradients stay below ~2, where the bar
measures the summation over the long lists rather than the operand format.

Also: bound vectors at the int32 limits through both backward paths, and at
the full 32K prefix-LM size the dK / dV columns of prefix keys that all
32,768 rows attend."""
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_close, dev_mask, log, np64
from oracle import attention as OA
from synth import configs as SC
from synth import tensors as ST

pytestmark = pytest.mark.gpu

SQ_LONG = 70000   # 1094 query tiles of 64 rows: two list passes per key tile


def _causal_rect(sq, sk):
    """Key j hidden from rows i < j (lower interval empty)."""
    j = np.arange(sk)
    return tuple(x.astype(np.int32)[None, None] for x in (np.full(sk, sq), np.full(sk, sq), np.zeros(sk), j))


def _random(rng, sq, sk, heads=1):
    return tuple(rng.integers(-20, sq + 20, (1, heads, sk)).astype(np.int32) for _ in range(4))


def _no_mask(sq, sk):
    return tuple(x.astype(np.int32)[None, None] for x in (np.full(sk, sq), np.full(sk, sq),
                                                         np.zeros(sk), np.zeros(sk)))


def _quarter(do):
    """dO at a quarter of its scale (exact in bf16 and float32)."""
    return (do.float() * 0.25).to(do.dtype)


def _both_paths(fm, q, k, v, do, vec, scale):
    """(dq, dk, dv) from the stored-dS workspace and from the minimum one."""
    q, k, v, do = (t.cuda() for t in (q, k, v, do))
    m = dev_mask(vec)
    o, lse = fm.fm_attn_fwd(q, k, v, m, scale)
    ws = torch.empty(fm.fm_bwd_workspace_size_ds(q, k, v, m, scale), dtype=torch.uint8, device="cuda")
    ds = fm.fm_attn_bwd(q, k, v, o, lse, do, m, scale, workspace=ws)
    used_ds = fm.fm_bwd_dq_path(q, k, v, m, ws)
    rc = fm.fm_attn_bwd(q, k, v, o, lse, do, m, scale)
    torch.cuda.synchronize()
    assert used_ds, "the stored-dS workspace did not select the stored-dS dQ path"
    return [t.cpu() for t in ds], [t.cpu() for t in rc]


def _compare(fm, q, k, v, do, vec, scale, tag):
    log(f"bwd long {tag}: q={tuple(q.shape)} k={tuple(k.shape)} dtype={q.dtype}")
    (dq, dk, dv), (dq0, dk0, dv0) = _both_paths(fm, q, k, v, do, vec, scale)
    rq, rk, rv = OA.backward(np64(q), np64(k), np64(v), np64(do), vec, scale, block=4096)
    log(f"  max |dK| {np.abs(rk).max():.3f}, max |dV| {np.abs(rv).max():.3f}")
    assert_close(np64(dk), rk, f"{tag} dK")
    assert_close(np64(dv), rv, f"{tag} dV")
    assert_close(np64(dq), rq, f"{tag} dQ (stored dS)")
    assert_close(np64(dq0), rq, f"{tag} dQ (recompute)")
    # dK and dV do not depend on the dQ path
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)


@pytest.mark.parametrize("d", [128, 64])
def test_long_lists_no_mask_and_causal(gpu_lib, d):
    scale = 1 / math.sqrt(d)
    q, k, v, do = ST.qkv(1, SQ_LONG, 256, 2, d, seed=80 + d, with_do=True)
    _compare(gpu_lib, q, k, v, _quarter(do), _no_mask(SQ_LONG, 256), scale, f"no mask d={d}")
    q, k, v, do = ST.qkv(1, SQ_LONG, 384, 2, d, seed=81 + d, with_do=True)
    _compare(gpu_lib, q, k, v, _quarter(do), _causal_rect(SQ_LONG, 384), scale, f"causal d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_long_lists_random_bounds(gpu_lib, d):
    """Random intervals make PARTIAL tiles in both passes; 320 keys leave a
    ragged last key tile."""
    rng = np.random.default_rng(90 + d)
    q, k, v, do = ST.qkv(1, SQ_LONG, 320, 2, d, seed=90 + d, with_do=True)
    _compare(gpu_lib, q, k, v, _quarter(do), _random(rng, SQ_LONG, 320), 1 / math.sqrt(d), f"random d={d}")


def test_long_lists_per_head_masks(gpu_lib):
    """Hm = H: no mask, causal and random bounds on three heads."""
    rng = np.random.default_rng(95)
    sk = 384
    parts = [_no_mask(SQ_LONG, sk), _causal_rect(SQ_LONG, sk), _random(rng, SQ_LONG, sk)]
    vec = tuple(np.concatenate([p[i] for p in parts], axis=1) for i in range(4))
    q, k, v, do = ST.qkv(1, SQ_LONG, sk, 3, 128, seed=96, with_do=True)
    _compare(gpu_lib, q, k, v, _quarter(do), vec, 0.088, "per-head masks")


@pytest.mark.parametrize("d", [128, 64])
def test_long_lists_float32(gpu_lib, d):
    rng = np.random.default_rng(97 + d)
    q, k, v, do = ST.qkv(1, SQ_LONG, 256, 1, d, seed=97 + d, dtype=torch.float32, with_do=True)
    _compare(gpu_lib, q, k, v, _quarter(do), _random(rng, SQ_LONG, 256), 1 / math.sqrt(d), f"float32 random d={d}")


def test_bwd_int32_limit_bounds(gpu_lib):
    """Bounds at INT_MIN / INT_MAX and just past the row range, on both dQ
    paths: row i is masked by [s, e) for any int32 s, e exactly when
    s <= i < e."""
    rng = np.random.default_rng(98)
    sq, sk = 700, 520
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    choices = np.array([lo, lo + 1, -1, 0, 1, sq // 2, sq - 1, sq, sq + 1, hi - 1, hi], dtype=np.int64)
    vec = tuple(rng.choice(choices, (1, 1, sk)).astype(np.int32) for _ in range(4))
    # a few keys fully open and a few hidden from every row, whatever the draw
    vec[0][0, 0, :8], vec[1][0, 0, :8] = hi, lo
    vec[2][0, 0, :8], vec[3][0, 0, :8] = 0, 0
    vec[0][0, 0, 8:16], vec[1][0, 0, 8:16] = lo, hi
    q, k, v, do = ST.qkv(1, sq, sk, 2, 128, seed=99, with_do=True)
    _compare(gpu_lib, q, k, v, do, vec, 0.088, "int32-limit bounds")


@pytest.mark.slow
def test_prefix_lm_32k_heavy_key_columns(gpu_lib):
    """Full 32K prefix-LM size with the stored-dS workspace the benchmark
    times: dK / dV of prefix keys (attended by all 32,768 rows, so their key
    tiles list all 512 query tiles) against the oracle column by column."""
    fm = gpu_lib
    w = SC.build("c3b_prefix_lm_32k", seed=0)
    q, k, v, do = (t.cuda() for t in (w.q, w.k, w.v, w.do))
    m = dev_mask(w.vectors)
    log("c3b_prefix_lm_32k: forward and backward (stored dS)")
    o, lse = fm.fm_attn_fwd(q, k, v, m, w.scale)
    ws = torch.empty(fm.fm_bwd_workspace_size_ds(q, k, v, m, w.scale), dtype=torch.uint8, device="cuda")
    _, dk, dv = fm.fm_attn_bwd(q, k, v, o, lse, do, m, w.scale, workspace=ws)
    torch.cuda.synchronize()
    assert fm.fm_bwd_dq_path(q, k, v, m, ws)
    dk, dv = dk.cpu(), dv.cpu()
    del ws, o, lse, q, k, v, do
    torch.cuda.empty_cache()
    cols = np.array([0, 1, 127, 128, 4095, 8190, 8191])
    h = 5
    log(f"  oracle columns {cols.tolist()} of head {h} (every row attends them)")
    rk, rv = OA.backward_cols(np64(w.q), np64(w.k), np64(w.v), np64(w.do), w.vectors, w.scale, 0, h, cols,
                              block=1024)
    assert_close(np64(dk)[0, cols, h], rk, "prefix keys dK")
    assert_close(np64(dv)[0, cols, h], rv, "prefix keys dV")
