"""Grouped-query attention parity: query heads in groups sharing one K/V head
(H_kv < H), forward O / LSE and backward dQ / dK / dV from the HIP kernels
(both dQ paths) against the float64 oracle, with shared and per-head masks,
strided and contiguous K/V, head_dim 64 and 128, float32 inputs."""
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
    return [SM.causal(n), SM.document_causal(SM.uniform_doc_lengths(rng, n, 40, 300)),
            SM.sliding_window_causal(n, 150), SM.prefix_lm(n, n // 4),
            SM.share_question(n // 6, SM.answer_lengths(rng, n - n // 6, 5)), SM.no_mask(n, n)]


def _inputs(B, n, H, hkv, d, seed, contiguous=True, dtype=torch.bfloat16):
    q, k, v, do = ST.qkv(B, n, n, H, d, seed=seed, dtype=dtype, with_do=True)
    k, v = k[:, :, :hkv], v[:, :, :hkv]     # head-axis slices: strided K/V
    if contiguous:
        k, v = k.contiguous(), v.contiguous()
    return q, k, v, do


def _check(fm, q, k, v, do, vec, scale, tag):
    log(f"gqa {tag} q={tuple(q.shape)} k={tuple(k.shape)} stride_k={k.stride()} dtype={q.dtype}")
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    m = dev_mask(vec)
    o, lse = fm.fm_attn_fwd(qc, kc, vc, m, scale)
    dq0, dk0, dv0 = fm.fm_attn_bwd(qc, kc, vc, o, lse, doc, m, scale)          # recompute dQ
    nbytes = fm.fm_bwd_workspace_size_ds(qc, kc, vc, m, scale)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = fm.fm_attn_bwd(qc, kc, vc, o, lse, doc, m, scale, workspace=ws)  # stored dS
    torch.cuda.synchronize()
    ro, rl = OA.forward(np64(q), np64(k), np64(v), vec, scale)
    rq, rk, rv = OA.backward(np64(q), np64(k), np64(v), np64(do), vec, scale)
    assert_close(np64(o.cpu()), ro, f"{tag} O")
    assert_close(lse.cpu().double().numpy(), rl, f"{tag} LSE")
    for got, ref, nm in ((dq, rq, "dQ"), (dq0, rq, "dQ recompute")):
        assert_close(np64(got.cpu()), ref, f"{tag} {nm}")
    # dK and dV of a shared K/V head sum the group's query heads, so they grow
    # with the group; for a bf16 output the bar adds the output's own rounding
    # (|ref| 2^-8), which a float32 output does not have
    rnd = BF16_ROUND if dk.dtype == torch.bfloat16 else 0.0
    for got, ref, nm in ((dk, rk, "dK"), (dv, rv, "dV")):
        log(f"  {nm}: max |ref| = {np.max(np.abs(ref)):.3f}")
        assert_close(np64(got.cpu()), ref, f"{tag} {nm}", out_round=rnd)
    assert torch.equal(dk.cpu(), dk0.cpu()) and torch.equal(dv.cpu(), dv0.cpu())


@pytest.mark.parametrize("hkv", [2, 1])
def test_gqa_shared_mask_families(gpu_lib, hkv):
    rng = np.random.default_rng(40 + hkv)
    n, H, d = 520, 4, 128
    for i, fam in enumerate(_families(n, rng)):
        q, k, v, do = _inputs(1, n, H, hkv, d, seed=50 + i, contiguous=(i % 2 == 0))
        _check(gpu_lib, q, k, v, do, tuple(x[None, None] for x in fam), 1 / math.sqrt(d), f"family {i} hkv={hkv}")


@pytest.mark.parametrize("hkv", [3, 1])
def test_gqa_per_batch_and_head_masks(gpu_lib, hkv):
    """Bm = B and Hm = H: the query heads of one K/V head have different
    masks (and so different tile lists in the dK/dV kernel)."""
    rng = np.random.default_rng(60 + hkv)
    n, B, H, d = 400, 2, 6, 128
    fams = _families(n, rng)
    vec = SM.stack([[fams[(b * H + h) % 6] for h in range(H)] for b in range(B)])
    q, k, v, do = _inputs(B, n, H, hkv, d, seed=61)
    _check(gpu_lib, q, k, v, do, vec, 0.09, f"per-(b,h) masks hkv={hkv}")


def test_gqa_head_dim_64_and_float32(gpu_lib):
    rng = np.random.default_rng(70)
    n = 300
    fam = tuple(x[None, None] for x in SM.document_causal(SM.uniform_doc_lengths(rng, n, 30, 120)))
    q, k, v, do = _inputs(2, n, 4, 2, 64, seed=71)
    _check(gpu_lib, q, k, v, do, fam, 0.125, "d=64")
    # float32 inputs are rounded to bf16 for the products; a pair of query
    # heads on one K/V head at the tiny causal workload's size keeps dK within
    # the same bar
    q, k, v, do = _inputs(1, 256, 2, 1, 64, seed=72, dtype=torch.float32)
    _check(gpu_lib, q, k, v, do, tuple(x[None, None] for x in SM.causal(256)), 0.125, "float32")


def _dead_keys(n, lo, hi, base):
    """`base` bounds with keys [lo, hi) masked for every row."""
    lts, lte, uts, ute = (np.array(x) for x in base)
    lts[lo:hi], lte[lo:hi] = 0, n
    return lts, lte, uts, ute


@pytest.mark.parametrize("case", ["shared", "per_head", "float32"])
def test_gqa_key_tiles_masked_for_every_row(gpu_lib, case):
    """Keys [128, 384) are masked for every row of every query head: their two
    key tiles have no non-SKIP tile in any head of the group, so the dK/dV
    workgroups write zeros without walking a list. Shared mask (float32
    partials per query head, summed afterwards), per-head masks (the group
    walked in one workgroup) and float32 inputs and outputs (one K/V head per
    query head)."""
    n, d = 520, 128
    rng = np.random.default_rng(75)
    if case == "per_head":
        H, hkv = 4, 2
        fams = [SM.causal(n), SM.document_causal(SM.uniform_doc_lengths(rng, n, 40, 300)),
                SM.prefix_lm(n, n // 4), SM.sliding_window_causal(n, 150)]
        vec = SM.stack([[_dead_keys(n, 128, 384, fams[h]) for h in range(H)]])
    else:
        H, hkv = (4, 2) if case == "shared" else (2, 2)
        vec = tuple(x[None, None] for x in _dead_keys(n, 128, 384, SM.causal(n)))
    dtype = torch.float32 if case == "float32" else torch.bfloat16
    q, k, v, do = _inputs(1, n, H, hkv, d, seed=76, dtype=dtype)
    _check(gpu_lib, q, k, v, do, vec, 1 / math.sqrt(d), f"dead key tiles, {case}")
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    m = dev_mask(vec)
    o, lse = gpu_lib.fm_attn_fwd(qc, kc, vc, m, 1 / math.sqrt(d))
    _, dk, dv = gpu_lib.fm_attn_bwd(qc, kc, vc, o, lse, doc, m, 1 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.all(dk[:, 128:384] == 0) and torch.all(dv[:, 128:384] == 0)
    assert torch.any(dk[:, :128] != 0) and torch.any(dv[:, 384:] != 0)


def test_gqa_rejects_non_dividing_heads(gpu_lib):
    q, k, v = ST.qkv(1, 64, 64, 4, 128, seed=1)
    k, v = k[:, :, :3].contiguous(), v[:, :, :3].contiguous()
    with pytest.raises(ValueError):
        gpu_lib.fm_attn_fwd(q.cuda(), k.cuda(), v.cuda(), dev_mask(tuple(x[None, None] for x in SM.causal(64))), 0.1)
