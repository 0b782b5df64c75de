"""The allocation-free forward (fm_attn_fwd_noalloc) against fm_attn_fwd,
through the C ABI: two calls in a row on one GPU, the second with a smaller
input, so the second reuses scratch the first left behind. Results must
equal fm_attn_fwd's bit for bit when both cut the key-tile lists into the
same parts (the same kernels run on the same inputs), and meet the float bar
against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_close, dev_mask, log, np64
from oracle import attention as OA
from synth import masks as SM
from synth import tensors as ST

pytestmark = pytest.mark.gpu


def _both(fm, q, k, v, vec, scale):
    q, k, v = (t.cuda() for t in (q, k, v))
    m = dev_mask(vec)
    o_ref, lse_ref = fm.fm_attn_fwd(q, k, v, m, scale)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(lse_ref.shape, float("nan"), dtype=torch.float32, device="cuda")
    fm.fm_attn_fwd_noalloc(q, k, v, m, o, lse, scale)
    torch.cuda.synchronize()
    return (o.cpu(), lse.cpu()), (o_ref.cpu(), lse_ref.cpu())


def _check(fm, q, k, v, vec, scale, tag, oracle=True):
    log(f"noalloc {tag}: q={tuple(q.shape)} k={tuple(k.shape)} dtype={q.dtype}")
    (o, lse), (o_ref, lse_ref) = _both(fm, q, k, v, vec, scale)
    assert torch.equal(o, o_ref), f"{tag}: O differs from fm_attn_fwd"
    assert torch.equal(lse, lse_ref), f"{tag}: LSE differs from fm_attn_fwd"
    if oracle:
        ro, rl = OA.forward(np64(q), np64(k), np64(v), vec, scale)
        assert_close(np64(o), ro, f"{tag} O")
        assert_close(lse.double().numpy(), rl, f"{tag} LSE")


def test_noalloc_forward_two_calls_second_smaller(gpu_lib):
    rng = np.random.default_rng(7)
    # first call: 8192 rows, 4 heads, document-causal
    n = 8192
    vec = tuple(x[None, None] for x in SM.document_causal(SM.uniform_doc_lengths(rng, n, 64, 1024)))
    q, k, v = ST.qkv(1, n, n, 4, 128, seed=70)
    _check(gpu_lib, q, k, v, vec, 1 / math.sqrt(128), "document-causal 8192", oracle=False)
    # second call, smaller: 1000 x 700, random bounds, head_dim 64
    vec = tuple(rng.integers(-20, 1020, (1, 1, 700)).astype(np.int32) for _ in range(4))
    q, k, v = ST.qkv(1, 1000, 700, 2, 64, seed=71)
    _check(gpu_lib, q, k, v, vec, 0.125, "random 1000x700")


def test_noalloc_forward_split_lists_then_smaller(gpu_lib):
    """Few query tiles against 65,536 keys: the lists are cut into parts whose
    partials also live in the scratch; then a smaller float32 problem."""
    sq, sk = 256, 65536
    vec = tuple(x[None, None] for x in SM.no_mask(sk, sq))
    q, k, v = ST.qkv(1, sq, sk, 2, 128, seed=72)
    _check(gpu_lib, q, k, v, vec, 0.088, "256x65536 split lists")
    q, k, v = ST.qkv(1, 300, 300, 2, 64, seed=73, dtype=torch.float32)
    _check(gpu_lib, q, k, v, tuple(x[None, None] for x in SM.causal(300)), 0.125, "float32 causal 300")
