"""Forward parity: HIP kernels (through the C ABI) vs the float64 oracle,
element by element, at sizes spanning several tiles with ragged tails, plus
the edge cases (fully masked rows, one row / one key, Sq != Sk, strided
layouts, head_dim 64, float32 inputs) and determinism."""
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_close, dev_mask, log, np64
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


def _run_fwd(fm, q, k, v, vec, scale):
    o, lse = fm.fm_attn_fwd(q.cuda(), k.cuda(), v.cuda(), dev_mask(vec), scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _compare_fwd(fm, q, k, v, vec, scale, tag):
    log(f"fwd {tag} q={tuple(q.shape)} k={tuple(k.shape)} dtype={q.dtype}")
    o, lse = _run_fwd(fm, q, k, v, vec, scale)
    ro, rl = OA.forward(np64(q), np64(k), np64(v), vec, scale)
    assert_close(np64(o), ro, f"{tag} O")
    assert_close(lse.double().numpy(), rl, f"{tag} LSE")
    return o, lse


@pytest.mark.parametrize("d", [128, 64])
def test_fwd_mask_families(gpu_lib, d):
    rng = np.random.default_rng(d)
    n = 700
    for name, v in _families(n, rng).items():
        q, k, vv = ST.qkv(2, n, n, 3, d, seed=d + len(name))
        _compare_fwd(gpu_lib, q, k, vv, tuple(x[None, None] for x in v), 1 / math.sqrt(d), f"{name} d={d}")


def test_fwd_per_batch_and_head_masks(gpu_lib):
    rng = np.random.default_rng(1)
    n, B, H, d = 520, 2, 3, 128
    per = [[list(_families(n, rng).values())[(b * H + h) % 6] for h in range(H)] for b in range(B)]
    vec = SM.stack(per)
    q, k, v = ST.qkv(B, n, n, H, d, seed=5)
    _compare_fwd(gpu_lib, q, k, v, vec, 0.09, "per-(b,h) masks")


def test_fwd_random_vectors_rectangular(gpu_lib):
    """Random (non-canonical, out-of-range, overlapping) bounds with Sq != Sk;
    includes fully masked rows (O = 0, LSE = -inf)."""
    rng = np.random.default_rng(2)
    for sq, sk in ((300, 900), (900, 300), (129, 65)):
        vec = tuple(rng.integers(-20, sq + 20, (1, 1, sk)).astype(np.int32) for _ in range(4))
        q, k, v = ST.qkv(1, sq, sk, 2, 128, seed=sq)
        o, lse = _compare_fwd(gpu_lib, q, k, v, vec, 0.1, f"random {sq}x{sk}")
        allowed = ~OA.dense_mask(*[x[0, 0].astype(np.int64) for x in vec], np.arange(sq), sk)
        empty = ~allowed.any(axis=1)
        if empty.any():
            assert torch.all(o[:, torch.from_numpy(empty)] == 0)
            assert torch.all(lse[:, :, torch.from_numpy(empty)] == -math.inf)


def test_fwd_split_lists(gpu_lib):
    """Few workgroups and long key lists (256 rows x 65536 keys, 2 heads):
    each query tile's key-tile list is cut into parts merged afterwards (8
    here). Masks: none; random bounds; rows 100..159 masked for every key
    (O = 0, LSE = -inf); only keys 0..319 open (five key tiles, so some parts
    are empty); head_dim 64 and 128, bf16 and float32."""
    rng = np.random.default_rng(5)
    sq, sk = 256, 65536
    j = np.arange(sk)
    i32 = lambda *xs: tuple(np.asarray(x, dtype=np.int32)[None, None] for x in xs)
    masks = {
        "none": i32(np.full(sk, sq), np.full(sk, sq), np.zeros(sk), np.zeros(sk)),
        "random": i32(*(rng.integers(-20, sq + 20, sk) for _ in range(4))),
        "dead rows": i32(np.full(sk, 100), np.full(sk, 160), rng.integers(0, sq, sk), rng.integers(0, sq, sk)),
        "few keys": i32(np.where(j >= 320, 0, sq), np.full(sk, sq), np.zeros(sk), np.zeros(sk)),
    }
    for d, dtype in ((128, torch.bfloat16), (64, torch.bfloat16), (64, torch.float32), (128, torch.float32)):
        for t, (name, vec) in enumerate(masks.items()):
            q, k, v = ST.qkv(1, sq, sk, 2, d, seed=80 + t, dtype=dtype)
            o, lse = _compare_fwd(gpu_lib, q, k, v, vec, 1 / math.sqrt(d), f"split {name} d={d} {dtype}")
            if name == "dead rows":
                assert torch.all(o[:, 100:160] == 0) and torch.all(lse[:, :, 100:160] == -math.inf)


@pytest.mark.parametrize("parts,sq,heads,sk", [(3, 1280, 40, 12288), (5, 1280, 30, 20480),
                                                (6, 1024, 32, 24576), (7, 1280, 20, 28672)])
def test_fwd_split_part_counts(gpu_lib, parts, sq, heads, sk):
    """Part counts that are not powers of two. The library cuts each list
    into min(8, 1536 // workgroups) parts (at most one per 64 key tiles), so
    these shapes take 3, 5, 6 and 7 parts (each count is a merge kernel of its
    own). Random bounds give PARTIAL tiles and uneven parts. Eight rows of
    every query tile of every head against the oracle, O and LSE."""
    nwg = -(-sq // 128) * heads
    assert min(8, 1536 // nwg, -(-sk // 64) // 64) == parts
    rng = np.random.default_rng(100 + parts)
    vec = tuple(rng.integers(-20, sq + 20, (1, 1, sk)).astype(np.int32) for _ in range(4))
    q, k, v = ST.qkv(1, sq, sk, heads, 64, seed=110 + parts)
    log(f"fwd {parts} parts: q={tuple(q.shape)} k={tuple(k.shape)}")
    o, lse = _run_fwd(gpu_lib, q, k, v, vec, 0.125)
    rows = np.concatenate([t + np.array([0, 1, 31, 64, 95, 100, 126, 127]) for t in range(0, sq, 128)])
    qn, kn, vn = np64(q), np64(k), np64(v)
    for h in range(heads):
        ro, rl = OA.forward_rows(qn, kn, vn, vec, 0.125, 0, h, rows)
        assert_close(np64(o)[0, rows, h], ro, f"{parts} parts head {h} O")
        assert_close(lse[0, h, rows].double().numpy(), rl, f"{parts} parts head {h} LSE")


def test_fwd_split_lists_ragged_rows_repeated(gpu_lib):
    """Split lists with a ragged last query tile (200 rows: tiles of 128 and
    72 rows), called twice on one workspace: nothing from the first call's
    partials leaks into the second, and both calls give the same bits."""
    rng = np.random.default_rng(6)
    sq, sk = 200, 65536
    vec = tuple(rng.integers(-20, sq + 20, (1, 1, sk)).astype(np.int32) for _ in range(4))
    q, k, v = ST.qkv(1, sq, sk, 3, 128, seed=86)
    o, lse = _compare_fwd(gpu_lib, q, k, v, vec, 0.088, "split ragged rows")
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    m = dev_mask(vec)
    ws = torch.empty(gpu_lib.fm_workspace_size(qd, kd, vd, m, False), dtype=torch.uint8, device="cuda")
    outs = [gpu_lib.fm_attn_fwd(qd, kd, vd, m, 0.088, workspace=ws) for _ in range(2)]
    torch.cuda.synchronize()
    for o2, l2 in outs:
        assert torch.equal(o2.cpu(), o) and torch.equal(l2.cpu(), lse)


def test_fwd_fully_masked_rows_and_tiles(gpu_lib):
    """Rows 100..299 see no key at all: whole query tiles are SKIP everywhere."""
    n = 600
    j = np.arange(n)
    lts = np.full(n, 100)
    lte = np.full(n, 300)
    uts = np.zeros(n, np.int64)
    ute = j
    vec = tuple(np.asarray(x, np.int32)[None, None] for x in (lts, lte, uts, ute))
    q, k, v = ST.qkv(1, n, n, 2, 128, seed=9)
    o, lse = _compare_fwd(gpu_lib, q, k, v, vec, 0.1, "masked rows 100..299")
    assert torch.all(o[:, 100:300] == 0) and torch.all(lse[:, :, 100:300] == -math.inf)


@pytest.mark.parametrize("sq,sk", [(1, 1), (1, 1000), (1000, 1), (64, 64), (128, 64), (127, 65)])
def test_fwd_tiny_and_edge_shapes(gpu_lib, sq, sk):
    rng = np.random.default_rng(sq * 7 + sk)
    vec = tuple(rng.integers(-2, sq + 2, (1, 1, sk)).astype(np.int32) for _ in range(2)) + \
        (np.zeros((1, 1, sk), np.int32), np.zeros((1, 1, sk), np.int32))
    q, k, v = ST.qkv(1, sq, sk, 1, 64, seed=sq + sk)
    _compare_fwd(gpu_lib, q, k, v, vec, 0.125, f"edge {sq}x{sk}")


def test_fwd_q_zero_closed_form(gpu_lib):
    """Q = 0: O_i is the mean of the open V rows and LSE_i = ln(open count)."""
    n = 333
    vec = tuple(x[None, None] for x in SM.sliding_window_causal(n, 50))
    _, k, v = ST.qkv(1, n, n, 1, 128, seed=4)
    q = torch.zeros((1, n, 1, 128), dtype=torch.bfloat16)
    o, lse = _run_fwd(gpu_lib, q, k, v, vec, 0.3)
    allowed = ~OA.dense_mask(*[x[0, 0].astype(np.int64) for x in vec], np.arange(n))
    cnt = allowed.sum(axis=1)
    assert_close(lse[0, 0].double().numpy(), np.log(cnt), "q=0 LSE")
    vd = np64(v)[0, :, 0]
    mean = (allowed.astype(np.float64) @ vd) / cnt[:, None]
    assert_close(np64(o)[0, :, 0], mean, "q=0 O")


def test_fwd_strided_layout(gpu_lib):
    """[B, H, S, D] storage viewed as [B, S, H, D] (non-contiguous strides)."""
    n, B, H, d = 400, 2, 2, 128
    g = torch.Generator().manual_seed(3)
    qh = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    kh = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    vh = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    q, k, v = (t.cuda().transpose(1, 2) for t in (qh, kh, vh))
    vec = tuple(x[None, None] for x in SM.causal(n))
    o, lse = gpu_lib.fm_attn_fwd(q, k, v, dev_mask(vec), 0.08)
    torch.cuda.synchronize()
    ro, rl = OA.forward(np64(q), np64(k), np64(v), vec, 0.08)
    assert_close(np64(o), ro, "strided O")
    assert_close(lse.cpu().double().numpy(), rl, "strided LSE")


def test_fwd_float32_inputs(gpu_lib):
    """Float32 inputs (rounded to bf16 for the products, fp32 softmax state and
    outputs): the tiny causal workload at its full size."""
    from synth import configs as SC
    w = SC.build("c1_tiny_causal", 0)
    _compare_fwd(gpu_lib, w.q, w.k, w.v, w.vectors, w.scale, "c1 fp32")


def test_fwd_key_permutation(gpu_lib):
    """Permuting K, V and the four vectors by one permutation changes nothing
    beyond rounding (exercises PARTIAL tiles everywhere)."""
    n = 500
    rng = np.random.default_rng(8)
    vec = tuple(x[None, None] for x in SM.document_causal(SM.uniform_doc_lengths(rng, n, 30, 120)))
    q, k, v = ST.qkv(1, n, n, 2, 128, seed=8)
    perm = rng.permutation(n)
    pv = tuple(x[..., perm] for x in vec)
    o1, l1 = _run_fwd(gpu_lib, q, k, v, vec, 0.1)
    tp = torch.from_numpy(perm)
    o2, l2 = _run_fwd(gpu_lib, q, k[:, tp].contiguous(), v[:, tp].contiguous(), pv, 0.1)
    ro, rl = OA.forward(np64(q), np64(k), np64(v), vec, 0.1)
    assert_close(np64(o2), ro, "permuted O")
    assert_close(l2.double().numpy(), rl, "permuted LSE")
    assert_close(np64(o1), np64(o2), "O vs permuted O")


def test_fwd_deterministic(gpu_lib):
    n = 1000
    vec = tuple(x[None, None] for x in SM.causal(n))
    q, k, v = (t.cuda() for t in ST.qkv(2, n, n, 4, 128, seed=1))
    m = dev_mask(vec)
    o1, l1 = gpu_lib.fm_attn_fwd(q, k, v, m, 0.1)
    o2, l2 = gpu_lib.fm_attn_fwd(q, k, v, m, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("slope", [4.0, 40.0])
def test_fwd_growing_scores(gpu_lib, slope):
    """Scores that grow along the key axis (and a few late spikes), so the
    running maximum moves in many tiles and in both halves of a tile: the
    reference moves and rescales of O and l, checked against the oracle."""
    n, d = 700, 128
    g = torch.Generator().manual_seed(int(slope))
    ramp = torch.linspace(0.0, slope, n)
    q = (torch.ones(1, n, 2, d) + 0.3 * torch.randn(1, n, 2, d, generator=g)).to(torch.bfloat16)
    k = (ramp[None, :, None, None] / math.sqrt(d) + 0.3 * torch.randn(1, n, 2, d, generator=g))
    k[:, [333, 517, 690]] += 3.0 * slope / math.sqrt(d)
    k = k.to(torch.bfloat16)
    v = torch.randn(1, n, 2, d, generator=g).to(torch.bfloat16)
    for name, vec in (("none", SM.no_mask(n, n)), ("causal", SM.causal(n))):
        _compare_fwd(gpu_lib, q, k, v, tuple(x[None, None] for x in vec), 1 / math.sqrt(d), f"growing {name} s={slope}")
