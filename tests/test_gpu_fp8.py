"""FP8 forward parity: the E4M3 kernel (through the C ABI) vs the float64
oracle on the dequantized operands.

Tolerance, derived from the arithmetic. Products of two E4M3 values are exact
in fp32 and the fp32 sums of 128 of them carry no error that matters here, so
scores, softmax state and LSE are fp32-accurate: LSE meets the float bar
(max-abs 2e-2, relative L2 1e-2). O differs from the exact value because the
probabilities are rounded to E4M3 (round to nearest even) before the second
product, while the row sum adds them unrounded. For row i, with p_j the
probabilities relative to the kernel's reference (between the row maximum and
2^8 times it) and l their sum, a normal E4M3 value is within 2^-4 of p_j
relatively and a subnormal one (below 2^-6) within 2^-10 absolutely, so

  |O_ic - O*_ic| <= vmax_i * (2^-4 + 2^-10 * n_i / l*_i) + 2^-8 |O*_ic|

where O* is exact, vmax_i the largest |V| entry over the row's open keys, l*_i
the sum of exp(s_ij - max_j s_ij) over them and n_i the number of open keys
with exp(s_ij - max s) < 2^-6 (a superset of those the kernel holds as
subnormals, its reference being at least the row maximum less 8 in log2
units); the last term is the bf16 rounding of the output. That bound is
checked on every element. The rounding errors are unbiased and largely cancel
over a row, so the relative L2 error is also checked, against 2^-4 (about
2^-4 / sqrt(3) is the expectation when attention is spread evenly over many
keys and O is itself an average)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_close, dev_mask, log, np64
from oracle import attention as OA
from oracle import fp8 as OF
from synth import masks as SM
from synth import tensors as ST

pytestmark = pytest.mark.gpu

D = 128


def _codes(B, Sq, Sk, H, Hkv, seed, gains=(64.0, 64.0, 64.0), d=D):
    q8 = ST.fp8_codes("q", (B, Sq, H, d), seed, gains[0])
    k8 = ST.fp8_codes("k", (B, Sk, Hkv, d), seed, gains[1])
    v8 = ST.fp8_codes("v", (B, Sk, Hkv, d), seed, gains[2])
    return q8, k8, v8, tuple(1.0 / g for g in gains)


def _row_bounds(q8, k8, v8, ds, vectors, scale):
    """The per-row bound above (vmax_i * (2^-4 + 2^-10 n_i / l*_i)), [B, Sq, H]."""
    qd, kd, vd = (OF.dequantize(x, d) for x, d in zip((q8, k8, v8), ds))
    B, Sq, H, _ = qd.shape
    Sk, Hkv = kd.shape[1], kd.shape[2]
    bound = np.zeros((B, Sq, H))
    for b in range(B):
        for h in range(H):
            hk = OA.kv_head(H, Hkv, h)
            masked = OA.dense_mask(*OA.vectors_for(vectors, b, h), np.arange(Sq), Sk)
            s = scale * (qd[b, :, h] @ kd[b, :, hk].T)
            s[masked] = -np.inf
            ok = ~masked.all(axis=1)
            mx = np.where(ok, s.max(axis=1), 0.0)
            p = np.exp(s - mx[:, None])
            l = np.where(ok, p.sum(axis=1), 1.0)
            n_small = ((p < 2.0 ** -6) & ~masked).sum(axis=1)
            vrow = np.abs(vd[b, :, hk]).max(axis=1)
            vmax = np.where(~masked, vrow[None, :], 0.0).max(axis=1)
            bound[b, :, h] = np.where(ok, vmax * (2.0 ** -4 + 2.0 ** -10 * n_small / l), 0.0)
    return bound


def _check_o(o, ref, bound, tag):
    """Every element within the derived bound; relative L2 within 2^-4."""
    o = np.asarray(o, dtype=np.float64)
    assert np.isfinite(o).all(), f"{tag}: non-finite output"
    err = np.abs(o - ref)
    lim = bound[..., None] + 2.0 ** -8 * np.abs(ref) + 1e-6
    worst = float(np.max(err - lim))
    rel = float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-30))
    log(f"  {tag} O: max_abs={err.max():.3e} rel_l2={rel:.3e} max(err/bound)={float(np.max(err / lim)):.3f}")
    assert worst <= 0, f"{tag}: O beyond the FP8 bound by {worst:.3e}"
    assert rel <= 2.0 ** -4, f"{tag}: O relative L2 {rel:.3e} > 2^-4"


def _compare(fm, q8, k8, v8, ds, vec, scale, tag):
    log(f"fp8 fwd {tag} q={tuple(q8.shape)} k={tuple(k8.shape)} descale={ds}")
    o, lse = fm.fm_attn_fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), ds, dev_mask(vec), scale)
    torch.cuda.synchronize()
    o, lse = np64(o), lse.double().cpu().numpy()
    qn, kn, vn = q8.numpy(), k8.numpy(), v8.numpy()
    ro, rl = OF.forward(qn, kn, vn, ds, vec, scale)
    _check_o(o, ro, _row_bounds(qn, kn, vn, ds, vec, scale), tag)
    assert_close(lse, rl, f"{tag} LSE")
    return o, lse


def _families(n, rng):
    return {
        "causal": SM.causal(n),
        "document": SM.document_causal(SM.uniform_doc_lengths(rng, n, 40, 300)),
        "window": SM.sliding_window_causal(n, 150),
        "prefix_lm": SM.prefix_lm(n, n // 4),
        "share_question": SM.share_question(n // 6, SM.answer_lengths(rng, n - n // 6, 5)),
        "none": SM.no_mask(n, n),
    }


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_mask_families(gpu_lib, d):
    rng = np.random.default_rng(8)
    n = 700
    for i, (name, v) in enumerate(_families(n, rng).items()):
        q8, k8, v8, ds = _codes(2, n, n, 3, 3, seed=40 + i, d=d)
        _compare(gpu_lib, q8, k8, v8, ds, tuple(x[None, None] for x in v), 1 / math.sqrt(d), f"{name} d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_ragged_gqa_per_head_masks(gpu_lib, d):
    """Sq != Sk, both ragged; 4 query heads on 2 K/V heads; a mask per
    (b, h) with fully masked rows."""
    rng = np.random.default_rng(9)
    B, H, Hkv, sq, sk = 2, 4, 2, 300, 333
    fams = []
    for _ in range(B * H):
        lts = rng.integers(0, sq, sk)
        lte = np.minimum(sq, lts + rng.integers(0, sq, sk))
        uts = rng.integers(0, sq, sk)
        ute = np.minimum(sq, uts + rng.integers(0, sq // 3, sk))
        fams.append((lts, lte, uts, ute))
    fams[3] = (np.zeros(sk, int), np.full(sk, 100), np.zeros(sk, int), np.zeros(sk, int))   # rows < 100 see nothing
    vec = SM.stack([[fams[b * H + h] for h in range(H)] for b in range(B)])
    q8, k8, v8, ds = _codes(B, sq, sk, H, Hkv, seed=50, d=d)
    o, lse = _compare(gpu_lib, q8, k8, v8, ds, vec, 0.1, f"ragged gqa d={d}")
    assert (o[0, :100, 3] == 0).all() and np.isneginf(lse[0, 3, :100]).all()


@pytest.mark.parametrize("gains,scale", [((16.0, 32.0, 8.0), 0.5), ((64.0, 4.0, 64.0), 1.0)])
def test_fp8_descales_and_wide_scores(gpu_lib, gains, scale):
    """Different descale per tensor, and scores wide enough (scale up to 1)
    that the reference moves often (the rare rescale branch)."""
    rng = np.random.default_rng(10)
    n = 520
    vec = tuple(x[None, None] for x in SM.document_causal(SM.uniform_doc_lengths(rng, n, 60, 400)))
    q8, k8, v8, ds = _codes(1, n, n, 2, 1, seed=60, gains=gains)
    _compare(gpu_lib, q8, k8, v8, ds, vec, scale, f"gains {gains} scale {scale}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("sq,sk", [(1, 1), (1, 200), (130, 1), (64, 64), (129, 65)])
def test_fp8_tiny_and_edge_shapes(gpu_lib, sq, sk, d):
    q8, k8, v8, ds = _codes(1, sq, sk, 2, 2, seed=sq * 1000 + sk, d=d)
    vec = tuple(x[None, None] for x in SM.no_mask(sk, sq))
    _compare(gpu_lib, q8, k8, v8, ds, vec, 1 / math.sqrt(d), f"{sq}x{sk} d={d}")


def test_fp8_float8_tensors_and_determinism(gpu_lib):
    """torch.float8_e4m3fn tensors go in as their codes; two runs agree bit
    for bit."""
    n = 400
    q8, k8, v8, ds = _codes(1, n, n, 2, 2, seed=70)
    vec = tuple(x[None, None] for x in SM.causal(n))
    mask = dev_mask(vec)
    f8 = [t.cuda().view(torch.float8_e4m3fn) for t in (q8, k8, v8)]
    o1, l1 = gpu_lib.fm_attn_fwd_fp8(*f8, ds, mask)
    o2, l2 = gpu_lib.fm_attn_fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), ds, mask)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_prefix_lm_32k_sampled(gpu_lib):
    """The 32k prefix-LM workload shape (B1 H8 S32768, bidirectional prefix
    8192) on FP8 codes with 2 K/V heads, checked on sampled rows: each output
    row depends only on its own query row."""
    from synth import configs as SC
    w = SC.build("c3b_prefix_lm_32k", seed=0, tensors=False)
    B, H, Hkv, n = 1, 8, 2, w.seq_q
    q8, k8, v8, ds = _codes(B, n, n, H, Hkv, seed=80)
    log(f"fp8 fwd prefix-LM 32k: running")
    o, lse = gpu_lib.fm_attn_fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), ds, dev_mask(w.vectors), w.scale)
    torch.cuda.synchronize()
    o, lse = np64(o), lse.double().cpu().numpy()
    rng = np.random.default_rng(2)
    rows = np.concatenate([rng.choice(n, 48, replace=False), [0, 1, 8191, 8192, n - 1]])
    qn, kn, vn = q8.numpy(), k8.numpy(), v8.numpy()
    qd, kd, vd = (OF.dequantize(x, d) for x, d in zip((qn, kn, vn), ds))
    for h in (0, 5):
        ro, rl = OF.forward_rows(qn, kn, vn, ds, w.vectors, w.scale, 0, h, rows)
        hk = OA.kv_head(H, Hkv, h)
        masked = OA.dense_mask(*OA.vectors_for(w.vectors, 0, h), rows, n)
        s = w.scale * (qd[0, rows, h] @ kd[0, :, hk].T)
        s[masked] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        n_small = ((p < 2.0 ** -6) & ~masked).sum(axis=1)
        vmax = np.where(~masked, np.abs(vd[0, :, hk]).max(axis=1)[None, :], 0.0).max(axis=1)
        bound = vmax * (2.0 ** -4 + 2.0 ** -10 * n_small / p.sum(axis=1))
        _check_o(o[0, rows, h], ro, bound, f"prefix-LM 32k h{h}")
        assert_close(lse[0, h, rows], rl, f"prefix-LM 32k h{h} LSE")


@pytest.mark.parametrize("name", ["c4_doc_causal_128k", "c4_causal_128k"])
def test_fp8_128k_sampled(gpu_lib, name):
    """The FP8 forward in the configuration the benchmark times (the 128K
    workloads' shape and mask, E4M3 codes with descales 1/64), checked on
    sampled rows of two heads against the oracle, each within its row's
    bound, and LSE within the float bar."""
    from synth import configs as SC
    w = SC.build(name, seed=0, tensors=False)
    n, H = w.seq_q, w.heads
    q8, k8, v8, ds = _codes(w.batch, n, n, H, H, seed=0)
    log(f"fp8 fwd {name}: running")
    o, lse = gpu_lib.fm_attn_fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), ds, dev_mask(w.vectors), w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.concatenate([rng.choice(n, 24, replace=False), [0, 1, n // 2, n - 1]])
    qn, kn, vn = q8.numpy(), k8.numpy(), v8.numpy()
    kd, vd = OF.dequantize(kn, ds[1]), OF.dequantize(vn, ds[2])
    qd = OF.dequantize(qn[:, rows], ds[0])
    o = np64(o[:, rows])
    lse = lse[:, :, rows].double().cpu().numpy()
    for h in (0, H - 1):
        ro, rl = OF.forward_rows(qn, kn, vn, ds, w.vectors, w.scale, 0, h, rows)
        masked = OA.dense_mask(*OA.vectors_for(w.vectors, 0, h), rows, n)
        s = w.scale * (qd[0, :, h] @ kd[0, :, h].T)
        s[masked] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        n_small = ((p < 2.0 ** -6) & ~masked).sum(axis=1)
        vmax = np.where(~masked, np.abs(vd[0, :, h]).max(axis=1)[None, :], 0.0).max(axis=1)
        bound = vmax * (2.0 ** -4 + 2.0 ** -10 * n_small / p.sum(axis=1))
        _check_o(o[0, :, h], ro, bound, f"{name} h{h}")
        assert_close(lse[0, h], rl, f"{name} h{h} LSE")
