"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the pages, a closed form, a library routine or a brute-force evaluation. They
are run as ordinary tests (test_oracle_pins.py) and again against oracles with
planted mistakes (test_oracle_mutations.py), where at least one must fail.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import masks as OM
from synth import masks as SM

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol=1e-9, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol * max(1.0, np.max(np.abs(b[fin]))), f"{what}: max err {err}"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"


def _vec3(v):
    """[Sk] vectors -> [1, 1, Sk] tuple."""
    return tuple(None if x is None else np.asarray(x)[None, None, :] for x in v)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# Mask semantics
# ---------------------------------------------------------------------------

def _family_cases():
    """(name, vectors, predicate(i, j) -> masked) on small sizes."""
    cases = []
    n = 37
    cases.append(("causal", SM.causal(n), lambda i, j: j > i, n))
    docs = [5, 11, 1, 13, 7]
    seg = np.repeat(np.arange(len(docs)), docs)
    cases.append(("document", SM.document_causal(docs),
                  lambda i, j: seg[i] != seg[j] or j > i, sum(docs)))
    w = 6
    cases.append(("window", SM.sliding_window_causal(n, w),
                  lambda i, j: not (0 <= i - j < w), n))
    p = 9
    cases.append(("prefix_lm", SM.prefix_lm(n, p),
                  lambda i, j: not (j < p or j <= i), n))
    qlen, ans = 7, [4, 9, 3, 6]
    owner = np.concatenate([np.full(qlen, -1), np.repeat(np.arange(len(ans)), ans)])
    cases.append(("share_question", SM.share_question(qlen, ans),
                  lambda i, j: j > i or (owner[j] >= 0 and owner[j] != owner[i]),
                  qlen + sum(ans)))
    cases.append(("none", SM.no_mask(n, n), lambda i, j: False, n))
    return cases


def pin_mask_generators():
    """Every generated family equals its row/key predicate, densely."""
    for name, vec, pred, n in _family_cases():
        dense = OA.dense_mask(*[x.astype(np.int64) for x in vec], np.arange(n))
        truth = np.array([[pred(i, j) for j in range(n)] for i in range(n)])
        assert np.array_equal(dense, truth), f"family {name}"


def pin_causal_tril():
    """Causal from vectors equals the strict upper triangle."""
    n = 64
    dense = OA.dense_mask(*SM.causal(n), np.arange(n))
    assert np.array_equal(~dense, np.tril(np.ones((n, n), bool))), "causal != tril"


def pin_interval_edge_cases():
    """Brute-force per-element evaluation on tiny inputs with adversarial
    bounds: empty, start >= end, negative, beyond Sq, touching, overlapping."""
    rng = np.random.default_rng(11)
    sq, sk = 9, 12
    for _ in range(40):
        v = [rng.integers(-3, sq + 4, sk) for _ in range(4)]
        dense = OA.dense_mask(*v, np.arange(sq))
        for i in range(sq):
            for j in range(sk):
                want = False
                if v[0][j] <= i and i < v[1][j]:
                    want = True
                if v[2][j] <= i and i < v[3][j]:
                    want = True
                assert dense[i, j] == want, (i, j)
    # a missing pair is the empty interval
    v = [None, None, np.array([0, 2]), np.array([3, 2])]
    dense = OA.dense_mask(*v, np.arange(4), 2)
    assert dense.tolist() == [[True, False], [True, False], [True, False], [False, False]]


def pin_nnz():
    """Dense count equals the O(n) closed form; causal(256) has 256*257/2."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        sq, sk = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        v = tuple(rng.integers(-5, sq + 5, (1, 1, sk)) for _ in range(4))
        assert OA.nnz(v, sq) == OA.nnz_closed_form(v, sq)
    c = _vec3(SM.causal(256))
    assert OA.nnz(c, 256) == 32896 == OA.nnz_closed_form(c, 256)


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, allowed, scale):
    """torch SDPA (float64, CPU) on [Sq, D] x [Sk, D] with a bool 'allowed' mask."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if allowed is None else t(allowed), scale=scale)
    return o[0, 0].numpy()


def pin_forward_sdpa_causal():
    """Causal special case equals torch's float64 SDPA with is_causal=True."""
    for n, d, seed in ((33, 8, 1), (70, 16, 2)):
        q, k, v = _rand((1, n, 1, d), seed), _rand((1, n, 1, d), seed + 1), _rand((1, n, 1, d), seed + 2)
        scale = 1 / math.sqrt(d)
        o, _ = OA.forward(q, k, v, _vec3(SM.causal(n)), scale, block=16)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a[0, :, 0]))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(q), t(k), t(v), is_causal=True, scale=scale)[0, 0].numpy()
        _close(o[0, :, 0], ref, 1e-12, "sdpa causal")


def pin_forward_sdpa_masked():
    """Every mask family (and random vectors) equals SDPA with the dense mask,
    on rows that see at least one key; LSE equals torch.logsumexp of the
    masked scores; rows with no open key give O = 0 and LSE = -inf."""
    rng = np.random.default_rng(3)
    cases = [(vec, n) for _, vec, _, n in _family_cases()]
    for _ in range(4):
        sq, sk = int(rng.integers(20, 50)), int(rng.integers(20, 50))
        vec = tuple(rng.integers(-2, sq + 2, sk) for _ in range(4))
        cases.append((vec, (sq, sk)))
    for vec, n in cases:
        sq, sk = (n, n) if isinstance(n, int) else n
        d = 8
        q, k, v = _rand((1, sq, 1, d), 7), _rand((1, sk, 1, d), 8), _rand((1, sk, 1, d), 9)
        scale = 0.3
        o, lse = OA.forward(q, k, v, _vec3(vec), scale, block=8)
        allowed = ~OA.dense_mask(*[np.asarray(x, np.int64) for x in vec], np.arange(sq), sk)
        rows = allowed.any(axis=1)
        ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], allowed, scale)
        _close(o[0, rows, 0], ref[rows], 1e-12, "sdpa masked O")
        s = torch.from_numpy(scale * (q[0, :, 0] @ k[0, :, 0].T))
        s = s.masked_fill(torch.from_numpy(~allowed), -math.inf)
        _close(lse[0, 0, rows], torch.logsumexp(s, dim=1).numpy()[rows], 1e-12, "lse")
        assert np.all(lse[0, 0, ~rows] == -np.inf) and np.all(o[0, ~rows, 0] == 0.0)


def pin_forward_q0_closed_form():
    """Q = 0: every open key scores 0, so O_i is the mean of the open V rows
    and LSE_i = ln(number of open keys)."""
    for _, vec, _, n in _family_cases():
        d = 5
        q = np.zeros((1, n, 1, d))
        k, v = _rand((1, n, 1, d), 1), _rand((1, n, 1, d), 2)
        o, lse = OA.forward(q, k, v, _vec3(vec), 0.7, block=7)
        allowed = ~OA.dense_mask(*vec, np.arange(n))
        for i in range(n):
            cnt = allowed[i].sum()
            if cnt == 0:
                continue
            _close(o[0, i, 0], v[0, allowed[i], 0].mean(axis=0), 1e-12, "q0 mean")
            _close(lse[0, 0, i], math.log(cnt), 1e-12, "q0 lse")


def pin_forward_diagonal():
    """A diagonal-only mask: O = V and LSE_i = scale * q_i . k_i."""
    n, d = 23, 6
    j = np.arange(n)
    vec = (j + 1, np.full(n, n), np.zeros(n, int), j)   # rows != j masked
    q, k, v = _rand((1, n, 1, d), 4), _rand((1, n, 1, d), 5), _rand((1, n, 1, d), 6)
    o, lse = OA.forward(q, k, v, _vec3(vec), 0.4)
    _close(o, v, 1e-12, "diag O")
    _close(lse[0, 0], 0.4 * np.einsum("id,id->i", q[0, :, 0], k[0, :, 0]), 1e-12, "diag lse")


def pin_forward_rows_sum_to_one():
    """With V = I the output is the probability matrix: rows sum to 1 and the
    masked entries are exactly 0."""
    for _, vec, _, n in _family_cases():
        q, k = _rand((1, n, 1, 6), 12), _rand((1, n, 1, 6), 13)
        v = np.eye(n)[None, :, None, :]
        p, _ = OA.forward(q, k, v, _vec3(vec), 0.9)
        p = p[0, :, 0]
        allowed = ~OA.dense_mask(*vec, np.arange(n))
        rows = allowed.any(axis=1)
        _close(p[rows].sum(axis=1), np.ones(rows.sum()), 1e-12, "row sums")
        assert np.all(p[~allowed] == 0.0)


def pin_golden_tiny():
    """Hand-derived values (tests/golden/tiny_causal_q0.json)."""
    with open(os.path.join(GOLDEN, "tiny_causal_q0.json")) as f:
        g = json.load(f)
    n = len(g["v"])
    v = np.asarray(g["v"], dtype=np.float64)[None, :, None, :]
    q = np.zeros_like(v)
    k = np.asarray(g["k"], dtype=np.float64)[None, :, None, :]
    o, lse = OA.forward(q, k, v, _vec3(SM.causal(n)), g["scale"])
    _close(o[0, :, 0], np.asarray(g["o"]), 1e-12, "golden O")
    _close(lse[0, 0], np.asarray(g["lse"]), 1e-12, "golden lse")
    with open(os.path.join(GOLDEN, "tiny_window_scores.json")) as f:
        g = json.load(f)
    n = len(g["k"])
    q = np.asarray(g["q"], dtype=np.float64)[None, :, None, :]
    k = np.asarray(g["k"], dtype=np.float64)[None, :, None, :]
    v = np.asarray(g["v"], dtype=np.float64)[None, :, None, :]
    o, lse = OA.forward(q, k, v, _vec3(SM.sliding_window_causal(n, g["window"])), g["scale"])
    _close(o[0, :, 0], np.asarray(g["o"]), 1e-12, "golden window O")
    _close(lse[0, 0], np.asarray(g["lse"]), 1e-12, "golden window lse")


def pin_key_permutation():
    """Permuting keys, values and all four vectors by one permutation leaves O
    and LSE unchanged and permutes dK, dV."""
    rng = np.random.default_rng(21)
    n, d = 41, 8
    docs = [9, 17, 15]
    vec = _vec3(SM.document_causal(docs))
    q, k, v, do = (_rand((1, n, 1, d), s) for s in (31, 32, 33, 34))
    perm = rng.permutation(n)
    pv = tuple(x[..., perm] for x in vec)
    o1, l1 = OA.forward(q, k, v, vec, 0.5, block=16)
    o2, l2 = OA.forward(q, k[:, perm], v[:, perm], pv, 0.5, block=16)
    _close(o1, o2, 1e-12, "perm O")
    _close(l1, l2, 1e-12, "perm lse")
    g1 = OA.backward(q, k, v, do, vec, 0.5, block=16)
    g2 = OA.backward(q, k[:, perm], v[:, perm], do, pv, 0.5, block=16)
    _close(g1[0], g2[0], 1e-12, "perm dQ")
    _close(g1[1][:, perm], g2[1], 1e-12, "perm dK")
    _close(g1[2][:, perm], g2[2], 1e-12, "perm dV")


def pin_fully_masked_row():
    """A row with no open key: O = 0, LSE = -inf, dQ = 0 and no dK/dV share."""
    n, d = 10, 4
    j = np.arange(n)
    vec = _vec3((np.full(n, 3), np.full(n, 4), np.zeros(n, int), j))  # row 3 sees nothing
    q, k, v, do = (_rand((1, n, 1, d), s) for s in (41, 42, 43, 44))
    o, lse = OA.forward(q, k, v, vec, 1.0)
    assert np.all(o[0, 3] == 0) and lse[0, 0, 3] == -np.inf
    dq, dk, dv = OA.backward(q, k, v, do, vec, 1.0)
    assert np.all(dq[0, 3] == 0)
    do2 = do.copy()
    do2[0, 3] += 100.0
    q2 = q.copy()
    q2[0, 3] += 7.0
    _, dk2, dv2 = OA.backward(q2, k, v, do2, vec, 1.0)
    _close(dk, dk2, 1e-12, "masked row dK share")
    _close(dv, dv2, 1e-12, "masked row dV share")


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def pin_backward_finite_difference():
    """Central differences of L = sum(dO * O) match the oracle gradients."""
    rng = np.random.default_rng(51)
    n, d, scale = 9, 3, 0.8
    vec = _vec3(SM.share_question(3, [2, 4]))
    q, k, v, do = (_rand((1, n, 1, d), s) for s in (52, 53, 54, 55))
    dq, dk, dv = OA.backward(q, k, v, do, vec, scale)
    eps = 1e-6

    def loss(q_, k_, v_):
        return float((OA.forward(q_, k_, v_, vec, scale)[0] * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(10):
            idx = (0, int(rng.integers(n)), 0, int(rng.integers(d)))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            fd = (up - dn) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def pin_backward_autograd():
    """Gradients equal torch autograd through float64 SDPA with the dense mask
    (rows with at least one open key; every family and random vectors)."""
    rng = np.random.default_rng(61)
    cases = [(vec, n, n) for _, vec, _, n in _family_cases()]
    sq, sk = 31, 26
    v_rand = tuple(rng.integers(-2, sq + 2, sk) for _ in range(4))
    cases.append((v_rand, sq, sk))
    for vec, sq, sk in cases:
        d = 6
        allowed = ~OA.dense_mask(*[np.asarray(x, np.int64) for x in vec], np.arange(sq), sk)
        rows = allowed.any(axis=1)
        q, k, v, do = _rand((1, sq, 1, d), 62), _rand((1, sk, 1, d), 63), _rand((1, sk, 1, d), 64), _rand((1, sq, 1, d), 65)
        do[0, ~rows] = 0.0       # SDPA yields NaN on empty rows; exclude them
        tq, tk, tv = (torch.from_numpy(a[0, :, 0].copy())[None, None].requires_grad_(True)
                      for a in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=torch.from_numpy(allowed)[None, None], scale=0.6)
        o = torch.nan_to_num(o, nan=0.0)
        (o * torch.from_numpy(do[0, :, 0])[None, None]).sum().backward()
        dq, dk, dv = OA.backward(q, k, v, do, _vec3(vec), 0.6, block=8)
        _close(dq[0, rows, 0], tq.grad[0, 0].numpy()[rows], 1e-10, "autograd dQ")
        _close(dk[0, :, 0], tk.grad[0, 0].numpy(), 1e-10, "autograd dK")
        _close(dv[0, :, 0], tv.grad[0, 0].numpy(), 1e-10, "autograd dV")


def pin_gqa_autograd():
    """Grouped K/V heads: O and the gradients equal torch float64 SDPA with
    the K/V heads expanded by repeat_interleave (autograd sums the gradients
    of a shared head over its group); per-head masks, 6 query heads on 2 and
    on 1 K/V heads."""
    rng = np.random.default_rng(67)
    sq = sk = 40
    d, H = 6, 6
    fams = [SM.causal(sq), SM.sliding_window_causal(sq, 9), SM.prefix_lm(sq, 12),
            SM.document_causal([9, 17, 14]), SM.no_mask(sq, sq),
            tuple(rng.integers(-2, sq + 2, sk) for _ in range(4))]
    vec = SM.stack([[fams[h] for h in range(H)]])
    for hkv in (2, 1):
        g = H // hkv
        q, do = _rand((1, sq, H, d), 68), _rand((1, sq, H, d), 69)
        k, v = _rand((1, sk, hkv, d), 70), _rand((1, sk, hkv, d), 71)
        allowed = np.stack([~OA.dense_mask(*[np.asarray(x[0, h], np.int64) for x in vec], np.arange(sq), sk)
                            for h in range(H)])
        rows = allowed.any(axis=2)                 # [H, Sq]
        for h in range(H):
            do[0, ~rows[h], h] = 0.0
        tq = torch.from_numpy(q[0].transpose(1, 0, 2).copy())[None].requires_grad_(True)
        tk = torch.from_numpy(k[0].transpose(1, 0, 2).copy())[None].requires_grad_(True)
        tv = torch.from_numpy(v[0].transpose(1, 0, 2).copy())[None].requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1),
            attn_mask=torch.from_numpy(allowed)[None], scale=0.45)
        o = torch.nan_to_num(o, nan=0.0)
        (o * torch.from_numpy(do[0].transpose(1, 0, 2).copy())[None]).sum().backward()
        oo, _ = OA.forward(q, k, v, vec, 0.45)
        dq, dk, dv = OA.backward(q, k, v, do, vec, 0.45, block=16)
        for h in range(H):
            _close(oo[0, rows[h], h], o.detach()[0, h].numpy()[rows[h]], 1e-10, "GQA O")
            _close(dq[0, rows[h], h], tq.grad[0, h].numpy()[rows[h]], 1e-10, "GQA dQ")
        _close(dk[0].transpose(1, 0, 2), tk.grad[0].numpy(), 1e-10, "GQA dK")
        _close(dv[0].transpose(1, 0, 2), tv.grad[0].numpy(), 1e-10, "GQA dV")


def pin_backward_invariants():
    """Softmax is shift invariant, so sum_j dK_j = 0; and sum_j dV_j equals the
    sum of dO over rows with an open key."""
    for _, vec, _, n in _family_cases():
        d = 5
        q, k, v, do = (_rand((1, n, 1, d), s) for s in (71, 72, 73, 74))
        _, dk, dv = OA.backward(q, k, v, do, _vec3(vec), 0.5, block=10)
        allowed = ~OA.dense_mask(*vec, np.arange(n))
        rows = allowed.any(axis=1)
        _close(dk[0, :, 0].sum(axis=0), np.zeros(d), 1e-10, "sum dK")
        _close(dv[0, :, 0].sum(axis=0), do[0, rows, 0].sum(axis=0), 1e-10, "sum dV")


def pin_sampled_equal_full():
    """The sampled-row and sampled-column oracles equal the full oracle."""
    rng = np.random.default_rng(81)
    B, H, n, d = 2, 3, 57, 8
    per = [[SM.document_causal([20, 30, 7]) for _ in range(H)],
           [SM.sliding_window_causal(n, 9) for _ in range(H)]]
    vec = SM.stack(per)
    q, k, v, do = (_rand((B, n, H, d), s) for s in (82, 83, 84, 85))
    o, lse = OA.forward(q, k, v, vec, 0.35, block=16)
    dq, dk, dv = OA.backward(q, k, v, do, vec, 0.35, block=16)
    for b in range(B):
        for h in range(H):
            rows = rng.choice(n, 9, replace=False)
            o_r, l_r = OA.forward_rows(q, k, v, vec, 0.35, b, h, rows)
            _close(o_r, o[b, rows, h], 1e-12, "rows O")
            _close(l_r, lse[b, h, rows], 1e-12, "rows lse")
            _close(OA.backward_rows(q, k, v, do, vec, 0.35, b, h, rows), dq[b, rows, h], 1e-12, "rows dQ")
            cols = rng.choice(n, 7, replace=False)
            dk_c, dv_c = OA.backward_cols(q, k, v, do, vec, 0.35, b, h, cols, block=5)
            _close(dk_c, dk[b, cols, h], 1e-12, "cols dK")
            _close(dv_c, dv[b, cols, h], 1e-12, "cols dV")


# ---------------------------------------------------------------------------
# Localization
# ---------------------------------------------------------------------------

def _random_chunks(rng, sq_glob):
    k = int(rng.integers(1, 6))
    cuts = np.sort(rng.choice(np.arange(sq_glob + 1), size=2 * k, replace=True))
    starts, lens = cuts[0::2], cuts[1::2] - cuts[0::2]
    keep = lens > 0
    if not keep.any():
        return np.array([0]), np.array([sq_glob])
    starts, lens = starts[keep], lens[keep]
    # drop chunks that would touch/overlap the previous one
    s_out, l_out, end = [], [], -1
    for s, l in zip(starts, lens):
        if s >= end:
            s_out.append(s)
            l_out.append(l)
            end = s + l
    return np.array(s_out), np.array(l_out)


def pin_localize_dense_slice():
    """dense(localize(v)) equals dense(v) restricted to the rank's rows."""
    rng = np.random.default_rng(91)
    for _ in range(60):
        sq, sk = int(rng.integers(4, 60)), int(rng.integers(1, 30))
        vec = tuple(rng.integers(-5, sq + 6, (1, 1, sk)) for _ in range(4))
        cs, cl = _random_chunks(rng, sq)
        loc = OM.localize(vec, cs, cl)
        rows = OM.local_rows(cs, cl)
        dl = OA.dense_mask(*[x[0, 0] for x in loc], np.arange(len(rows)), sk)
        dg = OA.dense_mask(*[x[0, 0] for x in vec], rows, sk)
        assert np.array_equal(dl, dg)
    # the dual-chunk assignment of a document mask
    docs = SM.lognormal_doc_lengths(np.random.default_rng(2), 256, 16, 1.0, 2, 128)
    vec = _vec3(SM.document_causal(docs))
    cs, cl = SM.dual_chunk(256, 4, 1)
    loc = OM.localize(vec, cs, cl)
    rows = OM.local_rows(cs, cl)
    assert np.array_equal(OA.dense_mask(*[x[0, 0] for x in loc], np.arange(len(rows))),
                          OA.dense_mask(*[x[0, 0] for x in vec], rows))


def pin_localize_golden():
    """Hand-worked examples (tests/golden/localize_examples.json)."""
    with open(os.path.join(GOLDEN, "localize_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.asarray(c["global"], dtype=np.int64)[None, None, :]
        got = OM.localize((x, x, x, x), c["chunk_start"], c["chunk_len"])[0][0, 0]
        assert got.tolist() == c["local"], (c["note"], got.tolist())


def pin_localize_then_attend():
    """Attention of the rank's rows under localized vectors equals the same
    rows of global attention (forward and dQ), and the rank's share of dK/dV
    equals global dK/dV with dO zero outside the rank's rows."""
    n, d = 64, 8
    docs = [13, 20, 8, 23]
    vec = _vec3(SM.document_causal(docs))
    cs, cl = SM.dual_chunk(n, 2, 1)
    rows = OM.local_rows(cs, cl)
    loc = OM.localize(vec, cs, cl)
    q, k, v, do = (_rand((1, n, 1, d), s) for s in (101, 102, 103, 104))
    og, lg = OA.forward(q, k, v, vec, 0.5)
    ol, ll = OA.forward(q[:, rows], k, v, loc, 0.5)
    _close(ol, og[:, rows], 1e-12, "localized O")
    _close(ll, lg[:, :, rows], 1e-12, "localized lse")
    do_g = np.zeros_like(do)
    do_g[:, rows] = do[:, rows]
    dqg, dkg, dvg = OA.backward(q, k, v, do_g, vec, 0.5)
    dql, dkl, dvl = OA.backward(q[:, rows], k, v, do[:, rows], loc, 0.5)
    _close(dql, dqg[:, rows], 1e-12, "localized dQ")
    _close(dkl, dkg, 1e-12, "localized dK")
    _close(dvl, dvg, 1e-12, "localized dV")


# ---------------------------------------------------------------------------
# Tile classes
# ---------------------------------------------------------------------------

def pin_classes_sound():
    """Rule classes never contradict the dense truth: a SKIP tile is fully
    masked, a FULL tile has no masked pair (random vectors, ragged tiles)."""
    rng = np.random.default_rng(111)
    for _ in range(80):
        sq, sk = int(rng.integers(1, 70)), int(rng.integers(1, 70))
        br, bc = int(rng.choice([4, 8, 16])), int(rng.choice([4, 8, 16]))
        kind = rng.integers(3)
        if kind == 0:
            vec = tuple(rng.integers(-3, sq + 3, (1, 1, sk)) for _ in range(4))
        elif kind == 1:   # structured: intervals anchored like the families
            lo = rng.integers(0, sq + 1, sk)
            up = rng.integers(0, sq + 1, sk)
            vec = _vec3((lo, np.full(sk, sq), np.zeros(sk, int), up))
        else:             # one pair missing
            vec = (None, None) + tuple(rng.integers(-3, sq + 3, (1, 1, sk)) for _ in range(2))
        rule = OM.tile_classes(vec, sq, sk, br, bc)
        truth = OM.tile_classes_dense(vec, sq, sk, br, bc)
        assert not np.any((rule == oracle.SKIP) & (truth != oracle.SKIP)), "unsound SKIP"
        assert not np.any((rule == oracle.FULL) & (truth != oracle.FULL)), "unsound FULL"


def pin_classes_exact_on_families():
    """With canonical empties the rule equals the dense truth on every mask
    family, with ragged tiles and Br != Bc, and on a localized dual-chunk
    document mask whose chunk length is a multiple of Br."""
    for _, vec, _, n in _family_cases():
        for br, bc in ((4, 4), (8, 4), (4, 16), (16, 8)):
            v3 = _vec3(vec)
            assert np.array_equal(OM.tile_classes(v3, n, n, br, bc),
                                  OM.tile_classes_dense(v3, n, n, br, bc)), (br, bc)
    docs = SM.lognormal_doc_lengths(np.random.default_rng(3), 512, 32, 1.0, 4, 256)
    vec = _vec3(SM.document_causal(docs))
    cs, cl = SM.dual_chunk(512, 4, 2)
    loc = OM.localize(vec, cs, cl)
    for br, bc in ((16, 16), (32, 16), (64, 32)):
        assert np.array_equal(OM.tile_classes(loc, 128, 512, br, bc),
                              OM.tile_classes_dense(loc, 128, 512, br, bc)), (br, bc)


# ---------------------------------------------------------------------------
# Mask-pruned K/V transfer set
# ---------------------------------------------------------------------------

def _tiles_of_keys(needed_keys, sk, bc):
    tk = -(-sk // bc)
    out = np.zeros(tk, dtype=np.uint8)
    for j in np.flatnonzero(needed_keys):
        out[j // bc] = 1
    return out


def pin_transfer_set_brute_force():
    """Element-by-element loops on tiny random vectors (any int values, a
    missing pair, broadcast shapes) against the oracle."""
    rng = np.random.default_rng(131)
    for it in range(40):
        sq, sk = int(rng.integers(1, 12)), int(rng.integers(1, 20))
        bc = int(rng.choice([1, 3, 4, 7]))
        bm, hm = (1, 1) if it % 3 else (2, 3)
        vec = [rng.integers(-4, sq + 5, (bm, hm, sk)) for _ in range(4)]
        if it % 5 == 0:
            vec[0] = vec[1] = None
        got = OM.transfer_set(tuple(vec), sq, sk, bc)
        tk = -(-sk // bc)
        assert got.shape == (bm, hm, tk)
        for b in range(bm):
            for h in range(hm):
                for t in range(tk):
                    want = 0
                    for j in range(t * bc, min((t + 1) * bc, sk)):
                        for i in range(sq):
                            lo = vec[0] is not None and vec[0][b, h, j] <= i < vec[1][b, h, j]
                            up = vec[2][b, h, j] <= i < vec[3][b, h, j]
                            if not (lo or up):
                                want = 1
                    assert got[b, h, t] == want, (it, b, h, t)


def pin_transfer_set_closed_forms():
    """The rank's rows R (dual-chunk assignment) and closed forms of the keys
    they reach: causal, keys 0 .. max R; document-causal, per document the
    keys from its start to its last row in R; sliding window W, keys j with
    some row of R in [j, j + W); no mask, every key."""
    n, bc = 96, 8
    for degree, rank in ((2, 0), (2, 1), (4, 3), (3, 2)):
        if n % (2 * degree):
            continue
        cs, cl = SM.dual_chunk(n, degree, rank)
        rows = OM.local_rows(cs, cl)
        sq = len(rows)
        # causal
        loc = OM.localize(_vec3(SM.causal(n)), cs, cl)
        need = np.arange(n) <= rows.max()
        assert np.array_equal(OM.transfer_set(loc, sq, n, bc)[0, 0], _tiles_of_keys(need, n, bc))
        # document-causal
        docs = [11, 30, 7, 26, 22]
        starts = np.concatenate([[0], np.cumsum(docs)[:-1]])
        loc = OM.localize(_vec3(SM.document_causal(docs)), cs, cl)
        need = np.zeros(n, dtype=bool)
        for s0, ln in zip(starts, docs):
            mine = rows[(rows >= s0) & (rows < s0 + ln)]
            if len(mine):
                need[s0:mine.max() + 1] = True
        assert np.array_equal(OM.transfer_set(loc, sq, n, bc)[0, 0], _tiles_of_keys(need, n, bc))
        # sliding window
        w = 13
        loc = OM.localize(_vec3(SM.sliding_window_causal(n, w)), cs, cl)
        need = np.array([np.any((rows >= j) & (rows < j + w)) for j in range(n)])
        assert np.array_equal(OM.transfer_set(loc, sq, n, bc)[0, 0], _tiles_of_keys(need, n, bc))
    # no mask
    assert OM.transfer_set((None, None, None, None), 5, 37, 8).tolist() == [[[1] * 5]]


def pin_transfer_set_matches_classes():
    """Where the tile classes are exact (every mask family, and a localized
    dual-chunk document mask), a key tile is needed exactly when some row
    tile's class for it is not SKIP."""
    for _, vec, _, n in _family_cases():
        v3 = _vec3(vec)
        for br, bc in ((4, 4), (8, 16), (16, 8)):
            cls = OM.tile_classes(v3, n, n, br, bc)
            assert np.array_equal(OM.transfer_set(v3, n, n, bc)[0, 0],
                                  (cls != oracle.SKIP).any(axis=0).astype(np.uint8)), (br, bc)
    docs = SM.lognormal_doc_lengths(np.random.default_rng(4), 512, 32, 1.0, 4, 256)
    vec = _vec3(SM.document_causal(docs))
    cs, cl = SM.dual_chunk(512, 4, 1)
    loc = OM.localize(vec, cs, cl)
    cls = OM.tile_classes(loc, 128, 512, 32, 16)
    assert np.array_equal(OM.transfer_set(loc, 128, 512, 16)[0, 0],
                          (cls != oracle.SKIP).any(axis=0).astype(np.uint8))


# ---------------------------------------------------------------------------
# Chunk work and the chunk -> rank plan
# ---------------------------------------------------------------------------

def pin_chunk_work_closed_forms():
    """Per-chunk open pairs against row-by-row closed forms: causal (row i
    sees i + 1 keys), document-causal (row i sees i - start(doc) + 1),
    sliding window W (min(i + 1, W)), no mask (all Sk keys)."""
    n = 120
    starts, lens = [0, 17, 40, 77, 90], [17, 23, 37, 13, 30]
    docs = [25, 8, 40, 47]
    doc_start = np.repeat(np.concatenate([[0], np.cumsum(docs)[:-1]]), docs)
    w = 19
    cases = [(SM.causal(n), lambda i: i + 1),
             (SM.document_causal(docs), lambda i: i - doc_start[i] + 1),
             (SM.sliding_window_causal(n, w), lambda i: min(i + 1, w)),
             (SM.no_mask(n, n), lambda i: n)]
    for vec, per_row in cases:
        got = OM.chunk_work(_vec3(vec), n, starts, lens)[0]
        want = [sum(per_row(i) for i in range(s0, s0 + ln)) for s0, ln in zip(starts, lens)]
        assert got.tolist() == want


def pin_chunk_work_partition_sums_to_nnz():
    """Chunks that partition the query axis add up to the O(Sk) closed-form
    count of open pairs (random vectors, broadcast shapes, a missing pair)."""
    rng = np.random.default_rng(141)
    for it in range(20):
        sq, sk = int(rng.integers(1, 60)), int(rng.integers(1, 40))
        bm, hm = (1, 1) if it % 2 else (2, 3)
        vec = [rng.integers(-5, sq + 6, (bm, hm, sk)) for _ in range(4)]
        if it % 4 == 0:
            vec[2] = vec[3] = None
        cuts = np.unique(np.concatenate([[0, sq], rng.integers(0, sq + 1, 3)]))
        starts, lens = cuts[:-1], np.diff(cuts)
        got = OM.chunk_work(tuple(vec), sk, starts, lens)
        for b in range(bm):
            for h in range(hm):
                sub = tuple(None if x is None else x[b:b + 1, h:h + 1] for x in vec)
                assert int(got[b * hm + h].sum()) == OA.nnz_closed_form(sub, sq)


def pin_best_plan_exhaustive():
    """The pruned exhaustive search equals plain enumeration of every
    assignment with len / ranks chunks per rank (tiny random works)."""
    import itertools
    rng = np.random.default_rng(151)
    for c, r in ((4, 2), (6, 3), (6, 2), (8, 4)):
        for _ in range(4):
            work = rng.integers(0, 100, c)
            per = c // r
            best = None
            for assign in itertools.product(range(r), repeat=c):
                if any(assign.count(k) != per for k in range(r)):
                    continue
                m = int(OM.plan_loads(work, assign, r).max())
                best = m if best is None else min(best, m)
            assert OM.best_plan_max(work, r) == best, (c, r, work)



# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) inputs
# ---------------------------------------------------------------------------

def _torch_e4m3(codes):
    """torch's own float8_e4m3fn -> float64 conversion (a library routine)."""
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_e4m3_decode_library():
    """Every one of the 256 codes decodes as torch.float8_e4m3fn does,
    signs of zero and NaN positions included."""
    codes = np.arange(256)
    a, b = OF.e4m3_decode(codes), _torch_e4m3(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b)), "NaN codes differ"
    fin = ~np.isnan(b)
    assert np.array_equal(a[fin], b[fin]), "decoded values differ"
    assert np.array_equal(np.signbit(a[fin]), np.signbit(b[fin])), "signed zeros differ"


def pin_e4m3_decode_hand_values():
    """Values fixed by the format's definition: 1.0, the largest finite
    value 448, the smallest normal 2^-6 and subnormal 2^-9, a subnormal
    7/8 * 2^-6, -2, 1.875, NaN at the all-ones code."""
    table = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6,
             0xC0: -2.0, 0x3F: 1.875, 0x00: 0.0}
    got = OF.e4m3_decode(list(table))
    assert np.array_equal(got, np.array(list(table.values()))), got
    assert np.isnan(OF.e4m3_decode([0x7F, 0xFF])).all()


def _fp8_case(n, d, seed, hkv=1):
    rng = np.random.default_rng(seed)
    q8 = rng.integers(0, 256, (1, n, 1, d)).astype(np.uint8)
    k8 = rng.integers(0, 256, (1, n, hkv, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, (1, n, hkv, d)).astype(np.uint8)
    for x in (q8, k8, v8):   # no NaN codes
        x[(x & 0x7F) == 0x7F] = 0x38
    return q8, k8, v8


def pin_fp8_forward_equal_keys():
    """All keys carry the same code vector: every open key scores the same,
    so O_i is the mean of the open V rows (decoded by torch, times the V
    descale) and LSE_i = scale * dq * dk * (q_i . k) + ln(open count)."""
    for _, vec, _, n in _family_cases():
        d = 4
        q8, _, v8 = _fp8_case(n, d, 11)
        k8 = np.broadcast_to(np.array([0x3C, 0xB0, 0x44, 0x28], np.uint8), (1, n, 1, d)).copy()
        ds = (0.5, 0.25, 1.5)
        o, lse = OF.forward(q8, k8, v8, ds, _vec3(vec), 0.3)
        vt = _torch_e4m3(v8)[0, :, 0] * 1.5
        qk = (_torch_e4m3(q8)[0, :, 0] * 0.5) @ (_torch_e4m3(k8)[0, 0, 0] * 0.25)
        allowed = ~OA.dense_mask(*vec, np.arange(n))
        for i in range(n):
            cnt = allowed[i].sum()
            if cnt == 0:
                continue
            _close(o[0, i, 0], vt[allowed[i]].mean(axis=0), 1e-12, "fp8 equal keys O")
            _close(lse[0, 0, i], 0.3 * qk[i] + math.log(cnt), 1e-12, "fp8 equal keys LSE")


def pin_fp8_forward_diagonal():
    """Diagonal-only mask: O_i = v_i * dv and LSE_i = scale * dq * dk * q_i . k_i,
    with every code decoded by torch."""
    n, d = 19, 8
    j = np.arange(n)
    vec = (j + 1, np.full(n, n), np.zeros(n, int), j)
    q8, k8, v8 = _fp8_case(n, d, 12)
    ds = (0.125, 2.0, 0.75)
    o, lse = OF.forward(q8, k8, v8, ds, _vec3(vec), 0.9)
    qd, kd, vd = (_torch_e4m3(x)[0, :, 0] for x in (q8, k8, v8))
    _close(o[0, :, 0], vd * 0.75, 1e-12, "fp8 diag O")
    _close(lse[0, 0], 0.9 * 0.125 * 2.0 * np.einsum("id,id->i", qd, kd), 1e-12, "fp8 diag LSE")


def pin_fp8_forward_descale_invariants():
    """Only the product dq * dk enters the scores, and O is linear in dv:
    (dq, dk, dv) = (2, 0.5, 3) gives LSE(1, 1, 1) and 3 * O(1, 1, 1); a
    permutation of the keys (with their bound vectors) changes nothing."""
    n, d = 29, 6
    q8, k8, v8 = _fp8_case(n, d, 13)
    vec = SM.sliding_window_causal(n, 7)
    o1, l1 = OF.forward(q8, k8, v8, (1.0, 1.0, 1.0), _vec3(vec), 0.2)
    o2, l2 = OF.forward(q8, k8, v8, (2.0, 0.5, 3.0), _vec3(vec), 0.2)
    _close(o2, 3.0 * o1, 1e-12, "fp8 dv linear")
    _close(l2, l1, 1e-12, "fp8 dq*dk")
    perm = np.random.default_rng(3).permutation(n)
    vp = tuple(None if x is None else np.asarray(x)[perm] for x in vec)
    o3, l3 = OF.forward(q8, k8[:, perm], v8[:, perm], (1.0, 1.0, 1.0), _vec3(vp), 0.2)
    _close(o3, o1, 1e-12, "fp8 key permutation O")
    _close(l3, l1, 1e-12, "fp8 key permutation LSE")

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
