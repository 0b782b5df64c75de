"""CPU oracle for masked attention under column-sparse masks.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the package smoke entry and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and has no CPU fallback.

Plain, slow, obviously correct float64 numpy. It shares nothing with the HIP
path: it materialises the dense mask from the four bound vectors (one block of
query rows at a time, since a 131072^2 boolean mask is 16 GiB) and evaluates
softmax attention and its gradients by their definitions.

Sources (the pages are three web pages; cited by title and section):
  * "FlashMask-3: ядро внимания с масками для GPU Hopper и распределённого
    обучения" (iitog.ru), paragraph on the predecessor FlashMask: the mask is
    stored column-sparse, as four bound vectors on the query axis per key
    column, O(n) instead of O(n^2).
  * same page, contributions paragraph and "Key facts": per-rank localization
    of the mask is clip / shift / max on the bound vectors and needs no
    communication.
  * "FlashAttention-2 ... GPU work partitioning" (iplexlaw.co.kr), section
    "Block processing keeps the global normalization": the tiled algorithm
    computes exact attention, normalised over the whole sequence; only the
    floating-point order differs, so outputs and gradients are compared with
    tolerances.

Readings taken where the pages are silent (they give no formula, no vector
names and no API):
  * names and semantics of the four vectors: for key column j, query row i is
    masked iff lts[j] <= i < lte[j] or uts[j] <= i < ute[j] (two half-open
    intervals, "lower" and "upper"); an interval with start >= end is empty.
    A missing (None) pair is the empty interval.
  * softmax scale as given; LSE is the natural-log logsumexp of the scaled
    scores; a row with no open key has O = 0, LSE = -inf and zero gradients.
  * grouped-query attention: "Современное состояние Flash Attention на ROCm"
    (kripta.biz), ranking paragraph, names GQA among the features of the FA2
    Triton backend without defining it. The usual reading is taken: k and v
    may hold H_kv heads with H_kv dividing H; query head h uses K/V head
    h // (H / H_kv) (groups of consecutive query heads), and a shared K/V
    head's gradients are the sums over its group (the chain rule for a
    shared input).

Array conventions: q, o, do are [B, Sq, H, D]; k, v are [B, Sk, H_kv, D]; each
bound vector is an integer array [Bm, Hm, Sk] with Bm in {1, B} and Hm in
{1, H} (size 1 broadcasts) or None. Inputs of any float dtype are upcast
exactly to float64.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

# Tile classes (pre-pass output). The pages say nothing about tiling masks;
# the class values are this implementation's encoding.
SKIP, PARTIAL, FULL = 0, 1, 2


# ---------------------------------------------------------------------------
# Mask semantics
# ---------------------------------------------------------------------------

def _pick(vec, b, h):
    """The [Sk] slice of a [Bm, Hm, Sk] vector for batch b, head h (broadcast)."""
    if vec is None:
        return None
    vec = np.asarray(vec)
    return vec[b if vec.shape[0] > 1 else 0, h if vec.shape[1] > 1 else 0].astype(np.int64)


def vectors_for(vectors, b, h):
    """(lts, lte, uts, ute) as int64 [Sk] arrays (None kept) for one (b, h)."""
    return tuple(_pick(x, b, h) for x in vectors)


def dense_mask(lts, lte, uts, ute, rows, n_keys=None):
    """Dense boolean mask, True = masked, for the given query row indices.

    Column-sparse form (FlashMask-3 page, predecessor paragraph): each key
    column j hides the query rows of its two intervals, so
    masked[i, j] = (lts[j] <= i < lte[j]) or (uts[j] <= i < ute[j]).
    A None pair contributes nothing.
    """
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    if n_keys is None:
        n_keys = len(next(x for x in (lts, lte, uts, ute) if x is not None))
    m = np.zeros((rows.shape[0], n_keys), dtype=bool)
    if lts is not None:
        m |= (np.asarray(lts)[None, :] <= rows) & (rows < np.asarray(lte)[None, :])
    if uts is not None:
        m |= (np.asarray(uts)[None, :] <= rows) & (rows < np.asarray(ute)[None, :])
    return m


def nnz(vectors, seq_q, batch=1, heads=1):
    """Number of open (query, key) pairs summed over batch and heads, by
    counting the dense mask row block by row block."""
    total = 0
    for b in range(batch):
        for h in range(heads):
            v = vectors_for(vectors, b, h)
            for r0 in range(0, seq_q, 4096):
                rows = np.arange(r0, min(r0 + 4096, seq_q))
                total += int((~dense_mask(*v, rows)).sum())
    return total


def nnz_closed_form(vectors, seq_q, batch=1, heads=1):
    """The same count in O(Sk): column j is open for Sq - |L_j U U_j| rows,
    with each interval first clipped to [0, Sq)."""
    total = 0
    for b in range(batch):
        for h in range(heads):
            lts, lte, uts, ute = vectors_for(vectors, b, h)
            n_keys = len(next(x for x in (lts, lte, uts, ute) if x is not None))

            def clip(s, e):
                if s is None:
                    z = np.zeros(n_keys, dtype=np.int64)
                    return z, z
                s = np.clip(s, 0, seq_q)
                e = np.clip(e, 0, seq_q)
                return s, np.maximum(e, s)

            a0, a1 = clip(lts, lte)
            b0, b1 = clip(uts, ute)
            inter = np.maximum(0, np.minimum(a1, b1) - np.maximum(a0, b0))
            union = (a1 - a0) + (b1 - b0) - inter
            total += int((seq_q - union).sum())
    return total


# ---------------------------------------------------------------------------
# Forward: exact softmax attention (FlashAttention-2 page, "Block processing
# keeps the global normalization": the result is the softmax over the whole
# key sequence, which is what is evaluated here, one row block at a time with
# no streaming or rescaling).
# ---------------------------------------------------------------------------

def _rows_forward(qrows, k, v, maskrows, scale):
    """O and LSE for a block of query rows of one (b, h).

    qrows [R, D]; k, v [Sk, D]; maskrows [R, Sk] (True = masked).
    """
    s = scale * (qrows @ k.T)
    s[maskrows] = -np.inf
    open_any = ~maskrows.all(axis=1)
    m = np.where(open_any, np.max(s, axis=1), 0.0)
    p = np.exp(s - m[:, None])                 # exp(-inf) = 0 on masked keys
    l = p.sum(axis=1)
    o = np.zeros((qrows.shape[0], v.shape[1]), dtype=F64)
    lse = np.full(qrows.shape[0], -np.inf)
    o[open_any] = (p[open_any] @ v) / l[open_any, None]
    lse[open_any] = m[open_any] + np.log(l[open_any])
    return o, lse


def kv_head(q_heads, kv_heads, h):
    """K/V head of query head h (grouped-query attention reading above)."""
    if kv_heads < 1 or q_heads % kv_heads:
        raise ValueError(f"{kv_heads} K/V heads do not divide {q_heads} query heads")
    return h // (q_heads // kv_heads)


def forward(q, k, v, vectors, scale, block=1024):
    """Masked attention forward. Returns O [B, Sq, H, D] and LSE [B, H, Sq]."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    B, Sq, H, _ = q.shape
    o = np.zeros((B, Sq, H, v.shape[-1]))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            vec = vectors_for(vectors, b, h)
            hk = kv_head(H, k.shape[2], h)
            kb, vb = k[b, :, hk], v[b, :, hk]
            for r0 in range(0, Sq, block):
                rows = np.arange(r0, min(r0 + block, Sq))
                ob, lb = _rows_forward(q[b, rows, h], kb, vb,
                                       dense_mask(*vec, rows, kb.shape[0]), scale)
                o[b, rows, h] = ob
                lse[b, h, rows] = lb
    return o, lse


# ---------------------------------------------------------------------------
# Backward: the gradient of the exact forward (same passage: outputs and
# gradients are the exact ones, compared with tolerances). For one row,
# P = softmax(S), O = P V, S = scale * Q K^T, so with dP = dO V^T:
#   dV = P^T dO,  dS = P * (dP - rowsum(P * dP)),
#   dQ = scale * dS K,  dK = scale * dS^T Q.
# Masked entries have P = 0 and so contribute nothing.
# ---------------------------------------------------------------------------

def _rows_probs(qrows, k, maskrows, scale):
    s = scale * (qrows @ k.T)
    s[maskrows] = -np.inf
    open_any = ~maskrows.all(axis=1)
    m = np.where(open_any, np.max(s, axis=1), 0.0)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    p[open_any] /= l[open_any, None]
    p[~open_any] = 0.0
    return p


def backward(q, k, v, do, vectors, scale, block=1024):
    """Masked attention backward. Returns dQ, dK, dV (float64, input shapes)."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    do = np.asarray(do, dtype=F64)
    B, Sq, H, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            vec = vectors_for(vectors, b, h)
            hk = kv_head(H, k.shape[2], h)
            kb, vb = k[b, :, hk], v[b, :, hk]
            for r0 in range(0, Sq, block):
                rows = np.arange(r0, min(r0 + block, Sq))
                p = _rows_probs(q[b, rows, h], kb, dense_mask(*vec, rows, kb.shape[0]), scale)
                dob = do[b, rows, h]
                dp = dob @ vb.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, rows, h] = scale * (ds @ kb)
                dk[b, :, hk] += scale * (ds.T @ q[b, rows, h])
                dv[b, :, hk] += p.T @ dob
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Sampled outputs at full size: every output row depends only on its own query
# row, and every dK/dV column only on the rows that attend that key.
# ---------------------------------------------------------------------------

def forward_rows(q, k, v, vectors, scale, b, h, rows):
    """O [R, D] and LSE [R] for the listed query rows of (b, h)."""
    rows = np.asarray(rows, dtype=np.int64)
    vec = vectors_for(vectors, b, h)
    hk = kv_head(q.shape[2], k.shape[2], h)
    kb = np.asarray(k[b, :, hk], dtype=F64)
    vb = np.asarray(v[b, :, hk], dtype=F64)
    qr = np.asarray(q[b, rows, h], dtype=F64)
    return _rows_forward(qr, kb, vb, dense_mask(*vec, rows, kb.shape[0]), scale)


def backward_rows(q, k, v, do, vectors, scale, b, h, rows):
    """dQ [R, D] for the listed query rows of (b, h)."""
    rows = np.asarray(rows, dtype=np.int64)
    vec = vectors_for(vectors, b, h)
    hk = kv_head(q.shape[2], k.shape[2], h)
    kb = np.asarray(k[b, :, hk], dtype=F64)
    vb = np.asarray(v[b, :, hk], dtype=F64)
    p = _rows_probs(np.asarray(q[b, rows, h], dtype=F64), kb,
                    dense_mask(*vec, rows, kb.shape[0]), scale)
    dp = np.asarray(do[b, rows, h], dtype=F64) @ vb.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ kb)


def backward_cols(q, k, v, do, vectors, scale, b, h, cols, block=512):
    """Query head h's share of dK [C, D] and dV [C, D] for the listed key
    columns of (b, h) (the whole of them without grouped K/V heads).

    Only the query rows that attend at least one listed key contribute; each
    such row's softmax is still taken over all of its keys.
    """
    cols = np.asarray(cols, dtype=np.int64)
    vec = vectors_for(vectors, b, h)
    Sq = q.shape[1]
    hk = kv_head(q.shape[2], k.shape[2], h)
    kb = np.asarray(k[b, :, hk], dtype=F64)
    vb = np.asarray(v[b, :, hk], dtype=F64)
    # rows touching the listed columns
    colvec = tuple(None if x is None else x[cols] for x in vec)
    touching = []
    for r0 in range(0, Sq, 8192):
        rows = np.arange(r0, min(r0 + 8192, Sq))
        hit = ~dense_mask(*colvec, rows, len(cols))
        touching.append(rows[hit.any(axis=1)])
    touching = np.concatenate(touching)
    dk = np.zeros((len(cols), kb.shape[1]))
    dv = np.zeros((len(cols), vb.shape[1]))
    for r0 in range(0, len(touching), block):
        rows = touching[r0:r0 + block]
        qr = np.asarray(q[b, rows, h], dtype=F64)
        p = _rows_probs(qr, kb, dense_mask(*vec, rows, kb.shape[0]), scale)
        dob = np.asarray(do[b, rows, h], dtype=F64)
        dp = dob @ vb.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dk += scale * (ds[:, cols].T @ qr)
        dv += p[:, cols].T @ dob
    return dk, dv
