"""Seeded structural masks in the column-sparse (four bound vectors) form.

Input construction only: this module builds the mask *encoding* that both the
oracle and the HIP path take as input. It computes no attention.

Representation (FlashMask-3 news page, paragraph on the predecessor FlashMask:
the mask is stored per key column as four bound vectors on the query axis,
O(n) memory instead of O(n^2)). Reading adopted for the names and semantics:
for key column ``j`` the query rows ``i`` with

    lts[j] <= i < lte[j]      ("lower" interval)      or
    uts[j] <= i < ute[j]      ("upper" interval)

are masked (cannot attend key ``j``); every other row attends it. Both
intervals are half open; an interval with start >= end is empty. The
canonical empty lower interval is ``[Sq, Sq)`` and the canonical empty upper
interval is ``[0, 0)``.

Every generator returns ``(lts, lte, uts, ute)`` as int32 numpy arrays of
length ``Sk`` (the number of key columns).
"""
from __future__ import annotations

import numpy as np

I32 = np.int32


def _pack(lts, lte, uts, ute):
    return tuple(np.ascontiguousarray(np.asarray(x, dtype=I32)) for x in (lts, lte, uts, ute))


def causal(n: int):
    """Plain causal over a square n x n problem: key j is hidden from rows i < j."""
    j = np.arange(n, dtype=np.int64)
    return _pack(np.full(n, n), np.full(n, n), np.zeros(n), j)


def document_causal(doc_lengths):
    """Causal inside each document, fully masked across documents.

    Key j in document [s, e): rows i < j are masked (upper interval [0, j)) and
    rows of later documents are masked (lower interval [e, n)).
    """
    lengths = np.asarray(doc_lengths, dtype=np.int64)
    n = int(lengths.sum())
    ends = np.cumsum(lengths)
    doc_end = np.repeat(ends, lengths)
    j = np.arange(n, dtype=np.int64)
    return _pack(doc_end, np.full(n, n), np.zeros(n), j)


def sliding_window_causal(n: int, window: int):
    """Row i attends keys j with 0 <= i - j < window.

    Key j: rows i < j masked (upper [0, j)); rows i >= j + window masked
    (lower [min(j + window, n), n)).
    """
    j = np.arange(n, dtype=np.int64)
    return _pack(np.minimum(j + window, n), np.full(n, n), np.zeros(n), j)


def prefix_lm(n: int, prefix: int):
    """Bidirectional prefix of ``prefix`` tokens, causal after it.

    Keys j < prefix are open to every row (both intervals empty); keys
    j >= prefix are causal (upper [0, j)).
    """
    j = np.arange(n, dtype=np.int64)
    ute = np.where(j < prefix, 0, j)
    return _pack(np.full(n, n), np.full(n, n), np.zeros(n), ute)


def share_question(question_len: int, answer_lengths):
    """A question followed by answers that share it.

    Question keys: causal inside the question and open to every answer row
    (upper [0, j), lower empty). Answer k keys in [s_k, e_k): causal inside the
    answer and hidden from later answers (upper [0, j), lower [e_k, n)).
    Rows of an answer therefore see the question and their own prefix only.
    """
    ans = np.asarray(answer_lengths, dtype=np.int64)
    n = int(question_len + ans.sum())
    j = np.arange(n, dtype=np.int64)
    lts = np.full(n, n, dtype=np.int64)
    ends = question_len + np.cumsum(ans)
    lts[question_len:] = np.repeat(ends, ans)
    return _pack(lts, np.full(n, n), np.zeros(n), j)


def no_mask(n_keys: int, n_rows: int):
    """Every row attends every key (canonical empty intervals)."""
    return _pack(np.full(n_keys, n_rows), np.full(n_keys, n_rows),
                 np.zeros(n_keys), np.zeros(n_keys))


# ----------------------------------------------------------------------------
# Length draws (seeded). The recipes are the readings of the workload text:
# draw until the lengths cover the sequence, then truncate the last one.
# ----------------------------------------------------------------------------

def _cover(draw, n: int):
    out, total = [], 0
    while total < n:
        x = int(draw())
        out.append(x)
        total += x
    out[-1] -= total - n
    if out[-1] <= 0:
        out.pop()
    return np.asarray(out, dtype=np.int64)


def uniform_doc_lengths(rng: np.random.Generator, n: int, lo: int = 64, hi: int = 1024):
    """Document lengths drawn uniformly from the integers [lo, hi]."""
    return _cover(lambda: rng.integers(lo, hi + 1), n)


def lognormal_doc_lengths(rng: np.random.Generator, n: int, median: float = 4096.0,
                          sigma: float = 1.0, lo: int = 128, hi: int = 65536):
    """Document lengths round(lognormal(ln median, sigma)) clipped to [lo, hi]."""
    mu = float(np.log(median))
    return _cover(lambda: min(max(int(round(rng.lognormal(mu, sigma))), lo), hi), n)


def answer_lengths(rng: np.random.Generator, total: int, count: int):
    """A uniform random composition of ``total`` into ``count`` positive parts.

    ``count - 1`` distinct cut points are drawn from [1, total - 1] and sorted.
    """
    cuts = np.sort(rng.choice(np.arange(1, total), size=count - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total]])
    return np.diff(edges).astype(np.int64)


def dual_chunk(global_len: int, degree: int, rank: int):
    """Dual-chunk context assignment for one rank.

    The sequence is cut into 2*degree equal chunks; rank r holds chunks r and
    2*degree - 1 - r, listed in ascending global order.
    Returns (chunk_start, chunk_len) as int32 arrays.
    """
    if global_len % (2 * degree):
        raise ValueError("global_len must be a multiple of 2*degree")
    c = global_len // (2 * degree)
    first, second = rank, 2 * degree - 1 - rank
    starts = sorted([first * c, second * c])
    return np.asarray(starts, dtype=I32), np.asarray([c, c], dtype=I32)


def stack(per_head):
    """Stack per-(batch, head) vector sets into [Bm, Hm, Sk] arrays.

    ``per_head`` is a nested list [Bm][Hm] of (lts, lte, uts, ute) tuples.
    """
    out = []
    for v in range(4):
        out.append(np.ascontiguousarray(np.asarray(
            [[hv[v] for hv in bv] for bv in per_head], dtype=I32)))
    return tuple(out)
