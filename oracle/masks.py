"""CPU oracle for the integer steps: mask localization and tile classes.

TEST INFRASTRUCTURE ONLY (see ``oracle/attention.py``): nothing on the
product path imports it.

Localization follows "FlashMask-3: ядро внимания с масками для GPU Hopper и
распределённого обучения" (iitog.ru), contributions paragraph and "Key
facts": the mask is indexed by key position but stores query-axis interval
bounds, so a rank that holds several fragments of the context localizes it by
operating on the bound vectors alone (clip, shift, max), with no
communication. The oracle does not use clip/shift/max: it uses the counting
definition that the operation must reproduce. With the rank's rows in
ascending global order g_0 < g_1 < ..., a global bound x becomes
    x' = #{ r : g_r < x },
the number of local rows whose global index is below x. Then local row r lies
in [S', E') exactly when g_r lies in [S, E), so every interval maps to one
contiguous local interval.

Transfer set: the same page (contributions paragraph and "Key facts") pairs
the overlap of computation and communication with dropping the transfers the
mask makes useless; it gives no rule or granularity. The reading adopted: a
rank needs key tile kt (keys [kt*Bc, min((kt+1)*Bc, Sk))) exactly when at
least one of its rows attends at least one key of the tile, which the oracle
takes from the dense mask over the rank's rows.

Chunk work: the same page names a sparsity-aware load balancer (HCC-IPO) for
context parallelism and nothing more. What it must balance is taken to be
the attention work of a rank, i.e. its open (row, key) pairs; the oracle
counts them per chunk of the global query axis from the dense mask.

Tile classes: the pages do not describe a tile pre-pass. The rule here is the
reading adopted for it. Per K/V tile, the minimum and maximum of each bound
vector over the tile's columns are reduced; a (Q tile, K tile) pair with rows
[r0, r1) is
    SKIP    if for the lower or for the upper interval every column's
            interval covers all rows: max(start) <= r0 and min(end) >= r1;
    FULL    else if for both intervals every column's interval misses the
            rows on one common side: max(end) <= r0 or min(start) >= r1;
    PARTIAL otherwise.
A missing (None) pair stands for the canonical empty intervals: lower
[Sq, Sq) and upper [0, 0). The dense-truth classes (all rows x columns
masked / none masked) are computed separately for soundness checks.
"""
from __future__ import annotations

import numpy as np

from .attention import dense_mask, vectors_for, SKIP, PARTIAL, FULL


def local_rows(chunk_start, chunk_len):
    """Global indices of a rank's rows, chunk by chunk in the listed order."""
    return np.concatenate([np.arange(int(s), int(s) + int(l), dtype=np.int64)
                           for s, l in zip(chunk_start, chunk_len)])


def localize(vectors, chunk_start, chunk_len):
    """Localized bound vectors by the counting definition.

    ``vectors`` is (lts, lte, uts, ute), each [Bm, Hm, Sk] or None; chunks must
    be listed in ascending global order and must not overlap. Returns int32
    arrays of the same shapes.
    """
    rows = local_rows(chunk_start, chunk_len)
    if np.any(np.diff(rows) <= 0):
        raise ValueError("chunks must be ascending and non-overlapping")
    out = []
    for x in vectors:
        if x is None:
            out.append(None)
            continue
        x = np.asarray(x, dtype=np.int64)
        out.append(np.searchsorted(rows, x, side="left").astype(np.int32))
    return tuple(out)


def transfer_set(vectors, seq_q, seq_k, block_k):
    """Mask-pruned K/V transfer set: uint8 [Bm, Hm, Tk], 1 where some row in
    [0, seq_q) attends some key of tile kt (dense truth, row block by row
    block). ``vectors`` are the rank's own (localized) vectors; a missing pair
    hides nothing. Bm, Hm come from the vectors' shapes (1, 1 if all missing).
    """
    ref = next((np.asarray(x) for x in vectors if x is not None), None)
    bm, hm = (1, 1) if ref is None else (ref.shape[0], ref.shape[1])
    tk = -(-seq_k // block_k)
    out = np.zeros((bm, hm, tk), dtype=np.uint8)
    for b in range(bm):
        for h in range(hm):
            v = vectors_for(vectors, b, h)
            open_key = np.zeros(seq_k, dtype=bool)
            for r0 in range(0, seq_q, 4096):
                rows = np.arange(r0, min(r0 + 4096, seq_q))
                open_key |= ~dense_mask(*v, rows, seq_k).all(axis=0)
            for t in range(tk):
                out[b, h, t] = open_key[t * block_k:min((t + 1) * block_k, seq_k)].any()
    return out


def chunk_work(vectors, seq_k, chunk_start, chunk_len):
    """Open (row, key) pairs per mask row and chunk: int64 [Bm * Hm, C], the
    rows of chunk c being [chunk_start[c], chunk_start[c] + chunk_len[c])
    (dense truth, 4096 rows at a time)."""
    ref = next((np.asarray(x) for x in vectors if x is not None), None)
    bm, hm = (1, 1) if ref is None else (ref.shape[0], ref.shape[1])
    out = np.zeros((bm * hm, len(chunk_start)), dtype=np.int64)
    for b in range(bm):
        for h in range(hm):
            v = vectors_for(vectors, b, h)
            for c, (s0, ln) in enumerate(zip(chunk_start, chunk_len)):
                for r0 in range(int(s0), int(s0) + int(ln), 4096):
                    rows = np.arange(r0, min(r0 + 4096, int(s0) + int(ln)))
                    out[b * hm + h, c] += int((~dense_mask(*v, rows, seq_k)).sum())
    return out


def plan_loads(work, rank_of_chunk, num_ranks):
    """Per-rank load of an assignment (work summed over its chunks)."""
    loads = np.zeros(num_ranks, dtype=np.int64)
    for c, r in enumerate(rank_of_chunk):
        loads[r] += int(work[c])
    return loads


def best_plan_max(work, num_ranks):
    """Smallest possible maximum rank load with len(work) / num_ranks chunks
    per rank, by exhaustive search (tiny inputs only)."""
    work = [int(x) for x in work]
    per = len(work) // num_ranks
    best = [None]

    def rec(rest, loads):
        if not rest:
            m = max(loads)
            if best[0] is None or m < best[0]:
                best[0] = m
            return
        first, others = rest[0], rest[1:]
        # the group holding the lowest-index remaining chunk (no symmetric repeats)
        from itertools import combinations
        for comb in combinations(range(len(others)), per - 1):
            grp = [first] + [others[i] for i in comb]
            left = [x for i, x in enumerate(others) if i not in comb]
            rec(left, loads + [sum(work[g] for g in grp)])
    rec(list(range(len(work))), [])
    return best[0]


def _canonical(vec, seq_q, n_keys):
    lts, lte, uts, ute = vec
    if lts is None:
        lts = np.full(n_keys, seq_q, dtype=np.int64)
        lte = np.full(n_keys, seq_q, dtype=np.int64)
    if uts is None:
        uts = np.zeros(n_keys, dtype=np.int64)
        ute = np.zeros(n_keys, dtype=np.int64)
    return lts, lte, uts, ute


def tile_summary(vectors, seq_q, seq_k, block_k, b=0, h=0):
    """Per K tile: (min, max) of lts, lte, uts, ute over the tile's columns.

    Returns int64 [Tk, 8] ordered
    (min lts, max lts, min lte, max lte, min uts, max uts, min ute, max ute).
    """
    vec = _canonical(vectors_for(vectors, b, h), seq_q, seq_k)
    tk = -(-seq_k // block_k)
    out = np.zeros((tk, 8), dtype=np.int64)
    for t in range(tk):
        c = slice(t * block_k, min((t + 1) * block_k, seq_k))
        for i, x in enumerate(vec):
            out[t, 2 * i] = x[c].min()
            out[t, 2 * i + 1] = x[c].max()
    return out


def tile_classes(vectors, seq_q, seq_k, block_q, block_k, b=0, h=0):
    """Class map [Tq, Tk] (uint8) by the min/max rule."""
    s = tile_summary(vectors, seq_q, seq_k, block_k, b, h)
    tq = -(-seq_q // block_q)
    out = np.zeros((tq, s.shape[0]), dtype=np.uint8)
    for qt in range(tq):
        r0, r1 = qt * block_q, min((qt + 1) * block_q, seq_q)
        for kt in range(s.shape[0]):
            min_ls, max_ls, min_le, max_le, min_us, max_us, min_ue, max_ue = s[kt]
            covers_l = max_ls <= r0 and min_le >= r1
            covers_u = max_us <= r0 and min_ue >= r1
            misses_l = max_le <= r0 or min_ls >= r1
            misses_u = max_ue <= r0 or min_us >= r1
            if covers_l or covers_u:
                out[qt, kt] = SKIP
            elif misses_l and misses_u:
                out[qt, kt] = FULL
            else:
                out[qt, kt] = PARTIAL
    return out


def tile_classes_dense(vectors, seq_q, seq_k, block_q, block_k, b=0, h=0):
    """Dense-truth classes [Tq, Tk]: SKIP if every pair of the tile is masked,
    FULL if none is, PARTIAL otherwise."""
    vec = vectors_for(vectors, b, h)
    tq, tk = -(-seq_q // block_q), -(-seq_k // block_k)
    out = np.zeros((tq, tk), dtype=np.uint8)
    for qt in range(tq):
        rows = np.arange(qt * block_q, min((qt + 1) * block_q, seq_q))
        m = dense_mask(*vec, rows, seq_k)
        for kt in range(tk):
            t = m[:, kt * block_k:min((kt + 1) * block_k, seq_k)]
            out[qt, kt] = SKIP if t.all() else (FULL if not t.any() else PARTIAL)
    return out
