"""The named synthetic workloads (input construction only).

Each workload is one mask family at one shape, with seeded Q/K/V/dO. The
mask families are the structural masks the FlashMask-3 news page lists in its
problem paragraph (document, prefix-LM, share-question, sliding window);
block-sparse masks are not built. The shapes and length recipes are:

  c1_tiny_causal        B1 H1 S256    d64  fp32, causal, forward only
  c2_doc_causal_4k      B2 H16 S4096  d128 bf16, document-causal, lengths U[64,1024] per batch row
  c3a_window_32k        B1 H8 S32768  d128 bf16, sliding-window causal, window 4096
  c3b_prefix_lm_32k     B1 H8 S32768  d128 bf16, prefix-LM, bidirectional prefix 8192
  c3c_share_question_32k B1 H8 S32768 d128 bf16, 4096-token question + 6 answers
  c4_doc_causal_128k    B1 H4 S131072 d128 bf16, document-causal, log-normal lengths
  c4_causal_128k        B1 H4 S131072 d128 bf16, plain causal (dense-tile reference point)
  c5_cp_rank3_of_8      global S65536 document-causal (log-normal lengths); queries of
                        context-parallel rank 3 of 8 under dual-chunk assignment (8192 rows),
                        keys/values over all 65536 positions; H8 d128 bf16

Mask lengths come from ``numpy.random.default_rng(seed + 5)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from . import masks as M
from . import tensors as T


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    heads: int
    seq_q: int
    seq_k: int
    head_dim: int
    dtype: torch.dtype
    backward: bool
    vectors: tuple                 # (lts, lte, uts, ute), each int32 [Bm, Hm, Sk]
    scale: float
    seed: int
    q: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    do: Optional[torch.Tensor] = None
    # context-parallel rank share only
    seq_q_global: Optional[int] = None
    global_vectors: Optional[tuple] = None
    chunk_start: Optional[np.ndarray] = None
    chunk_len: Optional[np.ndarray] = None
    local_rows: Optional[np.ndarray] = None
    description: str = ""


NAMES = (
    "c1_tiny_causal",
    "c2_doc_causal_4k",
    "c3a_window_32k",
    "c3b_prefix_lm_32k",
    "c3c_share_question_32k",
    "c4_doc_causal_128k",
    "c4_causal_128k",
    "c5_cp_rank3_of_8",
)


def _one(v):
    """[Sk] vectors -> [1, 1, Sk]."""
    return tuple(np.ascontiguousarray(x[None, None, :]) for x in v)


def _lognormal_scaled(rng, n, full_n, full_hi):
    """Log-normal document lengths (median 4096, sigma 1.0, clipped to
    [128, full_hi]) at the full length ``full_n``; at a reduced length the
    median and clip bounds shrink by n / full_n."""
    f = n / full_n
    return M.lognormal_doc_lengths(rng, n, median=4096.0 * f, sigma=1.0,
                                   lo=max(1, int(round(128 * f))),
                                   hi=max(2, int(round(full_hi * f))))


def mask_vectors(name: str, seed: int, seq: Optional[int] = None):
    """Bound vectors [Bm, Hm, Sk] of a named workload's mask family.

    ``seq`` overrides the sequence length (smaller parity cases use the same
    recipe at a reduced size; window/prefix/question sizes scale with it).
    """
    rng = np.random.default_rng(seed + 5)
    if name == "c1_tiny_causal":
        n = seq or 256
        return _one(M.causal(n))
    if name == "c2_doc_causal_4k":
        n = seq or 4096
        per_b = []
        for _ in range(2):
            per_b.append([M.document_causal(M.uniform_doc_lengths(rng, n, 64, 1024))])
        return M.stack(per_b)
    if name == "c3a_window_32k":
        n = seq or 32768
        return _one(M.sliding_window_causal(n, max(1, n // 8)))
    if name == "c3b_prefix_lm_32k":
        n = seq or 32768
        return _one(M.prefix_lm(n, n // 4))
    if name == "c3c_share_question_32k":
        n = seq or 32768
        qlen = n // 8
        return _one(M.share_question(qlen, M.answer_lengths(rng, n - qlen, 6)))
    if name == "c4_doc_causal_128k":
        n = seq or 131072
        return _one(M.document_causal(_lognormal_scaled(rng, n, 131072, 65536)))
    if name == "c4_causal_128k":
        n = seq or 131072
        return _one(M.causal(n))
    if name == "c5_cp_rank3_of_8":
        n = seq or 65536
        return _one(M.document_causal(_lognormal_scaled(rng, n, 65536, 65536)))
    raise KeyError(name)


def build(name: str, seed: int = 0, tensors: bool = True, seq: Optional[int] = None,
          heads: Optional[int] = None) -> Workload:
    """Build a named workload (vectors always; Q/K/V/dO when ``tensors``)."""
    if name not in NAMES:
        raise KeyError(name)
    vec = mask_vectors(name, seed, seq)
    spec = {
        "c1_tiny_causal": (1, 1, 64, torch.float32, False),
        "c2_doc_causal_4k": (2, 16, 128, torch.bfloat16, False),
        "c3a_window_32k": (1, 8, 128, torch.bfloat16, True),
        "c3b_prefix_lm_32k": (1, 8, 128, torch.bfloat16, True),
        "c3c_share_question_32k": (1, 8, 128, torch.bfloat16, True),
        "c4_doc_causal_128k": (1, 4, 128, torch.bfloat16, True),
        "c4_causal_128k": (1, 4, 128, torch.bfloat16, True),
        "c5_cp_rank3_of_8": (1, 8, 128, torch.bfloat16, True),
    }[name]
    batch, h, d, dtype, bwd = spec
    if heads is not None:
        h = heads
    sk = vec[0].shape[-1]
    w = Workload(name=name, batch=batch, heads=h, seq_q=sk, seq_k=sk, head_dim=d,
                 dtype=dtype, backward=bwd, vectors=vec, scale=1.0 / math.sqrt(d), seed=seed)
    if name == "c5_cp_rank3_of_8":
        degree, rank = 8, 3
        starts, lens = M.dual_chunk(sk, degree, rank)
        w.seq_q_global = sk
        w.global_vectors = vec
        w.vectors = None        # produced by localization
        w.chunk_start, w.chunk_len = starts, lens
        w.local_rows = np.concatenate([np.arange(s, s + l) for s, l in zip(starts, lens)])
        w.seq_q = int(lens.sum())
    if tensors:
        if name == "c5_cp_rank3_of_8":
            qg = T.randn("q", (batch, sk, h, d), seed, dtype)
            w.q = qg[:, torch.from_numpy(w.local_rows)].contiguous()
            w.k = T.randn("k", (batch, sk, h, d), seed, dtype)
            w.v = T.randn("v", (batch, sk, h, d), seed, dtype)
            if bwd:
                w.do = T.randn("do", (batch, w.seq_q, h, d), seed, dtype)
        else:
            out = T.qkv(batch, w.seq_q, sk, h, d, seed, dtype, with_do=bwd)
            w.q, w.k, w.v = out[:3]
            if bwd:
                w.do = out[3]
    return w
