"""Seeded synthetic Q/K/V/dO tensors (input construction only).

Each tensor comes from its own CPU generator seeded with ``seed + t``
(t = 1, 2, 3, 4 for Q, K, V, dO), drawn i.i.d. N(0, 1) in float32 and then
cast to the requested dtype. The layout is [batch, seq, heads, head_dim]
with head_dim contiguous.
"""
from __future__ import annotations

import torch

_OFFSETS = {"q": 1, "k": 2, "v": 3, "do": 4}


def randn(name: str, shape, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(int(seed) + _OFFSETS[name])
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dtype)


def qkv(batch, seq_q, seq_k, heads, head_dim, seed, dtype=torch.bfloat16, with_do=False):
    q = randn("q", (batch, seq_q, heads, head_dim), seed, dtype)
    k = randn("k", (batch, seq_k, heads, head_dim), seed, dtype)
    v = randn("v", (batch, seq_k, heads, head_dim), seed, dtype)
    if not with_do:
        return q, k, v
    do = randn("do", (batch, seq_q, heads, head_dim), seed, dtype)
    return q, k, v, do


def fp8_codes(name: str, shape, seed: int, gain: float = 64.0) -> torch.Tensor:
    """uint8 codes of the OCP E4M3 format (torch.float8_e4m3fn) for
    N(0, 1) draws (clipped to +-6.5) times ``gain``; the matching descale
    factor is 1 / gain. With gain <= 64 every product stays below 448, the
    format's largest finite value."""
    x = randn(name, shape, seed, torch.float32).clamp_(-6.5, 6.5) * float(gain)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)
