"""Helpers for the GPU parity tests: device transfer and the float bar.

The bar for bf16 (and fp32-rounded-to-bf16) inputs with fp32 accumulation:
max-abs error <= 2e-2 AND relative L2 error <= 1e-2 against the float64
oracle, on every compared tensor.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

MAX_ABS = 2e-2
REL_L2 = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_mask(vectors, device="cuda"):
    from masked_tiled_attention_amd import Mask
    return Mask.from_vectors(vectors, device)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "finite / non-finite pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), "non-finite values differ"
    if not fin.any():
        return 0.0, 0.0
    d = got[fin] - ref[fin]
    max_abs = float(np.max(np.abs(d)))
    nref = float(np.linalg.norm(ref[fin]))
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


BF16_ROUND = 2.0 ** -8   # relative rounding of a bf16 output (half an ulp is <= 2^-9)


def assert_close(got, ref, name, max_abs=MAX_ABS, rel_l2=REL_L2, out_round=0.0):
    """The bar: |got - ref| <= max_abs (+ out_round * |ref| where the exact
    value is too large for the output dtype to hold it within max_abs) on
    every element, and relative L2 error <= rel_l2."""
    a, r = metrics(got, ref)
    log(f"  {name}: max_abs={a:.3e} rel_l2={r:.3e}")
    if out_round:
        g = np.asarray(got, dtype=np.float64)
        f = np.asarray(ref, dtype=np.float64)
        fin = np.isfinite(f)
        excess = np.max(np.abs(g[fin] - f[fin]) - (max_abs + out_round * np.abs(f[fin])), initial=-1.0)
        assert excess <= 0 and r <= rel_l2, \
            f"{name}: error beyond max_abs + output rounding by {excess:.3e}, rel_l2 {r:.3e}"
        return
    assert a <= max_abs and r <= rel_l2, f"{name}: max_abs {a:.3e} (<= {max_abs}), rel_l2 {r:.3e} (<= {rel_l2})"
