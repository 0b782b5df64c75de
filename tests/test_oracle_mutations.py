"""Planted mistakes in the oracle (CPU only): each must make some pin fail.

Every mutation is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one, the tempting wrong localization formula, a
per-block normalisation) written into a copy of one oracle function and
patched in for the duration of the test.
"""
import numpy as np
import pytest

import pins
from oracle import attention as OA
from oracle import fp8 as OF
from oracle import masks as OM

F64 = np.float64


def _fwd_factory(variant):
    def rows_forward(qrows, k, v, maskrows, scale):
        s = (qrows @ k.T) if variant == "no_scale" else scale * (qrows @ k.T)
        if variant == "inverted_mask":
            s[~maskrows] = -np.inf
        else:
            s[maskrows] = -np.inf
        open_any = ~maskrows.all(axis=1)
        m = np.where(open_any, np.max(s, axis=1), 0.0)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        o = np.zeros((qrows.shape[0], v.shape[1]))
        lse = np.full(qrows.shape[0], -np.inf)
        if variant == "block_normalised":
            # normalise each block of 4 keys on its own and add the blocks
            acc = np.zeros_like(o)
            for c0 in range(0, s.shape[1], 4):
                pb = p[:, c0:c0 + 4]
                lb = pb.sum(axis=1)
                ok = open_any & (lb > 0)
                acc[ok] += (pb[ok] @ v[c0:c0 + 4]) / lb[ok, None]
            o[open_any] = acc[open_any]
        elif variant == "no_normalise":
            o[open_any] = p[open_any] @ v
        else:
            o[open_any] = (p[open_any] @ v) / l[open_any, None]
        if variant == "lse_drops_max":
            lse[open_any] = np.log(l[open_any])
        else:
            lse[open_any] = m[open_any] + np.log(l[open_any])
        return o, lse
    return rows_forward


def _dense_factory(variant):
    def dense_mask(lts, lte, uts, ute, rows, n_keys=None):
        rows = np.asarray(rows, dtype=np.int64)[:, None]
        if n_keys is None:
            n_keys = len(next(x for x in (lts, lte, uts, ute) if x is not None))
        m = np.zeros((rows.shape[0], n_keys), dtype=bool)
        if lts is not None:
            if variant == "closed_end":
                m |= (np.asarray(lts)[None, :] <= rows) & (rows <= np.asarray(lte)[None, :])
            else:
                m |= (np.asarray(lts)[None, :] <= rows) & (rows < np.asarray(lte)[None, :])
        if uts is not None and variant != "drop_upper":
            m |= (np.asarray(uts)[None, :] <= rows) & (rows < np.asarray(ute)[None, :])
        return m
    return dense_mask


def _bwd_factory(variant):
    def backward(q, k, v, do, vectors, scale, block=1024):
        q, k, v, do = (np.asarray(a, dtype=F64) for a in (q, k, v, do))
        B, Sq, H, _ = q.shape
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                vec = OA.vectors_for(vectors, b, h)
                kb, vb = k[b, :, h], v[b, :, h]
                for r0 in range(0, Sq, block):
                    rows = np.arange(r0, min(r0 + block, Sq))
                    p = OA._rows_probs(q[b, rows, h], kb, OA.dense_mask(*vec, rows, kb.shape[0]), scale)
                    dob = do[b, rows, h]
                    dp = dob @ vb.T
                    dterm = (p * dp).sum(axis=1, keepdims=True)
                    if variant == "drop_d":
                        ds = p * dp
                    elif variant == "sign":
                        ds = p * (dterm - dp)
                    else:
                        ds = p * (dp - dterm)
                    dq[b, rows, h] = scale * (ds @ kb)
                    if variant == "dk_no_scale":
                        dk[b, :, h] += ds.T @ q[b, rows, h]
                    elif variant == "dk_uses_k":
                        dk[b, :, h] += scale * (ds.T @ (q[b, rows, h] + 0.5 * kb[rows % kb.shape[0]]))
                    else:
                        dk[b, :, h] += scale * (ds.T @ q[b, rows, h])
                    if variant == "dv_uses_ds":
                        dv[b, :, h] += ds.T @ dob
                    else:
                        dv[b, :, h] += p.T @ dob
        return dq, dk, dv
    return backward


def _localize_factory(variant):
    def localize(vectors, chunk_start, chunk_len):
        out = []
        for x in vectors:
            if x is None:
                out.append(None)
                continue
            x = np.asarray(x, dtype=np.int64)
            if variant == "side_right":
                rows = OM.local_rows(chunk_start, chunk_len)
                out.append(np.searchsorted(rows, x, side="right").astype(np.int32))
            else:   # the tempting form: max over chunks of clamp-then-shift
                best = np.zeros_like(x)
                off = 0
                for s, l in zip(chunk_start, chunk_len):
                    best = np.maximum(best, np.clip(x, s, s + l) - s + off)
                    off += l
                out.append(best.astype(np.int32))
        return tuple(out)
    return localize


def _classes_factory(variant):
    orig = OM.tile_classes

    def tile_classes(vectors, seq_q, seq_k, block_q, block_k, b=0, h=0):
        s = OM.tile_summary(vectors, seq_q, seq_k, block_k, b, h)
        tq = -(-seq_q // block_q)
        out = np.zeros((tq, s.shape[0]), dtype=np.uint8)
        for qt in range(tq):
            r0 = qt * block_q
            r1 = r0 + block_q if variant == "no_ragged_clip" else min(r0 + block_q, seq_q)
            for kt in range(s.shape[0]):
                min_ls, max_ls, min_le, max_le, min_us, max_us, min_ue, max_ue = s[kt]
                covers_l = max_ls <= r0 and min_le >= r1
                covers_u = max_us <= r0 and min_ue >= r1
                misses_l = max_le <= r0 or min_ls >= r1
                misses_u = max_ue <= r0 or min_us >= r1
                if variant == "full_or":
                    full = misses_l or misses_u
                else:
                    full = misses_l and misses_u
                if variant == "skip_uses_min_start":
                    covers_l = min_ls <= r0 and min_le >= r1
                if covers_l or covers_u:
                    out[qt, kt] = 0
                elif full:
                    out[qt, kt] = 2
                else:
                    out[qt, kt] = 1
        return out
    del orig
    return tile_classes


def _transfer_factory(variant):
    def transfer_set(vectors, seq_q, seq_k, block_k):
        ref = next((np.asarray(x) for x in vectors if x is not None), None)
        bm, hm = (1, 1) if ref is None else (ref.shape[0], ref.shape[1])
        tk = -(-seq_k // block_k)
        out = np.zeros((bm, hm, tk), dtype=np.uint8)
        for b in range(bm):
            for h in range(hm):
                v = OA.vectors_for(vectors, b, h)
                m = OA.dense_mask(*v, np.arange(seq_q), seq_k)
                if variant == "any_masked":
                    key = m.any(axis=0)
                else:
                    key = ~m.all(axis=0)
                for t in range(tk):
                    hi = (t + 1) * block_k + (1 if variant == "tile_overlap" else 0)
                    out[b, h, t] = key[t * block_k:min(hi, seq_k)].any()
        return out
    return transfer_set


def _chunk_work_factory(variant):
    def chunk_work(vectors, seq_k, chunk_start, chunk_len):
        ref = next((np.asarray(x) for x in vectors if x is not None), None)
        bm, hm = (1, 1) if ref is None else (ref.shape[0], ref.shape[1])
        out = np.zeros((bm * hm, len(chunk_start)), dtype=np.int64)
        for b in range(bm):
            for h in range(hm):
                v = OA.vectors_for(vectors, b, h)
                for c, (s0, ln) in enumerate(zip(chunk_start, chunk_len)):
                    end = int(s0) + int(ln) + (1 if variant == "chunk_end_inclusive" else 0)
                    m = OA.dense_mask(*v, np.arange(int(s0), end), seq_k)
                    out[b * hm + h, c] = int(m.sum() if variant == "counts_masked" else (~m).sum())
        return out
    return chunk_work



def _e4m3_factory(variant):
    def e4m3_decode(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = (c & 0x7).astype(F64)
        bias = 8.0 if variant == "bias_8" else 7.0
        normal = (1.0 + m / 8.0) * np.exp2(e.astype(F64) - bias)
        sub = (1.0 + m / 8.0) * 2.0 ** -6 if variant == "subnormal_implicit_one" else (m / 8.0) * 2.0 ** -6
        val = np.where(e == 0, sub, normal)
        val = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
        return sign * val
    return e4m3_decode


def _fp8_forward_factory(variant):
    def forward(q8, k8, v8, descales, vectors, scale, block=1024):
        dq, dk, dv = descales
        if variant == "v_descale_dropped":
            dv = 1.0
        if variant == "k_descale_for_v":
            dv = dk
        return OA.forward(OF.dequantize(q8, dq), OF.dequantize(k8, dk), OF.dequantize(v8, dv), vectors, scale,
                          block=block)
    return forward

def _kv_head_mod(q_heads, kv_heads, h):
    return h % kv_heads


MUTATIONS = {
    "e4m3_bias_8": (OF, "e4m3_decode", _e4m3_factory("bias_8")),
    "e4m3_subnormal_implicit_one": (OF, "e4m3_decode", _e4m3_factory("subnormal_implicit_one")),
    "fp8_v_descale_dropped": (OF, "forward", _fp8_forward_factory("v_descale_dropped")),
    "fp8_k_descale_for_v": (OF, "forward", _fp8_forward_factory("k_descale_for_v")),
    "gqa_head_modulo": (OA, "kv_head", _kv_head_mod),
    "chunk_work_end_inclusive": (OM, "chunk_work", _chunk_work_factory("chunk_end_inclusive")),
    "chunk_work_counts_masked": (OM, "chunk_work", _chunk_work_factory("counts_masked")),
    "transfer_any_masked": (OM, "transfer_set", _transfer_factory("any_masked")),
    "transfer_tile_overlap": (OM, "transfer_set", _transfer_factory("tile_overlap")),
    "fwd_no_scale": (OA, "_rows_forward", _fwd_factory("no_scale")),
    "fwd_inverted_mask": (OA, "_rows_forward", _fwd_factory("inverted_mask")),
    "fwd_block_normalised": (OA, "_rows_forward", _fwd_factory("block_normalised")),
    "fwd_no_normalise": (OA, "_rows_forward", _fwd_factory("no_normalise")),
    "fwd_lse_drops_max": (OA, "_rows_forward", _fwd_factory("lse_drops_max")),
    "mask_closed_end": (OA, "dense_mask", _dense_factory("closed_end")),
    "mask_drop_upper": (OA, "dense_mask", _dense_factory("drop_upper")),
    "bwd_drop_d": (OA, "backward", _bwd_factory("drop_d")),
    "bwd_sign": (OA, "backward", _bwd_factory("sign")),
    "bwd_dk_no_scale": (OA, "backward", _bwd_factory("dk_no_scale")),
    "bwd_dk_wrong_operand": (OA, "backward", _bwd_factory("dk_uses_k")),
    "bwd_dv_uses_ds": (OA, "backward", _bwd_factory("dv_uses_ds")),
    "localize_side_right": (OM, "localize", _localize_factory("side_right")),
    "localize_clamp_then_shift": (OM, "localize", _localize_factory("tempting")),
    "classes_full_or": (OM, "tile_classes", _classes_factory("full_or")),
    "classes_no_ragged_clip": (OM, "tile_classes", _classes_factory("no_ragged_clip")),
    "classes_skip_min_start": (OM, "tile_classes", _classes_factory("skip_uses_min_start")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
