"""Python binding of libfmattn: the C entry points under the same names.

Argument marshalling only: tensors are checked for device, dtype and layout,
their pointers and strides are handed to the C ABI, and outputs / workspace
are allocated with torch (device memory and streams are torch's job here).
Every step of the computation runs in the HIP kernels.

Layout: q, o, do, dq are [B, Sq, H, D]; k, v, dk, dv are [B, Sk, H_kv, D]
with H_kv dividing H (grouped-query attention when H_kv < H); the last
dimension must be contiguous. lse is [B, H, Sq] float32. Mask vectors are
int32 [Bm, Hm, Sk] with the key axis contiguous (see ``Mask``).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import _lib as L

_DTYPES = {torch.bfloat16: L.FM_BF16, torch.float32: L.FM_FP32}


@dataclass
class Mask:
    """Column-sparse mask: for key j, rows lts[j] <= i < lte[j] or
    uts[j] <= i < ute[j] are masked. Each vector is an int32 device tensor
    [Bm, Hm, Sk] (key axis contiguous); a pair may be None (empty interval)."""
    lts: Optional[torch.Tensor]
    lte: Optional[torch.Tensor]
    uts: Optional[torch.Tensor]
    ute: Optional[torch.Tensor]

    @staticmethod
    def from_vectors(vectors: Sequence, device="cuda") -> "Mask":
        """Build from (lts, lte, uts, ute) arrays of shape [Bm, Hm, Sk] (numpy
        or torch; None allowed for a pair)."""
        out = []
        for x in vectors:
            if x is None:
                out.append(None)
                continue
            t = torch.as_tensor(x).to(torch.int32)
            if t.dim() == 1:
                t = t[None, None]
            out.append(t.contiguous().to(device))
        return Mask(*out)

    def first(self) -> torch.Tensor:
        for x in (self.lts, self.uts):
            if x is not None:
                return x
        raise ValueError("mask has no vectors; use empty intervals instead of both pairs None")

    @property
    def shape(self):
        return tuple(self.first().shape)

    def _c(self) -> L.fm_mask:
        ref = self.first()
        if ref.dim() != 3:
            raise ValueError("mask vectors must be [Bm, Hm, Sk]")
        for x in (self.lts, self.lte, self.uts, self.ute):
            if x is not None:
                if x.dtype != torch.int32 or not x.is_cuda:
                    raise ValueError("mask vectors must be int32 device tensors")
                if x.shape != ref.shape or x.stride() != ref.stride() or x.stride(2) != 1:
                    raise ValueError("mask vectors must share shape and strides, key axis contiguous")
        ptr = lambda x: None if x is None else x.data_ptr()
        return L.fm_mask(ptr(self.lts), ptr(self.lte), ptr(self.uts), ptr(self.ute),
                         ref.shape[0], ref.shape[1], ref.stride(0), ref.stride(1))


def _stream_obj(stream, device=None):
    """The torch stream the kernels go on: the current stream of `device` when
    `stream` is None, a torch stream as given, or a raw hipStream_t handle
    wrapped as an external stream."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _check_bshd(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, S, H, D]")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: head dimension must be contiguous")


def _same_device(ref: torch.Tensor, *named):
    for t, n in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{n} is on {t.device}, q on {ref.device}")


def _problem(q, k, v, o, scale) -> L.fm_problem:
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_bshd(t, n)
    _same_device(q, (k, "k"), (v, "v"), (o, "o"))
    if q.dtype not in _DTYPES or any(t.dtype != q.dtype for t in (k, v, o)):
        raise ValueError("q, k, v, o must share dtype bfloat16 or float32")
    B, Sq, H, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Sk, Hkv, D) or v.shape != (B, Sk, Hkv, D) or o.shape != (B, Sq, H, D):
        raise ValueError("shape mismatch between q, k, v, o")
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{Hkv} K/V heads do not divide {H} query heads")
    if scale is None:
        scale = D ** -0.5
    st = lambda t: (C.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    return L.fm_problem(B, H, Sq, Sk, D, _DTYPES[q.dtype], float(scale),
                        st(q), st(k), st(v), st(o), Hkv)


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    """E4M3 codes as a uint8 view (float8_e4m3fn tensors are viewed)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise ValueError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    return t


def _problem_fp8(q, k, v, o, scale) -> L.fm_problem:
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_bshd(t, n)
    _same_device(q, (k, "k"), (v, "v"), (o, "o"))
    if o.dtype != torch.bfloat16:
        raise ValueError("o must be bfloat16")
    B, Sq, H, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Sk, Hkv, D) or v.shape != (B, Sk, Hkv, D) or o.shape != (B, Sq, H, D):
        raise ValueError("shape mismatch between q, k, v, o")
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{Hkv} K/V heads do not divide {H} query heads")
    if scale is None:
        scale = D ** -0.5
    st = lambda t: (C.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))
    return L.fm_problem(B, H, Sq, Sk, D, L.FM_FP8_E4M3, float(scale), st(q), st(k), st(v), st(o), Hkv)


def fm_attn_fwd_fp8(q, k, v, descale, mask: "Mask", scale=None, o=None, lse=None, workspace=None, stream=None):
    """Masked attention forward on E4M3 inputs (uint8 codes or
    float8_e4m3fn tensors) with descale = (q, k, v) factors. Returns (o, lse),
    o in bfloat16."""
    q, k, v = _codes(q, "q"), _codes(k, "k"), _codes(v, "v")
    B, Sq, H, D = q.shape
    s = _stream_obj(stream, q.device)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, Sq):
            raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
        _same_device(q, (lse, "lse"))
        ds = [float(x) for x in descale]
        if len(ds) != 3:
            raise ValueError("descale must hold 3 factors (q, k, v)")
        prob = _problem_fp8(q, k, v, o, scale)
        m = mask._c()
        lib = L.load()
        n = C.c_size_t()
        L.check(lib.fm_workspace_size(C.byref(prob), C.byref(m), 0, C.byref(n)))
        ws, nws = _workspace(n.value, q.device, workspace)
        dsc = (C.c_float * 3)(*ds)
        L.check(lib.fm_attn_fwd_fp8(C.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), dsc, C.byref(m),
                                    o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nws, s.cuda_stream))
    return o, lse


def fm_workspace_size_fp8(q, k, v, mask: "Mask", scale=None) -> int:
    """Workspace bytes of fm_attn_fwd_fp8 (includes the V^T tile copy)."""
    q, k, v = _codes(q, "q"), _codes(k, "k"), _codes(v, "v")
    B, Sq, H, D = q.shape
    o = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q.device)
    prob = _problem_fp8(q, k, v, o, scale)
    m = mask._c()
    n = C.c_size_t()
    L.check(L.load().fm_workspace_size(C.byref(prob), C.byref(m), 0, C.byref(n)))
    return n.value


def fm_kernel_tile(head_dim: int, bwd: bool = False):
    """(block_q, block_k) of the forward or backward kernel."""
    bq, bk = C.c_int32(), C.c_int32()
    L.load().fm_kernel_tile(int(head_dim), int(bool(bwd)), C.byref(bq), C.byref(bk))
    return bq.value, bk.value


def fm_workspace_size(q, k, v, mask: Mask, with_bwd: bool, scale=None) -> int:
    o = q if q.dim() == 4 else None
    prob = _problem(q, k, v, o, scale)
    m = mask._c()
    n = C.c_size_t()
    L.check(L.load().fm_workspace_size(C.byref(prob), C.byref(m), int(bool(with_bwd)), C.byref(n)))
    return n.value


def fm_bwd_workspace_size_ds(q, k, v, mask: Mask, scale=None, stream=None) -> int:
    """Workspace bytes with which fm_attn_bwd stores dS and forms dQ from it
    (the count depends on the mask contents: classifies on the device and
    synchronizes the stream)."""
    prob = _problem(q, k, v, q, scale)
    m = mask._c()
    lib = L.load()
    n = C.c_size_t()
    L.check(lib.fm_workspace_size(C.byref(prob), C.byref(m), 1, C.byref(n)))
    s = _stream_obj(stream, q.device)
    with torch.cuda.stream(s):
        tmp = torch.empty(max(n.value, 256), dtype=torch.uint8, device=q.device)
        out = C.c_size_t()
        L.check(lib.fm_bwd_workspace_size_ds(C.byref(prob), C.byref(m), tmp.data_ptr(), tmp.numel(),
                                             s.cuda_stream, C.byref(out)))
    return out.value


def fm_bwd_dq_path(q, k, v, mask: Mask, workspace, scale=None, stream=None) -> bool:
    """True when the last fm_attn_bwd with these shapes, mask and workspace
    formed dQ from stored dS tiles, False when it recomputed S and dP (waits
    for the stream)."""
    prob = _problem(q, k, v, q, scale)
    m = mask._c()
    ws, nws = _workspace(0, q.device, workspace)
    flag = C.c_int32()
    L.check(L.load().fm_bwd_dq_path(C.byref(prob), C.byref(m), ws.data_ptr(), nws,
                                    _stream_obj(stream, q.device).cuda_stream, C.byref(flag)))
    return bool(flag.value)


def _workspace(nbytes: int, device, workspace):
    """(tensor, byte count) of the workspace: the caller's (a contiguous
    device tensor on `device`, any dtype; its whole storage counts) or a new
    uint8 one. Call it with the launch stream current, so that a temporary
    workspace is recycled only by work ordered after the launch."""
    if workspace is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return ws, ws.numel()
    if not workspace.is_cuda or workspace.device != torch.device(device):
        raise ValueError(f"workspace must be a device tensor on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace, workspace.numel() * workspace.element_size()


def fm_tile_classify(mask: Mask, seq_q: int, seq_k: int, block_q: int, block_k: int,
                     transposed: bool = False, stream=None):
    """Tile summaries int32 [Bm, Hm, Tk, 8] and classes uint8 [Bm, Hm, Tq, Tk]
    (or [Bm, Hm, Tk, Tq] when transposed)."""
    m = mask._c()
    bm, hm = m.batch, m.heads
    tq, tk = -(-seq_q // block_q), -(-seq_k // block_k)
    dev = mask.first().device
    s = _stream_obj(stream, dev)
    with torch.cuda.stream(s):
        summary = torch.empty((bm, hm, tk, 8), dtype=torch.int32, device=dev)
        shape = (bm, hm, tk, tq) if transposed else (bm, hm, tq, tk)
        classes = torch.empty(shape, dtype=torch.uint8, device=dev)
        L.check(L.load().fm_tile_classify(C.byref(m), int(seq_q), int(seq_k), int(block_q), int(block_k),
                                          int(bool(transposed)), summary.data_ptr(), classes.data_ptr(),
                                          s.cuda_stream))
    return summary, classes


def fm_attn_fwd(q, k, v, mask: Mask, scale=None, o=None, lse=None, workspace=None, stream=None):
    """Masked attention forward. Returns (o, lse)."""
    s = _stream_obj(stream, q.device)
    with torch.cuda.stream(s):
        if o is None:
            o = torch.empty_like(q)
        B, Sq, H, _ = q.shape
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, Sq):
            raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
        _same_device(q, (lse, "lse"))
        prob = _problem(q, k, v, o, scale)
        m = mask._c()
        lib = L.load()
        n = C.c_size_t()
        L.check(lib.fm_workspace_size(C.byref(prob), C.byref(m), 0, C.byref(n)))
        ws, nws = _workspace(n.value, q.device, workspace)
        L.check(lib.fm_attn_fwd(C.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), C.byref(m),
                                o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nws, s.cuda_stream))
    return o, lse


def fm_attn_fwd_noalloc(q, k, v, mask: Mask, o, lse, scale=None, stream=None):
    """The forward through the entry point that allocates nothing and takes
    no workspace (its scratch is a fixed device array of the library, shared
    by every call on the GPU). o and lse are the caller's; returns them."""
    B, Sq, H, _ = q.shape
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, Sq):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    _same_device(q, (lse, "lse"))
    prob = _problem(q, k, v, o, scale)
    m = mask._c()
    L.check(L.load().fm_attn_fwd_noalloc(C.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), C.byref(m),
                                         o.data_ptr(), lse.data_ptr(), _stream_obj(stream, q.device).cuda_stream))
    return o, lse


def fm_attn_bwd(q, k, v, o, lse, do, mask: Mask, scale=None, dq=None, dk=None, dv=None,
                workspace=None, stream=None):
    """Masked attention backward. Returns (dq, dk, dv)."""
    prob = _problem(q, k, v, o, scale)
    _check_bshd(do, "do")
    if do.shape != o.shape or do.stride() != o.stride() or do.dtype != o.dtype:
        raise ValueError("do must match o in shape, strides and dtype")
    B, Sq, H, _ = q.shape
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, H, Sq):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    s = _stream_obj(stream, q.device)
    with torch.cuda.stream(s):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        for g, ref, nm in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
            if g.shape != ref.shape or g.stride() != ref.stride() or g.dtype != ref.dtype:
                raise ValueError(f"{nm} must match its primal in shape, strides and dtype")
        _same_device(q, (do, "do"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv"))
        m = mask._c()
        lib = L.load()
        n = C.c_size_t()
        L.check(lib.fm_workspace_size(C.byref(prob), C.byref(m), 1, C.byref(n)))
        ws, nws = _workspace(n.value, q.device, workspace)
        L.check(lib.fm_attn_bwd(C.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), do.data_ptr(), C.byref(m), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), ws.data_ptr(), nws, s.cuda_stream))
    return dq, dk, dv


def fm_mask_localize(mask: Mask, seq_q_global: int, chunk_start, chunk_len, stream=None) -> Mask:
    """Localize the bound vectors to a rank holding the listed chunks of the
    global query axis (ascending, non-overlapping). Returns a new Mask with
    contiguous [Bm, Hm, Sk] vectors."""
    m = mask._c()
    ref = mask.first()
    bm, hm, sk = ref.shape
    starts = [int(x) for x in chunk_start]
    lens = [int(x) for x in chunk_len]
    if len(starts) != len(lens):
        raise ValueError("chunk_start and chunk_len differ in length")
    nck = len(starts)
    cs = (C.c_int32 * max(nck, 1))(*starts)
    cl = (C.c_int32 * max(nck, 1))(*lens)
    s = _stream_obj(stream, ref.device)
    with torch.cuda.stream(s):
        out = [None if (i < 2 and mask.lts is None) or (i >= 2 and mask.uts is None)
               else torch.empty((bm, hm, sk), dtype=torch.int32, device=ref.device) for i in range(4)]
        ptrs = (C.c_void_p * 4)(*[None if t is None else t.data_ptr() for t in out])
        L.check(L.load().fm_mask_localize(C.byref(m), int(sk), int(seq_q_global), cs, cl, nck, ptrs,
                                          s.cuda_stream))
    return Mask(*out)


def fm_chunk_work(mask: Mask, seq_q_global: int, chunk_start, chunk_len, stream=None) -> torch.Tensor:
    """Open (row, key) pairs per mask row and chunk of the global query axis:
    int64 [Bm * Hm, C] on the mask's device."""
    m = mask._c()
    ref = mask.first()
    bm, hm, sk = ref.shape
    starts = [int(x) for x in chunk_start]
    lens = [int(x) for x in chunk_len]
    if len(starts) != len(lens):
        raise ValueError("chunk_start and chunk_len differ in length")
    nck = len(starts)
    cs = (C.c_int32 * max(nck, 1))(*starts)
    cl = (C.c_int32 * max(nck, 1))(*lens)
    s = _stream_obj(stream, ref.device)
    with torch.cuda.stream(s):
        work = torch.empty((bm * hm, nck), dtype=torch.int64, device=ref.device)
        L.check(L.load().fm_chunk_work(C.byref(m), int(sk), int(seq_q_global), cs, cl, nck, work.data_ptr(),
                                       s.cuda_stream))
    return work


def fm_cp_plan(chunk_work, num_ranks: int):
    """Chunk -> rank plan (host): (rank_of_chunk list, largest rank load)."""
    w = [int(x) for x in chunk_work]
    n = len(w)
    arr = (C.c_int64 * max(n, 1))(*w)
    out = (C.c_int32 * max(n, 1))()
    mx = C.c_int64()
    L.check(L.load().fm_cp_plan(arr, n, int(num_ranks), out, C.byref(mx)))
    return list(out[:n]), mx.value


def fm_kv_transfer_set(mask: Mask, seq_q: int, block_k: int, with_count: bool = True, stream=None):
    """Mask-pruned K/V transfer set of a rank whose own (localized) vectors
    are `mask`, over its seq_q rows: (need uint8 [Bm, Hm, Tk], count int32
    [Bm, Hm] or None)."""
    m = mask._c()
    ref = mask.first()
    bm, hm, sk = ref.shape
    tk = -(-int(sk) // int(block_k))
    s = _stream_obj(stream, ref.device)
    with torch.cuda.stream(s):
        need = torch.empty((bm, hm, tk), dtype=torch.uint8, device=ref.device)
        count = torch.empty((bm, hm), dtype=torch.int32, device=ref.device) if with_count else None
        L.check(L.load().fm_kv_transfer_set(C.byref(m), int(seq_q), int(sk), int(block_k), need.data_ptr(),
                                            None if count is None else count.data_ptr(), s.cuda_stream))
    return need, count


def fm_profile_begin(max_launches: int = 4096) -> None:
    L.check(L.load().fm_profile_begin(int(max_launches)))


def fm_profile_end() -> dict:
    """{stage: (total_ms, launches)} for the launches since fm_profile_begin."""
    ms = (C.c_float * L.FM_NUM_STAGES)()
    cnt = (C.c_int32 * L.FM_NUM_STAGES)()
    L.check(L.load().fm_profile_end(ms, cnt))
    return {name: (ms[i], cnt[i]) for i, name in enumerate(L.STAGES)}
