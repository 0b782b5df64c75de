"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments with the documented status
before launching anything."""
import ctypes as C
import os
import re

import pytest

from masked_tiled_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fm_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fm_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = L.load()
    declared = _declared()
    assert set(declared) == set(L.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_kernel_tile():
    lib = L.load()
    q, k = C.c_int32(), C.c_int32()
    for d in (64, 128):
        lib.fm_kernel_tile(d, 0, C.byref(q), C.byref(k))
        assert (q.value, k.value) == (128, 64)
        lib.fm_kernel_tile(d, 1, C.byref(q), C.byref(k))
        assert (q.value, k.value) == (64, 128)
    lib.fm_kernel_tile(96, 0, C.byref(q), C.byref(k))
    assert (q.value, k.value) == (0, 0)


FAKE = 0x10000  # an aligned address that is never dereferenced: every case fails validation first


def _problem(B=1, H=2, Sq=100, Sk=120, D=128, dtype=L.FM_BF16, scale=0.1, strides=None, hkv=0):
    st = strides or (Sq * H * D, H * D, D)
    nk = hkv or H
    sk = (Sk * nk * D, nk * D, D)
    arr = lambda s: (C.c_int64 * 3)(*s)
    return L.fm_problem(B, H, Sq, Sk, D, dtype, scale, arr(st), arr(sk), arr(sk), arr(st), hkv)


def _mask(bm=1, hm=1, lower=True, upper=True, one_null=False):
    lts = FAKE if lower else None
    lte = (None if one_null else FAKE) if lower else None
    uts = FAKE if upper else None
    ute = FAKE if upper else None
    return L.fm_mask(lts, lte, uts, ute, bm, hm, 0, 0)


def _fwd(prob, mask, ws_bytes=1 << 30, ptrs=None):
    lib = L.load()
    q, k, v, o, lse = ptrs or (FAKE,) * 5
    return lib.fm_attn_fwd(C.byref(prob) if prob is not None else None, q, k, v,
                           C.byref(mask) if mask is not None else None, o, lse, FAKE, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("null_problem", L.FM_ERR_INVALID_ARGUMENT),
    ("null_mask", L.FM_ERR_INVALID_ARGUMENT),
    ("head_dim_96", L.FM_ERR_UNSUPPORTED),
    ("zero_seq", L.FM_ERR_INVALID_ARGUMENT),
    ("bad_scale", L.FM_ERR_INVALID_ARGUMENT),
    ("bad_dtype", L.FM_ERR_INVALID_ARGUMENT),
    ("misaligned_stride", L.FM_ERR_INVALID_ARGUMENT),
    ("mask_batch_3_of_2", L.FM_ERR_INVALID_ARGUMENT),
    ("mask_one_null", L.FM_ERR_INVALID_ARGUMENT),
    ("null_q", L.FM_ERR_INVALID_ARGUMENT),
    ("misaligned_q", L.FM_ERR_INVALID_ARGUMENT),
    ("small_workspace", L.FM_ERR_WORKSPACE),
    ("kv_heads_not_dividing", L.FM_ERR_INVALID_ARGUMENT),
    ("kv_heads_negative", L.FM_ERR_INVALID_ARGUMENT),
])
def test_fwd_rejects(case, expect):
    prob, mask, ws, ptrs = _problem(), _mask(), 1 << 30, None
    if case == "null_problem":
        prob = None
    elif case == "null_mask":
        mask = None
    elif case == "head_dim_96":
        prob = _problem(D=96, strides=(100 * 2 * 96, 2 * 96, 96))
    elif case == "zero_seq":
        prob = _problem(Sq=0)
    elif case == "bad_scale":
        prob = _problem(scale=-1.0)
    elif case == "bad_dtype":
        prob = _problem(dtype=7)
    elif case == "misaligned_stride":
        prob = _problem(strides=(100 * 2 * 128, 2 * 128 + 4, 128))
    elif case == "mask_batch_3_of_2":
        prob, mask = _problem(B=2), _mask(bm=3)
    elif case == "mask_one_null":
        mask = _mask(one_null=True)
    elif case == "null_q":
        ptrs = (0, FAKE, FAKE, FAKE, FAKE)
    elif case == "misaligned_q":
        ptrs = (FAKE + 8, FAKE, FAKE, FAKE, FAKE)
    elif case == "small_workspace":
        ws = 16
    elif case == "kv_heads_not_dividing":
        prob = _problem(H=6, hkv=4)
    elif case == "kv_heads_negative":
        prob = _problem(hkv=-1)
    assert _fwd(prob, mask, ws, ptrs) == expect
    assert L.load().fm_last_error()


def test_workspace_size_grows_with_backward():
    lib = L.load()
    prob, mask = _problem(B=2, H=4, Sq=1000, Sk=1000), _mask()
    a, b = C.c_size_t(), C.c_size_t()
    assert lib.fm_workspace_size(C.byref(prob), C.byref(mask), 0, C.byref(a)) == L.FM_OK
    assert lib.fm_workspace_size(C.byref(prob), C.byref(mask), 1, C.byref(b)) == L.FM_OK
    # the backward holds two class maps and D (B*H*Sq fp32)
    assert b.value >= 2 * 4 * 1000 * 4
    assert 0 < a.value < b.value


def test_fwd_noalloc_rejects_problems_beyond_its_scratch():
    """The allocation-free forward holds 64 MiB of scratch: 128 per-head
    masks over 65,536 x 65,536 need a 64 MiB class map alone, so the call
    fails with FM_ERR_WORKSPACE before touching the device."""
    lib = L.load()
    prob = _problem(B=1, H=128, Sq=65536, Sk=65536)
    mask = _mask(hm=128)
    rc = lib.fm_attn_fwd_noalloc(C.byref(prob), FAKE, FAKE, FAKE, C.byref(mask), FAKE, FAKE, None)
    assert rc == L.FM_ERR_WORKSPACE
    assert b"scratch" in lib.fm_last_error()
    assert lib.fm_attn_fwd_noalloc(None, FAKE, FAKE, FAKE, C.byref(mask), FAKE, FAKE, None) == \
        L.FM_ERR_INVALID_ARGUMENT


def test_bwd_dq_path_without_room_for_stored_ds():
    """A backward workspace of the minimum size has no room for the stored-dS
    slot map: the query answers "recompute" from the sizes alone, without
    touching the device; too small a workspace and a NULL result are
    rejected."""
    lib = L.load()
    prob, mask = _problem(B=1, H=2, Sq=1000, Sk=1000), _mask()
    n = C.c_size_t()
    assert lib.fm_workspace_size(C.byref(prob), C.byref(mask), 1, C.byref(n)) == L.FM_OK
    flag = C.c_int32(7)
    assert lib.fm_bwd_dq_path(C.byref(prob), C.byref(mask), FAKE, n.value, None, C.byref(flag)) == L.FM_OK
    assert flag.value == 0
    assert lib.fm_bwd_dq_path(C.byref(prob), C.byref(mask), FAKE, n.value - 1, None,
                              C.byref(flag)) == L.FM_ERR_WORKSPACE
    assert lib.fm_bwd_dq_path(C.byref(prob), C.byref(mask), FAKE, n.value, None, None) == L.FM_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("starts,lens,sq,expect", [
    ([0, 100], [200, 50], 1000, L.FM_ERR_INVALID_ARGUMENT),    # overlap
    ([500, 100], [10, 10], 1000, L.FM_ERR_INVALID_ARGUMENT),   # descending
    ([0], [0], 1000, L.FM_ERR_INVALID_ARGUMENT),               # empty chunk
    ([990], [20], 1000, L.FM_ERR_INVALID_ARGUMENT),            # past the end
    ([], [], 1000, L.FM_ERR_INVALID_ARGUMENT),                 # no chunk
])
def test_localize_rejects_bad_chunk_lists(starts, lens, sq, expect):
    lib = L.load()
    n = len(starts)
    cs = (C.c_int32 * max(n, 1))(*starts)
    cl = (C.c_int32 * max(n, 1))(*lens)
    out = (C.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    mask = _mask()
    assert lib.fm_mask_localize(C.byref(mask), 64, sq, cs, cl, n, out, None) == expect


def test_classify_rejects_bad_blocks():
    lib = L.load()
    mask = _mask()
    assert lib.fm_tile_classify(C.byref(mask), 100, 100, 0, 64, 0, FAKE, FAKE, None) == L.FM_ERR_INVALID_ARGUMENT
    assert lib.fm_tile_classify(C.byref(mask), 100, 100, 64, 2048, 0, FAKE, FAKE, None) == L.FM_ERR_INVALID_ARGUMENT
    assert lib.fm_tile_classify(C.byref(mask), 100, 100, 64, 64, 0, None, FAKE, None) == L.FM_ERR_INVALID_ARGUMENT


def test_profile_end_without_begin_fails():
    lib = L.load()
    assert lib.fm_profile_end(None, None) == L.FM_ERR_INVALID_ARGUMENT


def _fwd_fp8(prob, mask, descale=(1.0, 1.0, 1.0)):
    lib = L.load()
    ds = None if descale is None else (C.c_float * 3)(*descale)
    return lib.fm_attn_fwd_fp8(C.byref(prob), FAKE, FAKE, FAKE, ds, C.byref(mask), FAKE, FAKE, FAKE, 1 << 30, None)


def _problem_fp8(D=128, hkv=0):
    H, Sq, Sk = 2, 100, 120
    nk = hkv or H
    arr = lambda s: (C.c_int64 * 3)(*s)
    return L.fm_problem(1, H, Sq, Sk, D, L.FM_FP8_E4M3, 0.1, arr((Sq * H * D, H * D, D)),
                        arr((Sk * nk * D, nk * D, D)), arr((Sk * nk * D, nk * D, D)), arr((Sq * H * D, H * D, D)), hkv)


@pytest.mark.parametrize("case,expect", [
    ("head_dim_96", L.FM_ERR_UNSUPPORTED),
    ("bf16_problem", L.FM_ERR_INVALID_ARGUMENT),
    ("null_descale", L.FM_ERR_INVALID_ARGUMENT),
    ("zero_descale", L.FM_ERR_INVALID_ARGUMENT),
    ("nan_descale", L.FM_ERR_INVALID_ARGUMENT),
])
def test_fwd_fp8_rejects(case, expect):
    prob, ds = _problem_fp8(), (1.0, 1.0, 1.0)
    if case == "head_dim_96":
        prob = _problem_fp8(D=96)
    elif case == "bf16_problem":
        prob = _problem(D=128)
    elif case == "null_descale":
        ds = None
    elif case == "zero_descale":
        ds = (1.0, 0.0, 1.0)
    elif case == "nan_descale":
        ds = (1.0, 1.0, float("nan"))
    assert _fwd_fp8(prob, _mask(), ds) == expect
    assert L.load().fm_last_error()


def test_fp8_problem_rejected_by_bf16_forward_and_backward():
    lib = L.load()
    prob, mask = _problem_fp8(), _mask()
    assert _fwd(prob, mask) == L.FM_ERR_INVALID_ARGUMENT
    n = C.c_size_t()
    assert lib.fm_workspace_size(C.byref(prob), C.byref(mask), 1, C.byref(n)) == L.FM_ERR_UNSUPPORTED
    assert lib.fm_attn_bwd(C.byref(prob), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(mask), FAKE, FAKE, FAKE,
                           FAKE, 1 << 30, None) == L.FM_ERR_UNSUPPORTED


def test_fp8_workspace_holds_the_v_transpose():
    """The FP8 forward's workspace exceeds the bf16 one by at least the V^T
    copy: B * H_kv * ceil(Sk / 64) * 64 * 128 bytes."""
    lib = L.load()
    mask = _mask()
    a, b = C.c_size_t(), C.c_size_t()
    assert lib.fm_workspace_size(C.byref(_problem(D=128)), C.byref(mask), 0, C.byref(a)) == L.FM_OK
    assert lib.fm_workspace_size(C.byref(_problem_fp8()), C.byref(mask), 0, C.byref(b)) == L.FM_OK
    assert b.value - a.value >= 1 * 2 * 2 * 64 * 128
