"""ctypes view of libfmattn's C ABI (include/fm_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfmattn.so")

FM_OK, FM_ERR_INVALID_ARGUMENT, FM_ERR_UNSUPPORTED, FM_ERR_WORKSPACE, FM_ERR_HIP = range(5)
FM_BF16, FM_FP32, FM_FP8_E4M3 = 0, 1, 2
FM_TILE_SKIP, FM_TILE_PARTIAL, FM_TILE_FULL = 0, 1, 2
STAGES = ("classify_summary", "classify_map", "fwd", "bwd_pre", "bwd", "bwd_dq", "localize",
          "bwd_plan", "bwd_dq_ds", "order", "transfer", "chunk_work", "v_transpose")
FM_NUM_STAGES = len(STAGES)

STATUS_NAMES = {0: "FM_OK", 1: "FM_ERR_INVALID_ARGUMENT", 2: "FM_ERR_UNSUPPORTED",
                3: "FM_ERR_WORKSPACE", 4: "FM_ERR_HIP"}

# Every symbol the header declares (checked by the CPU test-suite).
EXPORTS = ("fm_kernel_tile", "fm_workspace_size", "fm_bwd_workspace_size_ds", "fm_bwd_dq_path", "fm_tile_classify",
           "fm_attn_fwd", "fm_attn_fwd_noalloc", "fm_attn_fwd_fp8", "fm_attn_bwd", "fm_mask_localize", "fm_kv_transfer_set", "fm_chunk_work", "fm_cp_plan",
           "fm_profile_begin",
           "fm_profile_end", "fm_last_error")


class fm_mask(C.Structure):
    _fields_ = [("lts", C.c_void_p), ("lte", C.c_void_p), ("uts", C.c_void_p), ("ute", C.c_void_p),
                ("batch", C.c_int32), ("heads", C.c_int32),
                ("stride_b", C.c_int64), ("stride_h", C.c_int64)]


class fm_problem(C.Structure):
    _fields_ = [("batch", C.c_int32), ("heads", C.c_int32), ("seqlen_q", C.c_int32),
                ("seqlen_k", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32),
                ("softmax_scale", C.c_float),
                ("q_stride", C.c_int64 * 3), ("k_stride", C.c_int64 * 3),
                ("v_stride", C.c_int64 * 3), ("o_stride", C.c_int64 * 3), ("heads_kv", C.c_int32)]


class FmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libfmattn once and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m masked_tiled_attention_amd.build` "
            "(there is no fallback implementation)")
    lib = C.CDLL(path)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    P = C.POINTER
    lib.fm_kernel_tile.restype = None
    lib.fm_kernel_tile.argtypes = [i32, i32, P(i32), P(i32)]
    lib.fm_workspace_size.restype = C.c_int
    lib.fm_workspace_size.argtypes = [P(fm_problem), P(fm_mask), i32, P(sz)]
    lib.fm_bwd_workspace_size_ds.restype = C.c_int
    lib.fm_bwd_workspace_size_ds.argtypes = [P(fm_problem), P(fm_mask), vp, sz, vp, P(sz)]
    lib.fm_bwd_dq_path.restype = C.c_int
    lib.fm_bwd_dq_path.argtypes = [P(fm_problem), P(fm_mask), vp, sz, vp, P(i32)]
    lib.fm_tile_classify.restype = C.c_int
    lib.fm_tile_classify.argtypes = [P(fm_mask), i32, i32, i32, i32, i32, vp, vp, vp]
    lib.fm_attn_fwd.restype = C.c_int
    lib.fm_attn_fwd.argtypes = [P(fm_problem), vp, vp, vp, P(fm_mask), vp, vp, vp, sz, vp]
    lib.fm_attn_fwd_noalloc.restype = C.c_int
    lib.fm_attn_fwd_noalloc.argtypes = [P(fm_problem), vp, vp, vp, P(fm_mask), vp, vp, vp]
    lib.fm_attn_fwd_fp8.restype = C.c_int
    lib.fm_attn_fwd_fp8.argtypes = [P(fm_problem), vp, vp, vp, P(C.c_float), P(fm_mask), vp, vp, vp, sz, vp]
    lib.fm_attn_bwd.restype = C.c_int
    lib.fm_attn_bwd.argtypes = [P(fm_problem), vp, vp, vp, vp, vp, vp, P(fm_mask), vp, vp, vp,
                                vp, sz, vp]
    lib.fm_mask_localize.restype = C.c_int
    lib.fm_mask_localize.argtypes = [P(fm_mask), i32, i32, P(i32), P(i32), i32, P(vp), vp]
    lib.fm_chunk_work.restype = C.c_int
    lib.fm_chunk_work.argtypes = [P(fm_mask), i32, i32, P(i32), P(i32), i32, vp, vp]
    lib.fm_cp_plan.restype = C.c_int
    lib.fm_cp_plan.argtypes = [P(C.c_int64), i32, i32, P(i32), P(C.c_int64)]
    lib.fm_kv_transfer_set.restype = C.c_int
    lib.fm_kv_transfer_set.argtypes = [P(fm_mask), i32, i32, i32, vp, vp, vp]
    lib.fm_profile_begin.restype = C.c_int
    lib.fm_profile_begin.argtypes = [i32]
    lib.fm_profile_end.restype = C.c_int
    lib.fm_profile_end.argtypes = [P(C.c_float), P(i32)]
    lib.fm_last_error.restype = C.c_char_p
    lib.fm_last_error.argtypes = []
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FM_OK:
        raise FmError(status, load().fm_last_error().decode(errors="replace"))
