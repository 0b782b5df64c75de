"""Masked tiled attention for AMD MI355X (gfx950).

Exact scaled-dot-product attention under structural masks in column-sparse
form (four int32 query-axis bound vectors per key column), forward and
backward, as hand-written HIP kernels behind a C ABI (libfmattn.so,
include/fm_attn.h). This package is the thin Python binding.
"""
from ._lib import FmError, load, EXPORTS  # noqa: F401
from .api import (Mask, fm_attn_bwd, fm_attn_fwd, fm_attn_fwd_fp8, fm_attn_fwd_noalloc, fm_bwd_dq_path, fm_bwd_workspace_size_ds,  # noqa: F401
                  fm_kernel_tile,
                  fm_chunk_work, fm_cp_plan, fm_kv_transfer_set, fm_mask_localize, fm_profile_begin, fm_profile_end, fm_tile_classify,
                  fm_workspace_size, fm_workspace_size_fp8)
