"""Top-k sparse attention for AMD Instinct MI355X (gfx950).

The compute lives in the C-ABI shared library ``libsparse_attn.so`` (hand-written
HIP kernels, declared in ``include/sparse_attn.h``); this package only marshals
torch tensors into that library's plain-pointer entry points. Importing the
package loads nothing; the library is loaded on the first call and a missing or
unloadable library raises immediately (there is no fallback path).
"""
from .api import (  # noqa: F401
    SparseAttnError,
    candidate_mask_apply,
    candidate_mask_grid,
    library_path,
    masked_attn,
    masked_attn_offset,
    new_workspace,
    sparse_attn,
    sparse_attn_fp8,
    sparse_attn_fp8_merge,
    sparse_attn_fp8_split,
    sparse_attn_merge,
    sparse_attn_noalloc,
    sparse_attn_split,
    sparse_attn_fp8_num_splits,
    sparse_attn_head_groups,
    sparse_attn_num_splits,
    sparse_attn_workspace_bytes,
    topk_bitmask_build,
    topk_bitmask_shape,
)
