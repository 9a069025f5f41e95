"""Exact blockwise multi-head attention (forward and backward) for MI355X (gfx950).

The computation runs in hand-written HIP kernels inside ``libattn.so`` behind the
C ABI of ``include/attn.h``; this package is its Python binding.  Build the
library with ``python -m exact_blockwise_attention_attn_amd._build``.
"""
from ._lib import (  # noqa: F401
    ATTN_DTYPE_BF16, ATTN_DTYPE_F32, ATTN_MASK_CAUSAL, ATTN_MASK_CAUSAL_WINDOW, ATTN_MASK_NONE, ATTN_MASK_WINDOW, ATTN_OK,
    AttnError, LIB_PATH, attn_bwd, attn_bwd_check_args, attn_check_args, attn_fwd, attn_fwd_kv, attn_fwd_kv_check_args, attn_fwd_kv_noalloc,
    attn_fwd_kv_workspace_size, attn_fwd_block_sparse, attn_fwd_block_sparse_check_args, attn_set_key_groups,
    attn_set_schedule, attn_set_work_queue,
    attn_strerror, attn_version,
    bwd, fwd, fwd_block_sparse, fwd_kv, load,
)

__version__ = "0.5.0"
