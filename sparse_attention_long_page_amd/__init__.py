"""MI355X (gfx950) dynamic page/block-sparse attention over a paged KV cache.

The compute lives in libsparse_attn.so (hand-written HIP, C ABI in
include/sparse_attn.h); ``binding`` marshals torch tensors into its calls.
"""
from .binding import (PagedKV, SparseAttnError, load_library, library_path, sa_page_summary,
                      sa_select_pages, sa_select_pages_workspace_size, sa_sparse_decode, sa_sparse_decode_noalloc,
                      sa_sparse_decode_workspace_size, sa_select_decode, sa_block_sparse_prefill,
                      sa_block_sparse_prefill_workspace_size, sa_prefill_block_mask, sa_page_value_summary,
                      sa_prefill_mean_correction, sa_prefill_mean_correction_workspace_size,
                      sa_head_page_mass, sa_head_page_mass_workspace_size, sa_autotune_tiers,
                      sa_autotune_tiers_workspace_size, sa_ambient_head_mask,
                      sa_set_debug_validate, sa_version, SA_SEL_PER_KV_HEAD,
                      SA_SEL_PER_Q_HEAD, SA_DTYPE_BF16, SA_DTYPE_FP32, SA_DTYPE_FP8_E4M3, SA_OK, SA_ERR_INVALID_ARGUMENT,
                      SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE_TOO_SMALL, SA_ERR_DEVICE, SA_ERR_DATA, SA_NOALLOC_SCRATCH_BYTES,
                      EXPORTED)

__all__ = [n for n in dir() if not n.startswith("_")]
