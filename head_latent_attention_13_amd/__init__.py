"""MI355X-native Multi-Head Latent Attention (MLA) decode library.

The compute lives in libmla.so (hand-written HIP for gfx950, C ABI in
include/mla.h); this package is its thin ctypes binding plus a small helper
that owns the device buffers of one layer (``MLALayer``).
"""
from ._lib import (MLA_BF16, MLA_F32, MLA_ROWS_DTYPE, MLA_ROWS_E4M3, MLA_WEIGHTS_FACTORED, MLA_WEIGHTS_MERGED, RAW_WEIGHT_NAMES, Cache, MLAError, EXPORTED, LIB_PATH, load, make_dims,
                   mla_absorb_weights, mla_absorbed_layout, mla_attention, mla_attention_noalloc, mla_cache_store_rows,
                   mla_compress_append, mla_decode,
                   mla_dims, mla_out_proj, mla_prefill_expanded, mla_prefill_workspace_size, mla_q_proj,
                   mla_prefill_workspace_check, mla_read_device_error, mla_version, mla_workspace_check,
                   mla_workspace_size)
from .layer import MLALayer

__all__ = [
    "MLA_BF16", "MLA_F32", "MLA_ROWS_DTYPE", "MLA_ROWS_E4M3", "MLA_WEIGHTS_FACTORED", "MLA_WEIGHTS_MERGED", "RAW_WEIGHT_NAMES", "Cache", "MLAError", "EXPORTED", "LIB_PATH", "load", "make_dims",
    "mla_absorb_weights", "mla_absorbed_layout", "mla_attention", "mla_attention_noalloc", "mla_cache_store_rows", "mla_compress_append",
    "mla_decode",
    "mla_dims", "mla_out_proj", "mla_prefill_expanded", "mla_prefill_workspace_size", "mla_q_proj",
    "mla_prefill_workspace_check", "mla_read_device_error", "mla_version", "mla_workspace_check",
    "mla_workspace_size",
    "MLALayer",
]
