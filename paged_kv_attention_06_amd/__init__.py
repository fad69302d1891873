"""Paged KV-cache attention for AMD MI355X (gfx950).

The compute path is libpkv.so (hand-written HIP kernels behind a C ABI,
include/pkv.h); this package is its ctypes binding.  Importing it fails
loudly when the library has not been built.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    PKV_BF16,
    PKV_F32,
    PKV_FP8_E4M3,
    PKV_LAYOUT_HEAD_KV_GRANULE16,
    Cache,
    PkvCache,
    PkvError,
    Pool,
    block_copy,
    block_swap,
    descriptor,
    paged_attention_decode,
    paged_attention_decode_noalloc,
    paged_attention_mixed,
    paged_kv_write,
    pkv_attention_workspace_bytes,
    pkv_block_bytes,
    pkv_block_hash,
    pkv_build_slot_mapping,
    pkv_layout,
    pkv_read_slices,
    pkv_validate_attention,
    pkv_validate_block_pairs,
    pkv_validate_slots,
    status_string,
    version,
)
