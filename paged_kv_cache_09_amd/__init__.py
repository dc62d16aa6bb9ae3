"""MI355X (gfx950) paged KV-cache decode library: Python binding of libpagedkv.so.

The functions here only marshal torch tensors into the C ABI declared in
include/paged_kv.h (device pointers, sizes, the current HIP stream); every step of
the computation runs in the library's HIP kernels.  Importing this package does
not load the library; the first call does, and fails loudly if it is not built.
"""
from ._lib import (  # noqa: F401
    PKV_BF16,
    PKV_FP16,
    PagedKVError,
    exported_symbols,
    header_symbols,
    lib_path,
    load,
    max_partitions,
    paged_attention_append_decode,
    paged_attention_decode,
    paged_attention_decode_ordered,
    paged_attention_decode_slotted,
    paged_attention_append_decode_slotted,
    paged_attention_append_decode_slotted_split,
    paged_attention_decode_slotted_split,
    paged_attention_prefix_decode,
    paged_attention_prefix_split_decode,
    paged_attention_reduce,
    paged_attention_split_decode,
    paged_attention_split_decode_noalloc,
    paged_kv_append,
    paged_kv_append_tokens,
    paged_kv_copy_blocks,
    paged_kv_copy_slots,
    status_string,
)
from .plan import long_first_order  # noqa: F401
