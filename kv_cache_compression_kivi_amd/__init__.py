"""KIVI-style low-bit KV cache for MI355X (gfx950).

Thin Python front end of the C ABI in include/kivi.h (libkivi.so, built
in-tree by kv_cache_compression_kivi_amd/build.py). Every function here only
marshals arguments: all quantization, ring and attention work runs in the HIP
kernels of the library. PyTorch provides device memory and streams.

The C names are exposed one to one (kivi_cache_bytes, kivi_cache_create,
kivi_append, kivi_flush, kivi_attend_decode, ...), plus KiviCache, a small
owner object that allocates the cache memory as a torch tensor and passes
tensors' device pointers and the current stream through.
"""

from ._native import (  # noqa: F401
    KIVI_BF16,
    KIVI_F16,
    KiviCache,
    KiviError,
    kivi_abi_version,
    kivi_append,
    kivi_append_rows,
    kivi_attend_decode,
    kivi_attend_decode_noalloc,
    kivi_cache_bytes,
    kivi_cache_create,
    kivi_cache_destroy,
    kivi_cache_layout,
    kivi_cache_query,
    kivi_cache_reset,
    kivi_config,
    kivi_decode_step,
    kivi_flush,
    kivi_last_error,
    kivi_layout,
    kivi_plan_append,
    kivi_plan_attend,
    kivi_query_row,
    kivi_reset_row,
    kivi_set_block_table,
    kivi_set_attend_splits,
    kivi_squat_build,
    kivi_state,
    library_path,
    load_library,
)
