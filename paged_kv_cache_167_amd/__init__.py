"""Paged KV-cache decode attention for AMD MI355X.

The computation lives in libpa.so (HIP kernels for gfx950, C ABI in
include/pa.h); this package is its Python binding.
"""
from ._lib import (  # noqa: F401
    DEFAULT_PARTITION,
    BlockAllocator,
    DenseKV,
    PA_F16,
    PA_F32,
    PaError,
    last_error,
    lib,
    pa_cache_write,
    pa_copy_blocks,
    pa_cache_write_fp8,
    pa_decode,
    pa_decode_append,
    pa_decode_append_partitions,
    pa_decode_fp8,
    pa_decode_fp8_append,
    pa_decode_fp8_append_partitions,
    pa_decode_fp8_partitions,
    pa_decode_noalloc,
    pa_decode_partitions,
    pa_decode_reduce,
    pa_decode_shared,
    pa_decode_shared_partitions,
    pa_decode_shared_workspace_bytes,
    pa_decode_workspace_bytes,
    pa_prefill,
)
