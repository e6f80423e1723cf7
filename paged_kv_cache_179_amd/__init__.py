"""Paged attention over a block-based KV cache, native to MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libpaged_attention.so``, built from ``csrc/``); this package is its thin
ctypes binding.  PyTorch supplies device memory and the current stream only.
Importing the package does not load the library: the first call does, and it
raises if the library is missing -- there is no fallback path.
"""
from .binding import (  # noqa: F401
    PagedAttentionError,
    copy_blocks,
    decode,
    decode_fused_write,
    decode_noalloc,
    decode_partitions,
    decode_reduce,
    decode_workspace_bytes,
    library,
    library_path,
    prefill_chunk,
    prefill_chunk_fused,
    prefill_workspace_bytes,
    reshape_and_cache,
    reshape_and_cache_fp8,
    stream_read_probe,
    swap_blocks,
)
