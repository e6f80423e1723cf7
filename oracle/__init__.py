"""fp64 CPU oracle for paged attention (test infrastructure only; see
``oracle.attention`` for what may import it)."""
from .attention import (  # noqa: F401
    attend,
    block_of,
    cap_scores,
    gather,
    kv_head_of,
    paged_decode,
    paged_prefill_chunk,
    query_position,
    reshape_and_cache,
    window_first_key,
)
from .blocks import copy_blocks, swap_blocks  # noqa: F401,E402
from .fp8 import dequantize as fp8_dequantize, reshape_and_cache_fp8  # noqa: F401,E402
