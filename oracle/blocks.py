"""Block-pool copies of the CPU oracle (test infrastructure only, like the
rest of ``oracle``: used by ``tests/`` and by nothing on the product path).

What the pages say these operations are for:

* Copy-on-write of a shared block -- the wLLM case study (ADR-001 on the
  KV-cache layout) makes prefix sharing a block-table operation: several
  tables name one physical block.  The mini-vLLM README ("Limitations") keeps
  a per-block reference count for prefix caching.  A sequence about to write
  into a block that others still read first gets a private copy of it.
* Swap -- the wLLM PyPI page ("Features -- Core engine") lists CPU-swap
  preemption: an evicted sequence's blocks go to host memory and come back
  later, so it resumes where it stopped.

Both are whole-block copies named by (source, destination) block-id pairs.
Readings where the pages are silent: a pair whose id falls outside its pool
is skipped; every copy reads the pool as it was before the call (the GPU runs
the pairs in no particular order, so destinations must be distinct and must
not be another pair's source).

Pinned by ``tests/test_oracle_pins.py`` (a hand-worked example, untouched
blocks, a swap round trip).
"""
from __future__ import annotations

import numpy as np


def _pairs(block_mapping):
    return [(int(s), int(d)) for s, d in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)]


def swap_blocks(src_pool, dst_pool, block_mapping):
    """Returns a copy of ``dst_pool`` ([NB_dst, ...]) in which block ``d`` of
    every pair (s, d) holds block ``s`` of ``src_pool`` (same block shape)."""
    src = np.asarray(src_pool)
    out = np.array(dst_pool, copy=True)
    for s, d in _pairs(block_mapping):
        if 0 <= s < src.shape[0] and 0 <= d < out.shape[0]:
            out[d] = src[s]
    return out


def copy_blocks(key_cache, value_cache, block_mapping):
    """Copy-on-write inside one pool: returns new (key_cache, value_cache) in
    which block ``d`` of every pair (s, d) holds the old block ``s``, for K
    and V alike."""
    return (swap_blocks(key_cache, key_cache, block_mapping),
            swap_blocks(value_cache, value_cache, block_mapping))
