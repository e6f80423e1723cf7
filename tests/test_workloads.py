"""Host-side checks of the seeded input generator (CPU only)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from paged_kv_cache_179_amd import workloads as W


def _check_tables(w, shared_prefix_blocks=0, group_size=1):
    ctx = w.context_lens.astype(np.int64)
    bs = w.block_size
    seen = {}
    for s in range(w.num_seqs):
        n = (int(ctx[s]) + bs - 1) // bs
        row = w.block_tables[s]
        assert (row[:n] >= 0).all() and (row[:n] < w.num_blocks).all()
        assert (row[n:] == -1).all()
        for j, b in enumerate(row[:n].tolist()):
            owner = (s // group_size, j) if j < shared_prefix_blocks else (s, j)
            prev = seen.setdefault(b, owner)
            assert prev == owner, f"physical block {b} used by two logical blocks"
    return seen


def _check_slots(w):
    bs = w.block_size
    assert len(np.unique(w.slot_mapping)) == len(w.slot_mapping)
    k = 0
    for r in range(w.num_seqs):
        C = int(w.context_lens[r])
        L = int(w.meta["chunk_lens"][r]) if r < len(w.prefill_rows) else 1
        for pos in range(C - L, C):
            assert w.slot_mapping[k] == int(w.block_tables[r, pos // bs]) * bs + pos % bs
            k += 1
    assert k == len(w.slot_mapping)


def test_tiny_matches_its_description():
    w = W.make("tiny")
    assert w.context_lens.tolist() == [1, 17, 33, 100]
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size) == (4, 2, 64, 16)
    assert w.num_blocks == 32 and w.max_blocks_per_seq == 7 and w.dtype == "fp32"
    used = _check_tables(w)
    assert len(used) == 13
    assert math.isclose(w.scale, 1 / 8)
    _check_slots(w)


@pytest.mark.parametrize("name", ["tinyllama", "llama2_7b", "qwen25_7b", "gemma_2b_mixed"])
def test_structure(name):
    w = W.make(name, with_pools=False)
    ctx = w.context_lens
    if name == "tinyllama":
        assert w.num_seqs == 64 and ctx.min() >= 128 and ctx.max() <= 2048
        assert (w.num_heads, w.num_kv_heads, w.head_dim, w.dtype) == (32, 4, 64, "bf16")
    if name == "llama2_7b":
        assert w.num_seqs == 128 and ctx.min() >= 512 and ctx.max() <= 4096
        assert (w.num_heads, w.num_kv_heads, w.head_dim, w.dtype) == (32, 32, 128, "fp16")
        assert w.partition_size == 512
    if name == "qwen25_7b":
        assert w.num_seqs == 256 and ctx.min() >= 513 and ctx.max() <= 8192
        assert (w.num_heads, w.num_kv_heads, w.head_dim, w.dtype) == (28, 4, 128, "bf16")
        _check_tables(w, shared_prefix_blocks=32, group_size=16)
        for g in range(16):
            rows = w.block_tables[16 * g:16 * g + 16, :32]
            assert (rows == rows[0]).all(), "a group must share its 32 prefix blocks"
        assert len(np.unique(w.block_tables[::16, :32])) == 16 * 32
        suffix = ctx - 512
        assert 400 < np.median(suffix) < 650  # lognormal with median 512
    else:
        _check_tables(w)
    if name == "gemma_2b_mixed":
        assert ctx[:4].tolist() == [512, 1536, 2560, 4096]
        assert w.query_start_loc.tolist() == [0, 512, 1024, 1536, 2048]
        assert len(w.decode_rows) == 124 and ctx[4:].min() >= 256 and ctx[4:].max() <= 4096
        assert len(w.slot_mapping) == 4 * 512 + 124
    else:
        assert len(w.prefill_rows) == 0 and len(w.slot_mapping) == w.num_seqs
    assert w.num_blocks == math.ceil(1.1 * w.meta["needed_blocks"])
    _check_slots(w)


def test_deterministic_and_nan_sentinel():
    a = W.make("tinyllama")
    b = W.make("tinyllama")
    assert torch.equal(a.key_cache.view(torch.int16), b.key_cache.view(torch.int16))
    assert torch.equal(a.query_decode, b.query_decode) and np.array_equal(a.block_tables, b.block_tables)
    bs = a.block_size
    blk = a.slot_mapping // bs
    off = a.slot_mapping % bs
    assert torch.isnan(a.key_cache[blk, :, off, :]).all()
    assert torch.isnan(a.value_cache[blk, :, off, :]).all()
    assert torch.isnan(a.key_cache).sum() == len(a.slot_mapping) * a.num_kv_heads * a.head_dim


def test_pool_chunks_independent_of_threads(monkeypatch):
    shape = (300, 2, 16, 64)
    monkeypatch.setattr(W, "POOL_CHUNK_ELEMS", 1 << 14)
    p1 = W._normal_pool(5, 1, shape, "bf16")
    monkeypatch.setattr(W, "_threads", lambda: 1)
    p2 = W._normal_pool(5, 1, shape, "bf16")
    assert torch.equal(p1.view(torch.int16), p2.view(torch.int16))
    assert abs(float(p1.float().mean())) < 0.02 and abs(float(p1.float().std()) - 1) < 0.02


def test_small_case_shapes():
    w = W.small_case(11, num_seqs=5, ctx_lo=1, ctx_hi=300, num_heads=6, num_kv_heads=2,
                     head_dim=64, block_size=16, dtype="bf16", chunk_lens=[40, 1],
                     extra_ctx=[100, 40, 1])
    assert w.context_lens[:3].tolist() == [100, 40, 1]
    assert w.query_start_loc.tolist() == [0, 40, 41]
    _check_tables(w)
    _check_slots(w)
    pairs = W.attended_pairs(w)
    assert pairs["prefill"] == 40 * 60 + 40 * 41 // 2 + 40
