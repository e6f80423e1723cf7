"""Seeded synthetic inputs for paged attention.

This module only draws inputs: context lengths, a shuffled physical block pool,
per-sequence block tables, slot mappings and N(0, 1) query/key/value tensors.
It holds none of the attention arithmetic, so both the HIP path and the CPU
oracle can be fed from it without sharing any of the method's code.

The memory model follows the mini-vLLM README ("How it works -- Paged
KV-cache"): preallocated equal blocks of ``block_size`` tokens, and for each
sequence a table giving the physical block behind each logical one.  Prefix sharing
is expressed the way the wLLM case study's ADR-001 ("KV-cache layout") puts it:
several tables name the same physical blocks.

Cache layout (both K and V): ``[num_blocks, num_kv_heads, block_size, head_dim]``.
Slot encoding: ``slot = physical_block * block_size + offset``; ``slot < 0``
means "skip".  Table entries past a sequence's last block are -1.

Workloads (sizes as named):
  tiny           4 seqs, ctx {1,17,33,100}, Hq 4 / Hkv 2, D 64, fp32, 32-block pool
  tinyllama      64 seqs, ctx U[128,2048], Hq 32 / Hkv 4, D 64, bf16
  llama2_7b      128 seqs, ctx U[512,4096], Hq 32 / Hkv 32, D 128, fp16, 512-token partitions
  qwen25_7b      256 seqs in 16 groups sharing a 512-token prefix, lognormal suffix,
                 Hq 28 / Hkv 4, D 128, bf16
  gemma_2b_mixed 4 prefill chunks of 512 (prior 0/1024/2048/3584) + 124 decode rows
                 with ctx U[256,4096], Hq 8 / Hkv 1, D 256, bf16

Every workload also carries the new tokens of the step: each decode row's
current token (position C-1) and each chunk's L tokens (positions C-L..C-1).
Their pool slots are pre-filled with NaN, so a step that attends before the
cache write has landed produces NaN instead of a plausible wrong answer.

Random draws: one ``numpy.random.default_rng(179000 + index)`` stream gives, in
order, the lengths, the block permutation, the queries and the new K/V.  The
two pools are drawn in fixed chunks of blocks, chunk ``c`` of the K pool from
``SeedSequence(179000 + index, spawn_key=(1, c))`` and of the V pool from
``spawn_key=(2, c)``, so they can be filled by several threads and still be
identical on every machine.  Values are drawn as float32 and rounded to the
storage dtype by round-to-nearest-even (torch's cast).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

SEED_BASE = 179_000
POOL_CHUNK_ELEMS = 1 << 22  # elements per independently seeded pool chunk

TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    """One batch of synthetic paged-attention inputs (all host tensors)."""

    name: str
    index: int
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    partition_size: int
    context_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, MBPS], -1 padded
    key_cache: torch.Tensor  # [NB, Hkv, bs, D], NaN at the new tokens' slots
    value_cache: torch.Tensor
    decode_rows: np.ndarray  # int64 indices of single-token rows
    prefill_rows: np.ndarray  # int64 indices of chunk rows
    query_decode: torch.Tensor  # [len(decode_rows), Hq, D]
    query_prefill: torch.Tensor  # [sum L, Hq, D]
    query_start_loc: np.ndarray  # int32 [len(prefill_rows) + 1]
    new_key: torch.Tensor  # [N_new, Hkv, D]
    new_value: torch.Tensor
    slot_mapping: np.ndarray  # int64 [N_new]
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return torch.empty((), dtype=self.torch_dtype).element_size()

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


@dataclass
class _Spec:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int = 16
    partition_size: int = 512


SPECS: List[_Spec] = [
    _Spec("tiny", "fp32", 4, 2, 64),
    _Spec("tinyllama", "bf16", 32, 4, 64),
    _Spec("llama2_7b", "fp16", 32, 32, 128),
    _Spec("qwen25_7b", "bf16", 28, 4, 128),
    _Spec("gemma_2b_mixed", "bf16", 8, 1, 256),
]
NAMES = [s.name for s in SPECS]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _round_to(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(TORCH_DTYPES[dtype])


def _normal_pool(seed: int, tag: int, shape, dtype: str) -> torch.Tensor:
    """N(0,1) pool drawn in independently seeded chunks of whole blocks."""
    nb = shape[0]
    per_block = int(np.prod(shape[1:]))
    blocks_per_chunk = max(1, POOL_CHUNK_ELEMS // per_block)
    out = torch.empty(shape, dtype=TORCH_DTYPES[dtype])
    n_chunks = (nb + blocks_per_chunk - 1) // blocks_per_chunk

    def fill(c: int) -> None:
        lo = c * blocks_per_chunk
        hi = min(nb, lo + blocks_per_chunk)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, c)))
        a = rng.standard_normal((hi - lo,) + tuple(shape[1:]), dtype=np.float32)
        out[lo:hi] = torch.from_numpy(a).to(out.dtype)

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def _alloc_tables(ctx, bs, shared_prefix_groups=None, prefix_blocks=0):
    """Assign physical blocks to every sequence's logical blocks.

    Returns (blocks per sequence, distinct blocks needed, {seq: group}).  With
    ``shared_prefix_groups`` (list of index lists), the first ``prefix_blocks``
    logical blocks of every member of a group name the same physical blocks.
    """
    nblk = [(int(c) + bs - 1) // bs for c in ctx]
    shared = {}
    needed = sum(nblk)
    if shared_prefix_groups:
        needed -= sum((len(g) - 1) * prefix_blocks for g in shared_prefix_groups)
        for gi, g in enumerate(shared_prefix_groups):
            for s in g:
                shared[s] = gi
    return nblk, needed, shared


def _tables_from_perm(perm, nblk, bs, mbps, shared, prefix_blocks):
    S = len(nblk)
    bt = np.full((S, mbps), -1, dtype=np.int32)
    cursor = 0
    group_blocks = {}
    for s in range(S):
        start = 0
        if s in shared:
            g = shared[s]
            if g not in group_blocks:
                group_blocks[g] = perm[cursor:cursor + prefix_blocks].astype(np.int32)
                cursor += prefix_blocks
            bt[s, :prefix_blocks] = group_blocks[g]
            start = prefix_blocks
        n = nblk[s] - start
        bt[s, start:nblk[s]] = perm[cursor:cursor + n]
        cursor += n
    return bt


def make(index_or_name, seed_offset: int = 0, with_pools: bool = True) -> Workload:
    """Build one of the five named workloads (by index 0-4 or name).

    ``with_pools=False`` skips drawing the two pools (zeros instead) for
    structural checks of the tables and slots."""
    if isinstance(index_or_name, str):
        index = NAMES.index(index_or_name)
    else:
        index = int(index_or_name)
    spec = SPECS[index]
    seed = SEED_BASE + index + seed_offset
    rng = np.random.default_rng(seed)
    bs = spec.block_size
    groups = None
    prefix_blocks = 0
    chunk_lens: List[int] = []

    # 1. lengths
    if spec.name == "tiny":
        ctx = np.array([1, 17, 33, 100], dtype=np.int64)
        mbps = 7
    elif spec.name == "tinyllama":
        ctx = rng.integers(128, 2048 + 1, size=64)
        mbps = 2048 // bs
    elif spec.name == "llama2_7b":
        ctx = rng.integers(512, 4096 + 1, size=128)
        mbps = 4096 // bs
    elif spec.name == "qwen25_7b":
        z = rng.standard_normal(256)
        suffix = np.clip(np.rint(np.exp(math.log(512.0) + 1.0 * z)), 1, 7680).astype(np.int64)
        ctx = 512 + suffix
        mbps = 8192 // bs
        prefix_blocks = 512 // bs
        groups = [list(range(16 * g, 16 * g + 16)) for g in range(16)]
    elif spec.name == "gemma_2b_mixed":
        prior = np.array([0, 1024, 2048, 3584], dtype=np.int64)
        chunk_lens = [512] * 4
        dec = rng.integers(256, 4096 + 1, size=124)
        ctx = np.concatenate([prior + 512, dec])
        mbps = 4096 // bs
    else:  # pragma: no cover
        raise ValueError(spec.name)
    ctx = ctx.astype(np.int64)
    S = len(ctx)

    # 2. block permutation and tables
    nblk, needed, shared = _alloc_tables(ctx, bs, groups, prefix_blocks)
    if spec.name == "tiny":
        nb = 32
    else:
        nb = int(math.ceil(1.1 * needed))
    perm = rng.permutation(nb)
    bt = _tables_from_perm(perm, nblk, bs, mbps, shared, prefix_blocks)

    n_chunks = len(chunk_lens)
    prefill_rows = np.arange(n_chunks, dtype=np.int64)
    decode_rows = np.arange(n_chunks, S, dtype=np.int64)
    Hq, Hkv, D = spec.num_heads, spec.num_kv_heads, spec.head_dim

    # 3. queries (decode rows first, then the chunk tokens)
    qd = rng.standard_normal((len(decode_rows), Hq, D), dtype=np.float32)
    n_q_prefill = int(sum(chunk_lens))
    qp = rng.standard_normal((n_q_prefill, Hq, D), dtype=np.float32)
    qsl = np.zeros(n_chunks + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(chunk_lens) if n_chunks else []

    # 4./5. the pools
    pool_shape = (nb, Hkv, bs, D)
    if with_pools:
        key_cache = _normal_pool(seed, 1, pool_shape, spec.dtype)
        value_cache = _normal_pool(seed, 2, pool_shape, spec.dtype)
    else:
        key_cache = torch.zeros(pool_shape, dtype=TORCH_DTYPES[spec.dtype])
        value_cache = torch.zeros(pool_shape, dtype=TORCH_DTYPES[spec.dtype])

    # 6. the new tokens of this step and their slots
    slots: List[int] = []
    for r in range(S):
        c = int(ctx[r])
        L = chunk_lens[r] if r < n_chunks else 1
        for pos in range(c - L, c):
            slots.append(int(bt[r, pos // bs]) * bs + pos % bs)
    slot_mapping = np.asarray(slots, dtype=np.int64)
    nk = rng.standard_normal((len(slots), Hkv, D), dtype=np.float32)
    nv = rng.standard_normal((len(slots), Hkv, D), dtype=np.float32)
    # A missed cache write must not look like a plausible answer.
    blk = torch.from_numpy(slot_mapping // bs)
    off = torch.from_numpy(slot_mapping % bs)
    key_cache[blk, :, off, :] = float("nan")
    value_cache[blk, :, off, :] = float("nan")

    return Workload(
        name=spec.name,
        index=index,
        dtype=spec.dtype,
        num_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        block_size=bs,
        num_blocks=nb,
        max_blocks_per_seq=mbps,
        scale=1.0 / math.sqrt(D),
        partition_size=spec.partition_size,
        context_lens=ctx.astype(np.int32),
        block_tables=bt,
        key_cache=key_cache,
        value_cache=value_cache,
        decode_rows=decode_rows,
        prefill_rows=prefill_rows,
        query_decode=_round_to(qd, spec.dtype),
        query_prefill=_round_to(qp, spec.dtype),
        query_start_loc=qsl,
        new_key=_round_to(nk, spec.dtype),
        new_value=_round_to(nv, spec.dtype),
        slot_mapping=slot_mapping,
        meta={"needed_blocks": needed, "groups": groups, "prefix_blocks": prefix_blocks,
              "chunk_lens": chunk_lens},
    )


def small_case(seed: int, *, num_seqs: int, ctx_lo: int, ctx_hi: int, num_heads: int,
               num_kv_heads: int, head_dim: int, block_size: int, dtype: str,
               chunk_lens: Optional[List[int]] = None, pool_slack: float = 1.25,
               extra_ctx: Optional[List[int]] = None) -> Workload:
    """A small seeded workload of arbitrary shape (for parity tests).

    ``chunk_lens`` makes the first ``len(chunk_lens)`` rows prefill chunks of
    those lengths; the remaining rows are decode rows.  ``extra_ctx`` fixes
    the context lengths of leading rows (edge cases such as 1 or an exact
    multiple of the block size); the rest are drawn from ``[ctx_lo, ctx_hi]``.
    """
    rng = np.random.default_rng(seed)
    chunk_lens = list(chunk_lens or [])
    fixed = list(extra_ctx or [])
    n_rand = num_seqs - len(fixed)
    ctx = np.concatenate([np.asarray(fixed, dtype=np.int64),
                          rng.integers(ctx_lo, ctx_hi + 1, size=max(0, n_rand))])
    for r, L in enumerate(chunk_lens):
        ctx[r] = max(int(ctx[r]), L)
    S = len(ctx)
    bs = block_size
    mbps = max(1, (int(ctx.max()) + bs - 1) // bs) if S else 1
    nblk = [(int(c) + bs - 1) // bs for c in ctx]
    needed = sum(nblk)
    nb = max(1, int(math.ceil(pool_slack * needed)))
    perm = rng.permutation(nb)
    bt = _tables_from_perm(perm, nblk, bs, mbps, {}, 0)
    n_chunks = len(chunk_lens)
    decode_rows = np.arange(n_chunks, S, dtype=np.int64)
    prefill_rows = np.arange(n_chunks, dtype=np.int64)
    qd = rng.standard_normal((len(decode_rows), num_heads, head_dim), dtype=np.float32)
    qp = rng.standard_normal((int(sum(chunk_lens)), num_heads, head_dim), dtype=np.float32)
    qsl = np.zeros(n_chunks + 1, dtype=np.int32)
    if n_chunks:
        qsl[1:] = np.cumsum(chunk_lens)
    pool_shape = (nb, num_kv_heads, bs, head_dim)
    kc = _round_to(rng.standard_normal(pool_shape, dtype=np.float32), dtype)
    vc = _round_to(rng.standard_normal(pool_shape, dtype=np.float32), dtype)
    slots = []
    for r in range(S):
        c = int(ctx[r])
        L = chunk_lens[r] if r < n_chunks else 1
        for pos in range(max(0, c - L), c):
            slots.append(int(bt[r, pos // bs]) * bs + pos % bs)
    slot_mapping = np.asarray(slots, dtype=np.int64)
    nk = rng.standard_normal((len(slots), num_kv_heads, head_dim), dtype=np.float32)
    nv = rng.standard_normal((len(slots), num_kv_heads, head_dim), dtype=np.float32)
    if len(slots):
        blk = torch.from_numpy(slot_mapping // bs)
        off = torch.from_numpy(slot_mapping % bs)
        kc[blk, :, off, :] = float("nan")
        vc[blk, :, off, :] = float("nan")
    return Workload(
        name=f"small_{seed}", index=-1, dtype=dtype, num_heads=num_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs, num_blocks=nb,
        max_blocks_per_seq=mbps, scale=1.0 / math.sqrt(head_dim), partition_size=512,
        context_lens=ctx.astype(np.int32), block_tables=bt, key_cache=kc, value_cache=vc,
        decode_rows=decode_rows, prefill_rows=prefill_rows,
        query_decode=_round_to(qd, dtype), query_prefill=_round_to(qp, dtype),
        query_start_loc=qsl, new_key=_round_to(nk, dtype), new_value=_round_to(nv, dtype),
        slot_mapping=slot_mapping, meta={"needed_blocks": needed, "chunk_lens": chunk_lens},
    )


def attended_pairs(w: Workload) -> Dict[str, int]:
    """Counts used for throughput figures: attended (query token, KV position) pairs."""
    ctx = w.context_lens.astype(np.int64)
    dec = int(ctx[w.decode_rows].sum()) if len(w.decode_rows) else 0
    pre = 0
    for i, r in enumerate(w.prefill_rows):
        L = int(w.query_start_loc[i + 1] - w.query_start_loc[i])
        C = int(ctx[r])
        pre += L * (C - L) + L * (L + 1) // 2
    return {"decode": dec, "prefill": pre}
