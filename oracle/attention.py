"""Plain fp64 CPU oracle for paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: it is used by ``tests/``, by the smoke check in the graft
entry point and by the benchmark's CPU-baseline leg, and by nothing else.  It
shares no code with the HIP library (no kernels, headers, helpers or tables).

What it computes, and where the pages define it:

* Block pool and tables -- mini-vLLM README, "How it works -- Paged KV-cache":
  the cache is a preallocated set of equal blocks of ``block_size`` tokens,
  and each sequence owns a table that says which physical block holds each
  of its logical blocks.  Logical token ``t`` of a sequence lives in physical
  block ``table[t // block_size]`` at offset ``t % block_size``.
* The cache write -- mini-vLLM README, "End-to-end throughput vs baselines",
  the paragraph on what changed from the previous run: all new K/V go into
  the cache in a single scatter rather than sequence by sequence.  Here: one
  slot per new token, ``slot = block * block_size + offset``; a negative slot
  is skipped.
* Attention -- mini-vLLM README, "Attention kernel path": the CPU path is
  standard scaled dot-product attention; wLLM's PyPI page ("CPU inference")
  likewise describes its CPU decode as a plain-PyTorch fallback with the same
  math as the kernel.  Per query row and head: softmax(scale * q . K^T) V.
* Grouped-query heads -- same mini-vLLM paragraph: each query head reads its
  KV head directly instead of expanding K/V to the query-head count.  The
  grouping is contiguous: head ``h`` uses KV head ``h // (Hq / Hkv)``.
* Chunked prefill -- wLLM PyPI page, "Features -- Core engine": long prompts
  are split into chunks.  A chunk of L query tokens at the end of a context of
  C tokens has its row ``i`` at absolute position ``C - L + i``; it attends to
  keys ``0 .. C - L + i`` (causal, aligned to the end of the context).  A
  decode row is the case L = 1.
* Two attention variants -- wLLM PyPI page, "Supported models": Gemma 2/3
  need sliding-window attention and attention-logit soft-capping, which it
  names as kernel work without defining them.  Read here in their usual
  (Gemma-2) form: soft-capping at ``c`` replaces each scaled score ``x`` by
  ``c * tanh(x / c)`` before the softmax; a sliding window of ``W`` tokens lets
  the row at position ``p`` attend keys ``p - W + 1 .. p`` only.  ``c = 0`` and
  ``W = 0`` switch them off.

Readings where the pages are silent: cache layout ``[num_blocks, Hkv,
block_size, D]``; ``context_lens`` counts the current token(s); an empty
context gives a zero output; the output keeps the query's dtype and is
computed here in float64.

Every function below is pinned by tests in ``tests/test_oracle_pins.py``
(contiguous brute force, permutation and block-size invariance, a library
SDPA, closed forms, planted-mistake detection).
"""
from __future__ import annotations

import numpy as np


def block_of(t: int, block_size: int):
    """Logical token ``t`` -> (logical block index, offset in that block)."""
    return t // block_size, t % block_size


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Contiguous grouped-query mapping: query head ``h`` -> its KV head."""
    return h // (num_heads // num_kv_heads)


def query_position(context_len: int, query_len: int, i: int) -> int:
    """Absolute position of row ``i`` of a chunk of ``query_len`` tokens that
    ends a context of ``context_len`` tokens."""
    return context_len - query_len + i


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, block_size):
    """Slot-mapped cache write on copies of the caches.

    ``key``/``value``: [N, Hkv, D]; caches: [NB, Hkv, bs, D]; ``slot_mapping``:
    [N] int.  Works on any dtype (pass raw integer views for a bit-exact
    comparison).  Returns the new (key_cache, value_cache).
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = block_of(int(slot), block_size)
        kc[b, :, o, :] = key[n]
        vc[b, :, o, :] = value[n]
    return kc, vc


def gather(cache, table_row, context_len: int, block_size: int) -> np.ndarray:
    """Contiguous [C, Hkv, D] float64 copy of a sequence's K or V, read token by
    token through its block table."""
    cache = np.asarray(cache)
    C = int(context_len)
    out = np.empty((C, cache.shape[1], cache.shape[3]), dtype=np.float64)
    for t in range(C):
        lb, o = block_of(t, block_size)
        out[t] = cache[int(table_row[lb]), :, o, :]
    return out


def window_first_key(position: int, window: int) -> int:
    """First key a row at ``position`` attends: the oldest of its ``window``
    most recent positions (its own included), or 0 without a window."""
    return max(0, position - window + 1) if window > 0 else 0


def cap_scores(z, softcap: float):
    """Logit soft-capping of scaled scores: ``softcap * tanh(z / softcap)``;
    ``softcap = 0`` leaves them unchanged."""
    return softcap * np.tanh(np.asarray(z) / softcap) if softcap > 0 else z


def attend(q, K, V, scale: float, positions, return_weights: bool = False,
           softcap: float = 0.0, window: int = 0):
    """softmax(cap(scale * q K^T)) V with a causal limit (and optionally a
    sliding window) per row.

    ``q``: [L, Hq, D]; ``K``/``V``: [C, Hkv, D] (contiguous, position order);
    ``positions[i]``: the last key position row ``i`` may attend.  Returns
    [L, Hq, D] float64 (and the [L, Hq, C] weights if asked).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, Hq, D = q.shape
    C, Hkv = K.shape[0], K.shape[1]
    out = np.zeros((L, Hq, V.shape[2]), dtype=np.float64)
    weights = np.zeros((L, Hq, C), dtype=np.float64)
    for i in range(L):
        n = int(positions[i]) + 1  # keys lo .. positions[i]
        if n <= 0:
            continue
        lo = window_first_key(int(positions[i]), window)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            z = cap_scores(scale * (K[lo:n, g, :] @ q[i, h, :]), softcap)
            e = np.exp(z - z.max())
            w = e / e.sum()
            out[i, h] = w @ V[lo:n, g, :]
            weights[i, h, lo:n] = w
    if return_weights:
        return out, weights
    return out


def paged_decode(query, key_cache, value_cache, block_tables, context_lens, scale,
                 block_size, num_kv_heads=None, softcap: float = 0.0, window: int = 0):
    """One decode token per sequence: row ``s`` of ``query`` ([S, Hq, D]) sits
    at position ``context_lens[s] - 1`` and attends all ``context_lens[s]``
    tokens (the last ``window`` of them with a window).  Returns [S, Hq, D]
    float64 (zeros for an empty context)."""
    query = np.asarray(query, dtype=np.float64)
    S, Hq, D = query.shape
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        C = int(context_lens[s])
        if C <= 0:
            continue
        K = gather(key_cache, block_tables[s], C, block_size)
        V = gather(value_cache, block_tables[s], C, block_size)
        out[s] = attend(query[s:s + 1], K, V, scale, [query_position(C, 1, 0)],
                        softcap=softcap, window=window)[0]
    return out


def paged_prefill_chunk(query, query_start_loc, key_cache, value_cache, block_tables,
                        context_lens, scale, block_size, softcap: float = 0.0, window: int = 0):
    """Chunked-prefill attention.  Sequence ``s`` owns query rows
    ``query_start_loc[s] .. query_start_loc[s+1]-1`` (L rows) and a context of
    ``context_lens[s]`` tokens that already includes the chunk; row ``i`` sits
    at position ``C - L + i``.  Returns [num_q_tokens, Hq, D] float64."""
    query = np.asarray(query, dtype=np.float64)
    out = np.zeros(query.shape, dtype=np.float64)
    S = len(context_lens)
    for s in range(S):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        L, C = b - a, int(context_lens[s])
        if L <= 0 or C <= 0:
            continue
        K = gather(key_cache, block_tables[s], C, block_size)
        V = gather(value_cache, block_tables[s], C, block_size)
        pos = [query_position(C, L, i) for i in range(L)]
        out[a:b] = attend(query[a:b], K, V, scale, pos, softcap=softcap, window=window)
    return out
