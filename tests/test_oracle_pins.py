"""Pins of the fp64 oracle to things other than itself (CPU only).

* P1  a one-token context returns that token's value row exactly;
* P2  contiguous brute force: Python loops with math.fsum over K/V laid out
      contiguously *before* they are scattered into a shuffled pool;
* P3  relabelling physical blocks (pool permuted, tables remapped) changes
      nothing, bit for bit;
* P4  the same logical K/V paged with block_size 1 and 16 give identical bits;
* P5  torch's scaled_dot_product_attention in float64 with an explicit
      end-aligned causal mask and its own grouped-query expansion;
* P6  closed forms: scale 0 gives the mean of the attended rows, identical V
      rows give that row, a chunk row equals a decode over its prefix;
* P7  softmax weights are non-negative and sum to 1;
* P8  the cache write changes exactly the addressed slots, bit for bit;
* hand-derived golden fixtures (tests/golden/);
* planted mistakes in the oracle (wrong head mapping, off-by-one causal
  limit, swapped block/offset, dropped scale, swapped K/V, ...) are each
  caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Independent builders (no oracle code).
# ---------------------------------------------------------------------------
def make_paged(rng, ctx_list, num_kv_heads, head_dim, block_size, extra_blocks=3):
    """Contiguous per-sequence K/V, then a shuffled pool holding them."""
    Kc = [rng.standard_normal((c, num_kv_heads, head_dim)) for c in ctx_list]
    Vc = [rng.standard_normal((c, num_kv_heads, head_dim)) for c in ctx_list]
    nblk = [(c + block_size - 1) // block_size for c in ctx_list]
    total = sum(nblk) + extra_blocks
    perm = rng.permutation(total)
    kpool = rng.standard_normal((total, num_kv_heads, block_size, head_dim)) * 100.0
    vpool = rng.standard_normal((total, num_kv_heads, block_size, head_dim)) * 100.0
    mbps = max(1, max(nblk) if nblk else 1)
    tables = np.full((len(ctx_list), mbps), -1, dtype=np.int64)
    cur = 0
    for s, c in enumerate(ctx_list):
        for j in range(nblk[s]):
            b = int(perm[cur])
            cur += 1
            tables[s, j] = b
            for o in range(block_size):
                t = j * block_size + o
                if t < c:
                    kpool[b, :, o, :] = Kc[s][t]
                    vpool[b, :, o, :] = Vc[s][t]
    return Kc, Vc, kpool, vpool, tables


def brute_rows(q_rows, K, V, scale, first_pos):
    """Attention of rows at positions first_pos, first_pos+1, ... over
    contiguous K/V [C][Hkv][D], with Python loops and math.fsum."""
    L, Hq, D = q_rows.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((L, Hq, V.shape[2]))
    for i in range(L):
        n = first_pos + i + 1
        for h in range(Hq):
            g = h // G
            z = [scale * math.fsum(float(q_rows[i, h, d]) * float(K[t, g, d]) for d in range(D))
                 for t in range(n)]
            zm = max(z)
            e = [math.exp(x - zm) for x in z]
            tot = math.fsum(e)
            for d in range(V.shape[2]):
                out[i, h, d] = math.fsum(e[t] * float(V[t, g, d]) for t in range(n)) / tot
    return out


# ---------------------------------------------------------------------------
# Pins, written against the module object so planted mistakes reach them.
# ---------------------------------------------------------------------------
def pin_single_token_context():
    rng = np.random.default_rng(1)
    for Hq, Hkv in ((4, 2), (3, 3), (8, 1)):
        _, Vc, kp, vp, bt = make_paged(rng, [1, 1], Hkv, 8, 4)
        q = rng.standard_normal((2, Hq, 8))
        out = OA.paged_decode(q, kp, vp, bt, [1, 1], 0.7, 4)
        G = Hq // Hkv
        for s in range(2):
            for h in range(Hq):
                assert np.array_equal(out[s, h], Vc[s][0, h // G]), "C=1 must return v0 exactly"


def pin_decode_brute_force():
    rng = np.random.default_rng(2)
    for Hq, Hkv, D, bs in ((4, 2, 8, 4), (6, 3, 5, 1), (4, 4, 6, 16), (8, 1, 4, 2)):
        ctx = [1, 5, 16, 17, 23]
        Kc, Vc, kp, vp, bt = make_paged(rng, ctx, Hkv, D, bs)
        q = rng.standard_normal((len(ctx), Hq, D))
        scale = 1.0 / math.sqrt(D)
        out = OA.paged_decode(q, kp, vp, bt, ctx, scale, bs)
        for s, c in enumerate(ctx):
            ref = brute_rows(q[s:s + 1], Kc[s], Vc[s], scale, c - 1)
            assert np.max(np.abs(out[s] - ref[0])) <= 1e-12


def pin_prefill_brute_force():
    rng = np.random.default_rng(3)
    for Hq, Hkv, D, bs in ((4, 2, 6, 4), (3, 1, 5, 2), (2, 2, 4, 8)):
        lens = [3, 1, 5, 4]
        prior = [0, 6, 9, 13]
        ctx = [p + L for p, L in zip(prior, lens)]
        Kc, Vc, kp, vp, bt = make_paged(rng, ctx, Hkv, D, bs)
        qsl = np.concatenate([[0], np.cumsum(lens)])
        q = rng.standard_normal((int(qsl[-1]), Hq, D))
        scale = 0.37
        out = OA.paged_prefill_chunk(q, qsl, kp, vp, bt, ctx, scale, bs)
        for s in range(len(ctx)):
            a, b = qsl[s], qsl[s + 1]
            ref = brute_rows(q[a:b], Kc[s], Vc[s], scale, prior[s])
            assert np.max(np.abs(out[a:b] - ref)) <= 1e-12


def pin_permutation_invariance():
    rng = np.random.default_rng(4)
    ctx = [7, 33, 2]
    _, _, kp, vp, bt = make_paged(rng, ctx, 2, 8, 4)
    q = rng.standard_normal((3, 4, 8))
    base = OA.paged_decode(q, kp, vp, bt, ctx, 0.5, 4)
    pi = rng.permutation(kp.shape[0])
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1)
    again = OA.paged_decode(q, kp2, vp2, bt2, ctx, 0.5, 4)
    assert np.array_equal(base, again)
    qsl = [0, 2, 5, 6]
    qp = rng.standard_normal((6, 4, 8))
    a = OA.paged_prefill_chunk(qp, qsl, kp, vp, bt, ctx, 0.5, 4)
    b = OA.paged_prefill_chunk(qp, qsl, kp2, vp2, bt2, ctx, 0.5, 4)
    assert np.array_equal(a, b)


def pin_block_size_equivalence():
    rng = np.random.default_rng(5)
    ctx = [31, 16, 1]
    Kc, Vc, kp16, vp16, bt16 = make_paged(rng, ctx, 2, 8, 16)
    # Same logical tokens, one token per block, another random placement.
    n = sum(ctx)
    perm = rng.permutation(n + 4)
    kp1 = rng.standard_normal((n + 4, 2, 1, 8))
    vp1 = rng.standard_normal((n + 4, 2, 1, 8))
    bt1 = np.full((3, max(ctx)), -1, dtype=np.int64)
    cur = 0
    for s, c in enumerate(ctx):
        for t in range(c):
            b = int(perm[cur])
            cur += 1
            bt1[s, t] = b
            kp1[b, :, 0, :] = Kc[s][t]
            vp1[b, :, 0, :] = Vc[s][t]
    q = rng.standard_normal((3, 4, 8))
    a = OA.paged_decode(q, kp16, vp16, bt16, ctx, 0.3, 16)
    b = OA.paged_decode(q, kp1, vp1, bt1, ctx, 0.3, 1)
    assert np.array_equal(a, b)


def pin_torch_sdpa():
    rng = np.random.default_rng(6)
    for Hq, Hkv in ((4, 4), (6, 2), (8, 1)):
        lens = [4, 1, 6]
        prior = [5, 0, 11]
        ctx = [p + L for p, L in zip(prior, lens)]
        D = 8
        Kc, Vc, kp, vp, bt = make_paged(rng, ctx, Hkv, D, 4)
        qsl = np.concatenate([[0], np.cumsum(lens)])
        q = rng.standard_normal((int(qsl[-1]), Hq, D))
        scale = 0.29
        out = OA.paged_prefill_chunk(q, qsl, kp, vp, bt, ctx, scale, 4)
        for s in range(len(ctx)):
            a, b = qsl[s], qsl[s + 1]
            L, C = b - a, ctx[s]
            qt = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]           # [1, Hq, L, D]
            kt = torch.from_numpy(Kc[s]).permute(1, 0, 2)[None].contiguous()  # [1, Hkv, C, D]
            vt = torch.from_numpy(Vc[s]).permute(1, 0, 2)[None].contiguous()
            i = torch.arange(L)[:, None]
            t = torch.arange(C)[None, :]
            mask = t <= (C - L + i)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=(Hq != Hkv))
            ref = ref[0].permute(1, 0, 2).numpy()
            assert np.max(np.abs(out[a:b] - ref)) <= 1e-12


def pin_closed_forms():
    rng = np.random.default_rng(7)
    ctx = [9, 20]
    Kc, Vc, kp, vp, bt = make_paged(rng, ctx, 2, 4, 4)
    lens = [3, 5]
    qsl = [0, 3, 8]
    q = rng.standard_normal((8, 4, 4))
    # scale 0 -> uniform weights over the attended prefix
    out = OA.paged_prefill_chunk(q, qsl, kp, vp, bt, ctx, 0.0, 4)
    for s in range(2):
        for i in range(lens[s]):
            n = ctx[s] - lens[s] + i + 1
            for h in range(4):
                mean = Vc[s][:n, h // 2].mean(axis=0)
                assert np.max(np.abs(out[qsl[s] + i, h] - mean)) <= 1e-12
    # identical V rows -> that row, whatever the weights
    vconst = vp.copy()
    vconst[...] = np.array([1.5, -2.0, 0.25, 3.0])
    out = OA.paged_decode(q[:2], kp, vconst, bt, ctx, 0.9, 4)
    assert np.max(np.abs(out - np.array([1.5, -2.0, 0.25, 3.0]))) <= 1e-12
    # a chunk row equals a decode over the tokens up to its position
    out = OA.paged_prefill_chunk(q, qsl, kp, vp, bt, ctx, 0.45, 4)
    for s in range(2):
        for i in range(lens[s]):
            n = ctx[s] - lens[s] + i + 1
            dec = OA.paged_decode(q[qsl[s] + i][None], kp, vp, bt[s:s + 1], [n], 0.45, 4)
            assert np.max(np.abs(out[qsl[s] + i] - dec[0])) <= 1e-13


def pin_weights_normalised():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((5, 4, 8)) * 3
    K = rng.standard_normal((12, 2, 8)) * 3
    V = rng.standard_normal((12, 2, 8))
    _, w = OA.attend(q, K, V, 0.8, [7, 8, 9, 10, 11], return_weights=True)
    assert (w >= 0).all()
    for i in range(5):
        n = 8 + i
        assert np.all(np.abs(w[i, :, :n].sum(axis=1) - 1.0) <= 1e-15 * n)
        assert np.all(w[i, :, n:] == 0)


def pin_cache_write():
    rng = np.random.default_rng(9)
    nb, hkv, bs, d = 6, 2, 4, 8
    kc = rng.integers(-2**15, 2**15, size=(nb, hkv, bs, d), dtype=np.int16)
    vc = rng.integers(-2**15, 2**15, size=(nb, hkv, bs, d), dtype=np.int16)
    key = rng.integers(-2**15, 2**15, size=(5, hkv, d), dtype=np.int16)
    val = rng.integers(-2**15, 2**15, size=(5, hkv, d), dtype=np.int16)
    slots = np.array([9, -1, 0, 23, 14])
    k2, v2 = OA.reshape_and_cache(key, val, kc, vc, slots, bs)
    touched = np.zeros((nb, bs), dtype=bool)
    for n, s in enumerate(slots):
        if s < 0:
            continue
        b, o = s // bs, s % bs  # slot = block * block_size + offset
        touched[b, o] = True
        assert np.array_equal(k2[b, :, o, :], key[n]) and np.array_equal(v2[b, :, o, :], val[n])
    for b in range(nb):
        for o in range(bs):
            if not touched[b, o]:
                assert np.array_equal(k2[b, :, o], kc[b, :, o]) and np.array_equal(v2[b, :, o], vc[b, :, o])
    assert np.array_equal(kc, kc.copy())  # inputs untouched (copies returned)


def pin_golden_fixtures():
    with open(os.path.join(GOLDEN, "two_token_weights.json")) as f:
        g = json.load(f)
    out = OA.paged_decode(np.array(g["query"]), np.array(g["key_cache"]), np.array(g["value_cache"]),
                          np.array(g["block_tables"]), g["context_lens"], g["scale"], g["block_size"])
    assert np.max(np.abs(out - np.array(g["expected"]))) <= g["tolerance"]
    with open(os.path.join(GOLDEN, "gqa_chunk_uniform.json")) as f:
        g = json.load(f)
    out = OA.paged_prefill_chunk(np.array(g["query"]), g["query_start_loc"], np.array(g["key_cache"]),
                                 np.array(g["value_cache"]), np.array(g["block_tables"]),
                                 g["context_lens"], g["scale"], g["block_size"])
    assert np.max(np.abs(out - np.array(g["expected"]))) <= g["tolerance"]


PINS = [pin_single_token_context, pin_decode_brute_force, pin_prefill_brute_force,
        pin_permutation_invariance, pin_block_size_equivalence, pin_torch_sdpa, pin_closed_forms,
        pin_weights_normalised, pin_cache_write, pin_golden_fixtures]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------
_orig_attend = OA.attend
_orig_gather = OA.gather
_orig_write = OA.reshape_and_cache


def _attend_unnormalised(q, K, V, scale, positions, return_weights=False):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, Hq, _ = q.shape
    out = np.zeros((L, Hq, V.shape[2]))
    w_all = np.zeros((L, Hq, K.shape[0]))
    for i in range(L):
        n = int(positions[i]) + 1
        for h in range(Hq):
            g = OA.kv_head_of(h, Hq, K.shape[1])
            z = scale * (K[:n, g, :] @ q[i, h, :])
            w = np.exp(z - z.max())  # missing division by the sum
            out[i, h] = w @ V[:n, g, :]
            w_all[i, h, :n] = w
    return (out, w_all) if return_weights else out


def _write_swapped(key, value, key_cache, value_cache, slot_mapping, block_size):
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = slot % block_size, slot // block_size  # block and offset swapped
        if b < kc.shape[0] and o < kc.shape[2]:
            kc[b, :, o, :] = key[n]
            vc[b, :, o, :] = value[n]
    return kc, vc


def _write_k_into_v(key, value, key_cache, value_cache, slot_mapping, block_size):
    return _orig_write(key, key, key_cache, value_cache, slot_mapping, block_size)


MUTANTS = {
    "gqa_modulo_mapping": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "causal_off_by_one": ("query_position", lambda C, L, i: C - L + i - 1),
    "causal_top_left": ("query_position", lambda C, L, i: i),
    "block_offset_swapped": ("block_of", lambda t, bs: (t % bs, t // bs)),
    "offset_rotated_in_block": ("block_of", lambda t, bs: (t // bs, (t + 1) % bs)),
    "scale_dropped": ("attend", lambda q, K, V, s, p, return_weights=False:
                      _orig_attend(q, K, V, 1.0, p, return_weights)),
    "k_v_swapped": ("attend", lambda q, K, V, s, p, return_weights=False:
                    _orig_attend(q, V, K, s, p, return_weights)),
    "v_rows_reversed": ("attend", lambda q, K, V, s, p, return_weights=False:
                        _orig_attend(q, K, np.asarray(V)[::-1], s, p, return_weights)),
    "gather_head_zero": ("gather", lambda c, row, C, bs:
                         np.repeat(_orig_gather(c, row, C, bs)[:, :1], np.asarray(c).shape[1], axis=1)),
    "softmax_unnormalised": ("attend", _attend_unnormalised),
    "write_block_offset_swapped": ("reshape_and_cache", _write_swapped),
    "write_key_into_value": ("reshape_and_cache", _write_k_into_v),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion or a crash both count as detection
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
