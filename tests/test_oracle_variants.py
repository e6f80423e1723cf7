"""Pins of the oracle's soft-capped and sliding-window attention (CPU only).

* brute force: Python loops with math.tanh and math.fsum over contiguous K/V
  built before they are scattered into a shuffled pool, for decode and
  chunk rows, several caps and windows;
* a window that covers the whole context changes nothing, bit for bit;
* a window of one token returns that token's value row exactly;
* a very large cap approaches plain attention;
* torch's scaled_dot_product_attention with an explicit banded mask (window
  only, float64);
* planted mistakes in the two variant helpers are each caught.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.attention as OA
from tests.test_oracle_pins import make_paged


def brute(q_rows, K, V, scale, first_pos, cap, window):
    """Rows at positions first_pos, first_pos + 1, ...: each attends keys
    max(0, p - W + 1) .. p (all of 0 .. p for W = 0), scores capped to
    cap * tanh(x / cap) (none for cap = 0)."""
    L, Hq, D = q_rows.shape
    G = Hq // K.shape[1]
    out = np.zeros((L, Hq, V.shape[2]))
    for i in range(L):
        p = first_pos + i
        lo = max(0, p - window + 1) if window else 0
        for h in range(Hq):
            g = h // G
            z = []
            for t in range(lo, p + 1):
                x = scale * math.fsum(float(q_rows[i, h, d]) * float(K[t, g, d]) for d in range(D))
                z.append(cap * math.tanh(x / cap) if cap else x)
            zm = max(z)
            e = [math.exp(x - zm) for x in z]
            tot = math.fsum(e)
            for d in range(V.shape[2]):
                out[i, h, d] = math.fsum(e[j] * float(V[lo + j, g, d]) for j in range(len(z))) / tot
    return out


def pin_brute_force():
    rng = np.random.default_rng(21)
    for cap, window in ((0.0, 3), (5.0, 0), (0.7, 7), (2.0, 1), (30.0, 100)):
        for Hq, Hkv, D, bs in ((4, 2, 6, 4), (3, 1, 5, 2)):
            ctx = [1, 6, 17, 23]
            Kc, Vc, kp, vp, bt = make_paged(rng, ctx, Hkv, D, bs)
            q = rng.standard_normal((len(ctx), Hq, D)) * 2.0
            scale = 0.9
            out = OA.paged_decode(q, kp, vp, bt, ctx, scale, bs, softcap=cap, window=window)
            for s, c in enumerate(ctx):
                ref = brute(q[s:s + 1], Kc[s], Vc[s], scale, c - 1, cap, window)
                assert np.max(np.abs(out[s] - ref[0])) <= 1e-12, (cap, window, s)
            lens = [3, 1, 5, 4]
            prior = [0, 6, 9, 13]
            ctx = [p + L for p, L in zip(prior, lens)]
            Kc, Vc, kp, vp, bt = make_paged(rng, ctx, Hkv, D, bs)
            qsl = np.concatenate([[0], np.cumsum(lens)])
            q = rng.standard_normal((int(qsl[-1]), Hq, D)) * 2.0
            out = OA.paged_prefill_chunk(q, qsl, kp, vp, bt, ctx, scale, bs, softcap=cap,
                                         window=window)
            for s in range(len(ctx)):
                a, b = qsl[s], qsl[s + 1]
                ref = brute(q[a:b], Kc[s], Vc[s], scale, prior[s], cap, window)
                assert np.max(np.abs(out[a:b] - ref)) <= 1e-12, (cap, window, s)


def pin_covering_window_is_plain():
    rng = np.random.default_rng(22)
    ctx = [5, 31, 12]
    _, _, kp, vp, bt = make_paged(rng, ctx, 2, 8, 4)
    q = rng.standard_normal((3, 4, 8))
    plain = OA.paged_decode(q, kp, vp, bt, ctx, 0.4, 4)
    assert np.array_equal(plain, OA.paged_decode(q, kp, vp, bt, ctx, 0.4, 4, window=31))
    assert np.array_equal(plain, OA.paged_decode(q, kp, vp, bt, ctx, 0.4, 4, window=1000))
    assert not np.allclose(plain, OA.paged_decode(q, kp, vp, bt, ctx, 0.4, 4, window=30))


def pin_window_of_one():
    rng = np.random.default_rng(23)
    ctx = [9, 1, 16]
    _, Vc, kp, vp, bt = make_paged(rng, ctx, 2, 8, 4)
    q = rng.standard_normal((3, 6, 8))
    out = OA.paged_decode(q, kp, vp, bt, ctx, 0.6, 4, softcap=3.0, window=1)
    for s, c in enumerate(ctx):
        for h in range(6):
            assert np.array_equal(out[s, h], Vc[s][c - 1, h // 3])


def pin_large_cap_is_plain():
    rng = np.random.default_rng(24)
    ctx = [14, 40]
    _, _, kp, vp, bt = make_paged(rng, ctx, 1, 8, 8)
    q = rng.standard_normal((2, 2, 8)) * 3
    plain = OA.paged_decode(q, kp, vp, bt, ctx, 0.5, 8)
    capped = OA.paged_decode(q, kp, vp, bt, ctx, 0.5, 8, softcap=1e7)
    assert np.max(np.abs(plain - capped)) <= 1e-9
    small = OA.paged_decode(q, kp, vp, bt, ctx, 0.5, 8, softcap=0.5)
    assert np.max(np.abs(plain - small)) > 1e-3  # a small cap does change the result


def pin_torch_sdpa_band():
    rng = np.random.default_rng(25)
    for Hq, Hkv, W in ((4, 4, 3), (6, 2, 5), (8, 1, 1)):
        lens = [4, 1, 6]
        prior = [5, 0, 11]
        ctx = [p + L for p, L in zip(prior, lens)]
        D = 8
        Kc, Vc, kp, vp, bt = make_paged(rng, ctx, Hkv, D, 4)
        qsl = np.concatenate([[0], np.cumsum(lens)])
        q = rng.standard_normal((int(qsl[-1]), Hq, D))
        out = OA.paged_prefill_chunk(q, qsl, kp, vp, bt, ctx, 0.31, 4, window=W)
        for s in range(len(ctx)):
            a, b = qsl[s], qsl[s + 1]
            L, C = b - a, ctx[s]
            qt = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]
            kt = torch.from_numpy(Kc[s]).permute(1, 0, 2)[None].contiguous()
            vt = torch.from_numpy(Vc[s]).permute(1, 0, 2)[None].contiguous()
            pos = (C - L + torch.arange(L))[:, None]
            t = torch.arange(C)[None, :]
            mask = (t <= pos) & (t > pos - W)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, attn_mask=mask, scale=0.31, enable_gqa=(Hq != Hkv))
            ref = ref[0].permute(1, 0, 2).numpy()
            assert np.max(np.abs(out[a:b] - ref)) <= 1e-12


PINS = [pin_brute_force, pin_covering_window_is_plain, pin_window_of_one, pin_large_cap_is_plain,
        pin_torch_sdpa_band]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


MUTANTS = {
    "window_off_by_one": ("window_first_key", lambda p, w: max(0, p - w) if w > 0 else 0),
    "window_ignored": ("window_first_key", lambda p, w: 0),
    "cap_without_outer_factor": ("cap_scores", lambda z, c: np.tanh(np.asarray(z) / c) if c > 0 else z),
    "cap_ignored": ("cap_scores", lambda z, c: z),
    "cap_as_clamp": ("cap_scores", lambda z, c: np.clip(z, -c, c) if c > 0 else z),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
