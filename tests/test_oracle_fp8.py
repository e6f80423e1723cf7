"""Pins of the oracle's E4M3 codec and fp8 cache write (CPU only).

* decoding: all 256 codes against torch's float8_e4m3fn (an independent
  implementation of the same OCP format), and hand-checked codes;
* encoding: torch agrees on every value that does not overflow (random values,
  every exactly representable value, and every midpoint between neighbours,
  where ties must go to the even code); saturation and NaN as specified;
* the fp8 cache write quantises exactly the addressed slots;
* planted mistakes in the codec are each caught.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.fp8 as OF


def torch_decode(codes):
    return torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_decode_table():
    ref = torch_decode(list(range(256)))
    for c in range(256):
        got = OF.e4m3_decode(c)
        assert (math.isnan(ref[c]) and math.isnan(got)) or ref[c] == got, c
    hand = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x77: 240.0, 0x40: 2.0, 0x3C: 1.5}
    for c, v in hand.items():
        assert OF.e4m3_decode(c) == v, hex(c)
    assert math.isnan(OF.e4m3_decode(0x7F)) and math.isnan(OF.e4m3_decode(0xFF))
    assert math.copysign(1.0, OF.e4m3_decode(0x80)) < 0


def pin_encode_against_torch():
    finite = [OF.e4m3_decode(c) for c in range(256) if not math.isnan(OF.e4m3_decode(c))]
    pos = sorted(set(abs(v) for v in finite))
    mids = [(a + b) / 2 for a, b in zip(pos, pos[1:])]
    rng = np.random.default_rng(11)
    rand = (rng.standard_normal(20000) * rng.choice([0.01, 1.0, 40.0], 20000)).tolist()
    vals = [v for v in finite + mids + [-m for m in mids] + rand if abs(v) < 464.0]
    ref = torch_encode(vals)
    got = np.array([OF.e4m3_encode(v) for v in vals], dtype=np.uint8)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(vals[i], hex(ref[i]), hex(got[i])) for i in bad[:5]]
    # round trip of every finite code, the sign of zero included
    for c in range(256):
        if not math.isnan(OF.e4m3_decode(c)):
            assert OF.e4m3_encode(OF.e4m3_decode(c)) == c, hex(c)


def pin_ties_saturation_nan():
    assert OF.e4m3_encode(1.0625) == 0x38      # midway 1.0 / 1.125: even mantissa 0
    assert OF.e4m3_encode(1.1875) == 0x3A      # midway 1.125 / 1.25: even mantissa 2
    assert OF.e4m3_encode(2.0 ** -10) == 0x00  # midway 0 / 2^-9: even
    assert OF.e4m3_encode(3 * 2.0 ** -10) == 0x02  # midway 2^-9 / 2^-8: even (2)
    for big in (448.0001, 464.0, 1e30, math.inf):
        assert OF.e4m3_encode(big) == 0x7E and OF.e4m3_encode(-big) == 0xFE
    assert OF.e4m3_encode(math.nan) == 0x7F


def pin_fp8_cache_write():
    rng = np.random.default_rng(12)
    nb, hkv, bs, d = 5, 2, 4, 8
    kc = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    key = rng.standard_normal((4, hkv, d)).astype(np.float32) * 3
    val = rng.standard_normal((4, hkv, d)).astype(np.float32) * 3
    slots = np.array([7, -1, 0, 19])
    k2, v2 = OF.reshape_and_cache_fp8(key, val, kc, vc, slots, bs, 0.02, 0.5)
    for n, s in enumerate(slots):
        if s < 0:
            continue
        b, o = s // bs, s % bs
        for h in range(hkv):
            for j in range(d):
                assert k2[b, h, o, j] == OF.e4m3_encode(float(np.float32(key[n, h, j]) / np.float32(0.02)))
                assert v2[b, h, o, j] == OF.e4m3_encode(float(np.float32(val[n, h, j]) / np.float32(0.5)))
    touched = {(s // bs, s % bs) for s in slots if s >= 0}
    for b in range(nb):
        for o in range(bs):
            if (b, o) not in touched:
                assert np.array_equal(k2[b, :, o], kc[b, :, o]) and np.array_equal(v2[b, :, o], vc[b, :, o])
    # slot 0 holds token 2: dequantised within half a quantum (at most 16 * scale
    # below 448 * scale), or saturated at +-448 * scale
    deq = OF.dequantize(k2, 0.02)[0, :, 0, :]
    inside = np.abs(key[2]) < 448 * 0.02
    assert np.all(np.abs(deq - key[2])[inside] <= 16 * 0.02)
    assert np.all(np.abs(deq[~inside]) == 448 * 0.02)


PINS = [pin_decode_table, pin_encode_against_torch, pin_ties_saturation_nan, pin_fp8_cache_write]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


_orig_encode = OF.e4m3_encode


def _decode_bias8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8) * 2.0 ** -7
    return sign * (1 + m / 8) * 2.0 ** (e - 8)


def _encode_half_up(y):
    y = float(y)
    if math.isnan(y):
        return 0x7F
    a = abs(y)
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    if a >= 448.0:
        return sign | 0x7E
    e = max(math.frexp(a)[1] - 1, -6) if a > 0 else -6
    q = 2.0 ** (e - 3)
    v = math.floor(a / q + 0.5) * q
    return _orig_encode(math.copysign(v, y))


def _encode_overflow_nan(y):
    return 0x7F if abs(float(y)) >= 448.0 and not math.isnan(y) and abs(float(y)) > 448.0 else _orig_encode(y)


def _decode_subnormal_wrong(code):
    code = int(code) & 0xFF
    if (code >> 3) & 0xF == 0:
        return (-1.0 if code & 0x80 else 1.0) * (code & 7) / 8 * 2.0 ** -7
    return OF_decode_orig(code)


OF_decode_orig = OF.e4m3_decode

MUTANTS = {
    "exponent_bias_8": ("e4m3_decode", _decode_bias8),
    "ties_away_from_zero": ("e4m3_encode", _encode_half_up),
    "overflow_to_nan": ("e4m3_encode", _encode_overflow_nan),
    "subnormal_scale": ("e4m3_decode", _decode_subnormal_wrong),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OF, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
