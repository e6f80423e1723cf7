"""fp8 (E4M3) KV cache of the CPU oracle (test infrastructure only, like the
rest of ``oracle``: used by ``tests/`` and by nothing on the product path).

The vLLM native-Windows build README lists fp8 among its KV-cache
compression options (release table, "KV compression"); the pages say nothing
more.  Read here as the usual fp8 KV cache: each cached K (and V) element is
stored as one byte in the OCP 8-bit floating-point format E4M3 -- 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN and there is no
infinity, so the largest finite value is 1.75 * 2^8 = 448 -- together with a
per-tensor scale: a cached value is ``decode(byte) * scale``.

Quantisation on write: ``y = float32(x) / float32(scale)`` (correctly rounded
fp32 division), then rounded to the nearest E4M3 value, ties to even, with
saturation: any finite or infinite ``y`` beyond the largest finite value
becomes +-448; NaN becomes 0x7F.

Pinned by ``tests/test_oracle_fp8.py`` (torch's float8_e4m3fn as an
independent codec, exhaustive round trips, hand-checked codes and ties).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import block_of

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 byte."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_encode(y: float) -> int:
    """Nearest E4M3 byte to ``y`` (ties to even), saturating to +-448."""
    y = float(y)
    if math.isnan(y):
        return NAN_CODE
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0x00
    a = abs(y)
    if a >= E4M3_MAX:
        return sign | 0x7E
    # The binade of a (subnormals share the quantum of the lowest binade).
    e = max(math.frexp(a)[1] - 1, -6) if a > 0 else -6
    quantum = 2.0 ** (e - 3)
    n = a / quantum  # exact: a power-of-two division
    r = math.floor(n)
    frac = n - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    value = r * quantum  # <= 448: a < 448 rounds at most up to 448
    if value == 0:
        return sign
    e2 = max(math.frexp(value)[1] - 1, -6)
    if value < 2.0 ** -6:  # subnormal: field 0, mantissa in units of 2^-9
        return sign | int(round(value / 2.0 ** -9))
    m = int(round((value / 2.0 ** e2 - 1.0) * 8))
    return sign | ((e2 + 7) << 3) | m


def quantize(x, scale: float) -> np.ndarray:
    """Bytes of ``x / scale`` (the division in float32, as written above)."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    flat = [e4m3_encode(v) for v in y.reshape(-1).tolist()]
    return np.asarray(flat, dtype=np.uint8).reshape(y.shape)


def dequantize(codes, scale: float) -> np.ndarray:
    """float64 values of E4M3 bytes times ``scale``."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes] * float(scale)


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, block_size,
                          k_scale: float, v_scale: float):
    """The slot-mapped write into E4M3 caches (uint8 arrays [NB, Hkv, bs, D]):
    each new token's K row is quantised with ``k_scale``, its V row with
    ``v_scale``.  Returns new (key_cache, value_cache); negative slots skip."""
    kc = np.array(key_cache, dtype=np.uint8, copy=True)
    vc = np.array(value_cache, dtype=np.uint8, copy=True)
    kq = quantize(key, k_scale)
    vq = quantize(value, v_scale)
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        b, o = block_of(int(slot), block_size)
        kc[b, :, o, :] = kq[n]
        vc[b, :, o, :] = vq[n]
    return kc, vc
