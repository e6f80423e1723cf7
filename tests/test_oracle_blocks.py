"""Pins of the oracle's block-pool copies (CPU only).

* a hand-worked example whose expected pool is written out literally;
* blocks that no pair names stay bit-for-bit unchanged, and the inputs are
  not modified (copies are returned);
* a swap round trip (device pool -> host pool -> fresh device pool) gives the
  original blocks back;
* pairs with an id outside their pool are skipped;
* planted mistakes in the oracle are each caught by at least one pin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.blocks as OB


def pin_hand_worked():
    # Four blocks, block b filled with the value 10 * (b + 1); copy 0 -> 3, 2 -> 1.
    pool = np.stack([np.full((2, 3, 4), 10 * (b + 1), dtype=np.int16) for b in range(4)])
    k, v = OB.copy_blocks(pool, pool + 1, [[0, 3], [2, 1]])
    assert k[:, 0, 0, 0].tolist() == [10, 30, 30, 10]
    assert v[:, 0, 0, 0].tolist() == [11, 31, 31, 11]
    assert np.all(k == k[:, :1, :1, :1]) and np.all(v == v[:, :1, :1, :1])  # whole blocks


def pin_untouched_blocks():
    rng = np.random.default_rng(3)
    kc = rng.integers(-2**15, 2**15, size=(9, 2, 4, 8), dtype=np.int16)
    vc = rng.integers(-2**15, 2**15, size=(9, 2, 4, 8), dtype=np.int16)
    kc0, vc0 = kc.copy(), vc.copy()
    mapping = np.array([[5, 0], [7, 2], [1, 8]])
    k, v = OB.copy_blocks(kc, vc, mapping)
    assert np.array_equal(kc, kc0) and np.array_equal(vc, vc0)
    for b in range(9):
        src = {d: s for s, d in mapping.tolist()}.get(b)
        want_k = kc0[src] if src is not None else kc0[b]
        want_v = vc0[src] if src is not None else vc0[b]
        assert np.array_equal(k[b], want_k) and np.array_equal(v[b], want_v)


def pin_swap_round_trip():
    rng = np.random.default_rng(4)
    dev = rng.integers(-2**31, 2**31, size=(12, 3, 16), dtype=np.int32)
    host = np.zeros((5, 3, 16), dtype=np.int32)
    out_ids = [11, 2, 7]
    host_ids = [4, 0, 2]
    host = OB.swap_blocks(dev, host, list(zip(out_ids, host_ids)))
    back = OB.swap_blocks(host, np.zeros_like(dev), list(zip(host_ids, out_ids)))
    for b in range(12):
        assert np.array_equal(back[b], dev[b] if b in out_ids else np.zeros_like(dev[b]))
    assert np.all(host[[1, 3]] == 0)


def pin_out_of_range_skipped():
    pool = np.arange(4 * 6, dtype=np.int16).reshape(4, 6)
    out = OB.swap_blocks(pool, pool, [[-1, 0], [0, 4], [9, 1], [3, 2]])
    want = pool.copy()
    want[2] = pool[3]
    assert np.array_equal(out, want)


PINS = [pin_hand_worked, pin_untouched_blocks, pin_swap_round_trip, pin_out_of_range_skipped]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


_orig_swap = OB.swap_blocks


def _swap_reversed(src_pool, dst_pool, block_mapping):
    m = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)[:, ::-1]
    return _orig_swap(src_pool, dst_pool, m)


def _swap_off_by_one(src_pool, dst_pool, block_mapping):
    m = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2) + np.array([0, 1])
    return _orig_swap(src_pool, dst_pool, m)


def _swap_first_row_only(src_pool, dst_pool, block_mapping):
    src = np.asarray(src_pool)
    out = np.array(dst_pool, copy=True)
    for s, d in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2).tolist():
        if 0 <= s < src.shape[0] and 0 <= d < out.shape[0]:
            out[d][:1] = src[s][:1]
    return out


def _copy_keys_only(key_cache, value_cache, block_mapping):
    return _orig_swap(key_cache, key_cache, block_mapping), np.array(value_cache, copy=True)


MUTANTS = {
    "source_and_destination_swapped": ("swap_blocks", _swap_reversed),
    "destination_off_by_one": ("swap_blocks", _swap_off_by_one),
    "partial_block": ("swap_blocks", _swap_first_row_only),
    "values_not_copied": ("copy_blocks", _copy_keys_only),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OB, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
