"""The test helper that feeds the oracle one sequence at a time (with only
that sequence's blocks) gives bitwise the oracle's whole-pool result, so the
full-size parity tests that use it check the same definition."""
from __future__ import annotations

import numpy as np

from paged_kv_cache_179_amd import workloads as W
from tests.helpers import (decode_workspace_layout, oracle_decode, oracle_decode_per_seq,
                           written_caches)


def test_per_sequence_feed_equals_whole_pool():
    w = W.small_case(5150, num_seqs=9, ctx_lo=1, ctx_hi=300, num_heads=6, num_kv_heads=2,
                     head_dim=64, block_size=16, dtype="bf16", extra_ctx=[1, 16, 17, 0])
    kc, vc = written_caches(w)
    whole = oracle_decode(w, kc, vc)
    per = oracle_decode_per_seq(w, kc, vc)
    assert np.array_equal(whole, per)
    rows = [2, 5, 0]
    assert np.array_equal(oracle_decode(w, kc, vc, rows), oracle_decode_per_seq(w, kc, vc, rows))
    assert np.array_equal(oracle_decode(w, kc, vc, softcap=20.0, window=9),
                          oracle_decode_per_seq(w, kc, vc, softcap=20.0, window=9))


def test_workspace_layout_matches_the_library():
    """The tests' reading of the decode workspace layout (used to read the
    work plan back) has the library's size for every shape tried."""
    import paged_kv_cache_179_amd as pa

    for S, Hq, D, maxc, part in [(1, 4, 64, 100, 512), (7, 28, 128, 3000, 512), (256, 28, 128, 8192, 512),
                                 (40, 8, 256, 1400, 64), (3, 32, 128, 5000, 0), (9, 6, 64, 64, 64)]:
        P = max(1, -(-maxc // part)) if part else 1
        assert decode_workspace_layout(S, Hq, D, P)["bytes"] == pa.decode_workspace_bytes(S, Hq, D, maxc, part)
