"""pa_decode_noalloc (the decode entry point that allocates nothing) against
pa_decode with its own workspace, through the C ABI: two calls in a row on the
shared fixed scratch, the second with a smaller input, each compared bitwise
with pa_decode (the same kernels) and with the oracle at the usual tolerance;
and a call too large for the scratch rejected before anything is launched."""
from __future__ import annotations

import sys

import pytest
import torch

import paged_kv_cache_179_amd as pa
from paged_kv_cache_179_amd import workloads as W
from tests.helpers import TOL, max_err, oracle_decode, to_dev, written_caches

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # seed, seqs, ctx range, Hq, Hkv, D, bs, dtype, extra contexts, partition, cap, window
    (6101, 64, (1, 3000), 28, 4, 128, 16, "bf16", [1, 512, 513, 2048], 512, 0.0, 0),
    (6102, 9, (1, 900), 8, 8, 64, 16, "fp16", [1, 64, 65], 64, 30.0, 300),
]


def test_noalloc_two_calls_match_decode(gpu):
    for i, (seed, s, (lo, hi), hq, hkv, d_, bs, dt, extra, part, cap, win) in enumerate(CASES):
        say(f"noalloc call {i}: {s} seqs, Hq {hq}/Hkv {hkv}, D {d_}, {dt}, partition {part}")
        w = W.small_case(seed, num_seqs=s, ctx_lo=lo, ctx_hi=hi, num_heads=hq, num_kv_heads=hkv,
                         head_dim=d_, block_size=bs, dtype=dt, extra_ctx=extra)
        d = to_dev(w, gpu)
        pa.reshape_and_cache(d["new_key"], d["new_value"], d["key_cache"], d["value_cache"],
                             d["slot_mapping"])
        maxc = int(w.context_lens.max())
        ref_out = torch.full_like(d["query_decode"], float("nan"))
        pa.decode(ref_out, d["query_decode"], d["key_cache"], d["value_cache"], d["bt_decode"],
                  d["cl_decode"], w.scale, maxc, partition_size=part, logit_softcap=cap,
                  sliding_window=win)
        out = torch.full_like(d["query_decode"], float("nan"))
        pa.decode_noalloc(out, d["query_decode"], d["key_cache"], d["value_cache"],
                          d["bt_decode"], d["cl_decode"], w.scale, maxc, partition_size=part,
                          logit_softcap=cap, sliding_window=win)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "noalloc output differs from pa_decode"
        kc, vc = written_caches(w)
        err = max_err(out, oracle_decode(w, kc, vc, softcap=cap, window=win))
        say(f"  max abs err {err:.3e}")
        assert err <= TOL[dt]


def test_noalloc_rejects_calls_beyond_the_scratch(gpu):
    """A call whose partition states exceed the fixed scratch raises (status
    PA_ERR_TOO_LARGE) and leaves the output untouched."""
    s, hq, hkv, d_, mbps, maxc = 2048, 64, 8, 256, 512, 8192
    need = pa.decode_workspace_bytes(s, hq, d_, maxc, 512)
    assert need > 64 << 20
    q = torch.zeros((s, hq, d_), dtype=torch.bfloat16, device=gpu)
    out = torch.full_like(q, 7.0)
    kc = torch.zeros((4, hkv, 16, d_), dtype=torch.bfloat16, device=gpu)
    bt = torch.zeros((s, mbps), dtype=torch.int32, device=gpu)
    cl = torch.ones((s,), dtype=torch.int32, device=gpu)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode_noalloc(out, q, kc, kc, bt, cl, 0.0625, maxc, partition_size=512)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
