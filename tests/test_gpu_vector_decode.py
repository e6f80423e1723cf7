"""The vector decode kernel on 16-bit caches (PA_DECODE_KERNEL=vector), the
baseline the MFMA kernel is measured against: parity with the fp64 oracle.

The switch is read once per process, so the cases run in a child process
with the variable set; the child prints each case before it runs it.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

CASES = [
    # dtype, Hq, Hkv, D, bs, partition
    ("fp16", 8, 8, 128, 16, 512),    # MHA (G = 1)
    ("bf16", 28, 4, 128, 16, 512),   # G = 7
    ("bf16", 28, 4, 128, 16, 64),
    ("bf16", 8, 1, 256, 16, 512),
    ("bf16", 32, 4, 64, 32, 0),
]


def child() -> None:
    import torch

    import paged_kv_cache_179_amd as pa
    from paged_kv_cache_179_amd import workloads as W
    from tests.helpers import TOL, max_err, oracle_decode, to_dev, written_caches

    dev = torch.device("cuda:0")
    for dtype, hq, hkv, d_, bs, part in CASES:
        print(f"vector decode {dtype} h{hq}x{hkv} d{d_} bs{bs} part {part}", flush=True)
        w = W.small_case(300 + hq + d_ + bs, num_seqs=7, ctx_lo=1, ctx_hi=1300, num_heads=hq,
                         num_kv_heads=hkv, head_dim=d_, block_size=bs, dtype=dtype,
                         extra_ctx=[1, 2, 512, 513, 1025])
        d = to_dev(w, dev)
        pa.reshape_and_cache(d["new_key"], d["new_value"], d["key_cache"], d["value_cache"],
                             d["slot_mapping"])
        out = torch.full_like(d["query_decode"], float("nan"))
        maxc = int(w.context_lens[w.decode_rows].max())
        pa.decode(out, d["query_decode"], d["key_cache"], d["value_cache"], d["bt_decode"],
                  d["cl_decode"], w.scale, maxc, partition_size=part)
        torch.cuda.synchronize()
        kc, vc = written_caches(w)
        err = max_err(out, oracle_decode(w, kc, vc))
        print(f"  max abs err {err:.3e}", flush=True)
        assert err <= TOL[dtype], (dtype, hq, hkv, d_, bs, part, err)
    print("all cases within tolerance", flush=True)


@pytest.mark.gpu
def test_vector_kernel_on_16bit_caches(gpu):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PA_DECODE_KERNEL="vector")
    r = subprocess.run([sys.executable, "-u", "-m", "tests.test_gpu_vector_decode"], cwd=root, env=env,
                       capture_output=True, text=True, timeout=300)
    sys.stderr.write(r.stdout[-4000:] + r.stderr[-4000:])
    assert r.returncode == 0
    assert "all cases within tolerance" in r.stdout


if __name__ == "__main__":
    child()
