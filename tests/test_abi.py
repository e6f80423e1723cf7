"""The C ABI loads, exports every declared symbol, and rejects bad arguments
on the host (CPU only: every call here fails validation, so nothing is ever
launched)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from paged_kv_cache_179_amd import binding

# The validation tests pass placeholder device pointers that must never reach
# a kernel; keep them off machines where a launch could actually happen.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-validation tests use placeholder pointers")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

OK, NULLP, SHAPE, UNSUP, WS, LAUNCH = 0, 1, 2, 3, 4, 5
F32, F16, BF16 = 0, 1, 2
P = ctypes.c_void_p(1 << 20)  # non-null, 256-aligned; never dereferenced (validation fails first)
N = None


@pytest.fixture(scope="module")
def lib():
    if not binding.library_path().exists():
        from paged_kv_cache_179_amd.build import build

        build()
    return binding.library()


def declared_functions():
    names = []
    for fn in sorted(os.listdir(HEADER_DIR)):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(pa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"pa_reshape_and_cache", "pa_decode", "pa_prefill_chunk"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(binding.EXPORTED) == set(names), "binding and header disagree"


def test_status_strings(lib):
    for s in range(7):
        assert lib.pa_status_str(s) and lib.pa_status_str(s) != b"unknown status"
    assert lib.pa_status_str(99) == b"unknown status"
    assert lib.pa_version() >= 100


def write(lib, key=P, value=P, kc=P, vc=P, slots=P, n=4, hkv=2, d=64, bs=16, nb=8, dt=BF16):
    return lib.pa_reshape_and_cache(key, value, kc, vc, slots, n, hkv, d, bs, nb, dt, N)


def test_write_validation(lib):
    assert write(lib, n=-1) == SHAPE
    assert write(lib, hkv=0) == SHAPE
    assert write(lib, d=96) == UNSUP
    assert write(lib, bs=3) == UNSUP
    assert write(lib, bs=512) == UNSUP
    assert write(lib, dt=7) == UNSUP
    assert write(lib, key=N) == NULLP
    assert write(lib, slots=N) == NULLP
    assert write(lib, kc=ctypes.c_void_p((1 << 20) + 8)) == UNSUP  # misaligned
    assert write(lib, n=0, key=N, value=N, kc=N, vc=N, slots=N) == OK  # empty is a no-op


def copy_blocks(lib, kc=P, vc=P, m=P, n=4, hkv=2, d=64, bs=16, nb=8, dt=BF16):
    return lib.pa_copy_blocks(kc, vc, m, n, hkv, d, bs, nb, dt, N)


def swap_blocks(lib, src=P, dst=P, m=P, n=4, bb=4096, sn=8, dn=8):
    return lib.pa_swap_blocks(src, dst, m, n, bb, sn, dn, N)


def test_block_ops_validation(lib):
    assert copy_blocks(lib, n=-1) == SHAPE
    assert copy_blocks(lib, hkv=0) == SHAPE
    assert copy_blocks(lib, nb=-1) == SHAPE
    assert copy_blocks(lib, d=96) == UNSUP
    assert copy_blocks(lib, bs=3) == UNSUP
    assert copy_blocks(lib, dt=7) == UNSUP
    assert copy_blocks(lib, kc=N) == NULLP
    assert copy_blocks(lib, vc=N) == NULLP
    assert copy_blocks(lib, m=N) == NULLP
    assert copy_blocks(lib, kc=ctypes.c_void_p((1 << 20) + 8)) == UNSUP
    assert copy_blocks(lib, m=ctypes.c_void_p((1 << 20) + 4)) == UNSUP
    assert copy_blocks(lib, n=0, kc=N, vc=N, m=N) == OK  # empty is a no-op
    assert swap_blocks(lib, n=-1) == SHAPE
    assert swap_blocks(lib, bb=0) == SHAPE
    assert swap_blocks(lib, sn=-1) == SHAPE
    assert swap_blocks(lib, dn=-1) == SHAPE
    assert swap_blocks(lib, bb=24) == UNSUP  # not a multiple of 16
    assert swap_blocks(lib, src=N) == NULLP
    assert swap_blocks(lib, dst=N) == NULLP
    assert swap_blocks(lib, m=N) == NULLP
    assert swap_blocks(lib, dst=ctypes.c_void_p((1 << 20) + 8)) == UNSUP
    assert swap_blocks(lib, n=0, src=N, dst=N, m=N) == OK


def test_stream_probe_validation(lib):
    probe = lib.pa_stream_read_probe
    assert probe(P, 0, P, 1, N) == SHAPE
    assert probe(P, 24, P, 1, N) == SHAPE  # not a multiple of 16
    assert probe(P, 16, P, -1, N) == SHAPE
    assert probe(N, 16, P, 1, N) == NULLP
    assert probe(P, 16, N, 1, N) == NULLP
    assert probe(ctypes.c_void_p((1 << 20) + 8), 16, P, 1, N) == UNSUP
    assert probe(P, (256 << 10) + 16, P, 1, N) == WS  # two spans, one sink word


def test_fp8_validation(lib):
    w8 = lambda n=4, dt=BF16, ks=0.1, vs=0.1, key=P, kc=P, d=64: lib.pa_reshape_and_cache_fp8(
        key, P, kc, P, P, n, 2, d, 16, 8, dt, ks, vs, N)
    assert w8(ks=0.0) == SHAPE
    assert w8(vs=-1.0) == SHAPE
    assert w8(ks=float("inf")) == SHAPE
    assert w8(ks=float("nan")) == SHAPE
    assert w8(dt=7) == UNSUP
    assert w8(d=80) == UNSUP
    assert w8(key=N) == NULLP
    assert w8(kc=ctypes.c_void_p((1 << 20) + 8)) == UNSUP
    assert w8(n=0, key=N, kc=N) == OK
    dec8 = lambda fn="pa_decode_fp8", dt=F16, ks=0.1, vs=0.1, ws=P, s=4: getattr(lib, fn)(
        P, P, P, P, P, 100, P, s, 8, 2, 128, 16, 64, 1000, 0.1, 0.0, 0, 512, ks, vs, ws, 1 << 30, dt, N)
    for fn in ("pa_decode_fp8", "pa_decode_partitions_fp8"):
        assert dec8(fn, dt=F32) == UNSUP  # fp8 caches need a 16-bit query
        assert dec8(fn, ks=0.0) == SHAPE
        assert dec8(fn, vs=float("nan")) == SHAPE
        assert dec8(fn, ws=N) == NULLP
        assert dec8(fn, s=0) == OK
    pre8 = lambda ks=0.1, dt=BF16: lib.pa_prefill_chunk_fp8(
        P, P, P, 64, 32, P, P, P, 8, P, 2, 8, 1, 256, 16, 64, 100, 0.1, 0.0, 0, ks, 0.1, P,
        1 << 30, dt, N)
    assert pre8(ks=-0.1) == SHAPE
    assert pre8(dt=F32) == UNSUP


def test_fused_prefill_validation(lib):
    f = lambda key=P, value=P, slots=P, nq=64, dt=BF16: lib.pa_prefill_chunk_fused(
        P, P, key, value, slots, P, nq, 32, P, P, P, 8, P, 2, 8, 1, 256, 16, 64, 100, 0.1, 0.0, 0,
        P, 1 << 30, dt, N)
    assert f(key=N) == NULLP
    assert f(slots=N) == NULLP
    assert f(value=ctypes.c_void_p((1 << 20) + 8)) == UNSUP
    assert f(slots=ctypes.c_void_p((1 << 20) + 4)) == UNSUP
    assert f(dt=F32) == UNSUP
    assert f(nq=0, key=N, value=N, slots=N) == OK


def decode(lib, fn="pa_decode", out=P, q=P, kc=P, vc=P, bt=P, mbps=100, cl=P, s=4, hq=8, hkv=2,
           d=128, bs=16, nb=64, maxc=1000, scale=0.1, cap=0.0, win=0, part=512, ws=P,
           wsb=1 << 30, dt=F16):
    return getattr(lib, fn)(out, q, kc, vc, bt, mbps, cl, s, hq, hkv, d, bs, nb, maxc, scale, cap,
                            win, part, ws, wsb, dt, N)


@pytest.mark.parametrize("fn", ["pa_decode", "pa_decode_partitions"])
def test_decode_validation(lib, fn):
    assert decode(lib, fn, hkv=3) == SHAPE           # 8 % 3 != 0
    assert decode(lib, fn, s=-1) == SHAPE
    assert decode(lib, fn, maxc=-5) == SHAPE
    assert decode(lib, fn, d=80) == UNSUP
    assert decode(lib, fn, bs=24) == UNSUP
    assert decode(lib, fn, dt=3) == UNSUP
    assert decode(lib, fn, part=100) == SHAPE        # not a multiple of 64
    assert decode(lib, fn, part=64, bs=128) == SHAPE  # not a multiple of block_size
    assert decode(lib, fn, mbps=0) == SHAPE
    assert decode(lib, fn, cap=-1.0) == SHAPE
    assert decode(lib, fn, cap=float("nan")) == SHAPE
    assert decode(lib, fn, cap=float("inf")) == SHAPE
    assert decode(lib, fn, win=-1) == SHAPE
    assert decode(lib, fn, cap=30.0, win=64, ws=N) == NULLP  # valid variant, then the workspace check
    assert decode(lib, fn, nb=0) == SHAPE
    assert decode(lib, fn, out=N) == NULLP
    assert decode(lib, fn, cl=N) == NULLP
    assert decode(lib, fn, q=ctypes.c_void_p((1 << 20) + 4)) == UNSUP
    assert decode(lib, fn, ws=N) == NULLP            # 2 partitions need a workspace
    need = lib.pa_decode_workspace_bytes(4, 8, 128, 1000, 512)
    assert need > 0
    assert decode(lib, fn, wsb=need - 1) == WS
    assert decode(lib, fn, s=0, out=N, q=N, kc=N, vc=N, bt=N, cl=N) == OK


def test_decode_fused_write_validation(lib):
    """The write's checks, then pa_decode's (no GPU call on any of these)."""
    f = lambda key=P, value=P, slots=P, nt=4, s=4, kc=P, out=P, ws=P, dt=F16: \
        lib.pa_decode_fused_write(out, P, key, value, slots, nt, kc, P, P, 100, P, s, 8, 2, 128, 16,
                                  64, 1000, 0.1, 0.0, 0, 512, ws, 1 << 30, dt, N)
    assert f(nt=-1) == SHAPE
    assert f(key=N) == NULLP
    assert f(slots=N) == NULLP
    assert f(kc=N) == NULLP
    assert f(value=ctypes.c_void_p((1 << 20) + 8)) == UNSUP
    assert f(slots=ctypes.c_void_p((1 << 20) + 4)) == UNSUP
    assert f(dt=3) == UNSUP
    assert f(out=N) == NULLP        # the decode's own checks
    assert f(ws=N) == NULLP         # 2 partitions need a workspace
    assert f(nt=0, key=N, value=N, slots=N, s=0, out=N) == OK  # nothing to do


def decode_noalloc(lib, out=P, q=P, kc=P, vc=P, bt=P, mbps=100, cl=P, s=4, hq=8, hkv=2, d=128,
                   bs=16, nb=64, maxc=1000, scale=0.1, cap=0.0, win=0, part=512, dt=F16):
    return lib.pa_decode_noalloc(out, q, kc, vc, bt, mbps, cl, s, hq, hkv, d, bs, nb, maxc, scale,
                                 cap, win, part, dt, N)


def test_decode_noalloc_validation(lib):
    """Every argument check of pa_decode, then the fixed scratch's limit, all
    before the library touches a device."""
    TOO_LARGE = 6
    assert decode_noalloc(lib, hkv=3) == SHAPE
    assert decode_noalloc(lib, d=80) == UNSUP
    assert decode_noalloc(lib, part=100) == SHAPE
    assert decode_noalloc(lib, win=-1) == SHAPE
    assert decode_noalloc(lib, out=N) == NULLP
    assert decode_noalloc(lib, cl=N) == NULLP
    assert decode_noalloc(lib, q=ctypes.c_void_p((1 << 20) + 4)) == UNSUP
    assert decode_noalloc(lib, s=0, out=N, q=N, kc=N, vc=N, bt=N, cl=N) == OK
    # 4096 sequences x 64 heads x 16 partitions of (256 + 2) floats: far past 64 MiB
    big = dict(s=4096, hq=64, hkv=8, d=256, mbps=512, maxc=8192)
    assert lib.pa_decode_workspace_bytes(4096, 64, 256, 8192, 512) > 64 << 20
    assert decode_noalloc(lib, **big) == TOO_LARGE
    assert decode_noalloc(lib, out=N, **big) == NULLP  # pointer checks come first
    # The limit counts the context the tables can reach, not max_context_len
    # alone: with 32-block tables the call fits, passes validation and then
    # fails at the scratch lookup, since this machine has no device.
    assert lib.pa_decode_workspace_bytes(4096, 64, 256, 512, 512) <= 64 << 20
    assert decode_noalloc(lib, **dict(big, mbps=32)) == LAUNCH


def test_reduce_validation(lib):
    r = lib.pa_decode_reduce
    # mbps 100 x block 16 >= 1000 tokens: two partitions, so a workspace is needed.
    assert r(P, P, 4, 8, 128, 100, 16, 1000, 0, 512, N, 0, F16, N) == NULLP
    assert r(P, P, 4, 8, 128, 100, 16, 1000, 0, 512, P, 10, F16, N) == WS
    assert r(P, P, 4, 8, 96, 100, 16, 1000, 0, 512, P, 1 << 30, F16, N) == UNSUP
    assert r(N, P, 4, 8, 128, 100, 16, 1000, 0, 512, P, 1 << 30, F16, N) == NULLP
    assert r(P, P, 4, 8, 128, 100, 16, 1000, 0, 100, P, 1 << 30, F16, N) == SHAPE
    assert r(P, P, 4, 8, 128, 100, 16, 1000, -1, 512, P, 1 << 30, F16, N) == SHAPE


def test_workspace_sizes(lib):
    f = lib.pa_decode_workspace_bytes
    a256 = lambda x: (x + 255) // 256 * 256
    # One partition: only the work plan (a 256-byte header, then 16 bytes per item).
    assert f(128, 32, 128, 4096, 0) == 256 + a256(128 * 16)       # never split
    assert f(128, 32, 128, 512, 512) == 256 + a256(128 * 16)      # always one partition
    # Eight partitions: max and sum per (seq, head, partition), D floats of
    # partial output, then the plan with one item per (seq, partition), the
    # shared-partition count per sequence and a group member per (seq, partition).
    n = 128 * 32 * 8
    expect = (2 * a256(n * 4) + a256(n * 128 * 4) + 256 + a256(128 * 8 * 16) + a256(128 * 4)
              + a256(128 * 8 * 4))
    assert f(128, 32, 128, 4096, 512) == expect
    assert f(0, 32, 128, 4096, 512) == 0
    g = lib.pa_prefill_workspace_bytes
    # One key range: only the work plan, one 16-byte item per (chunk, 16-position tile).
    assert g(2048, 4, 8, 1, 256, 512, 1024) == 256 + a256(4 * 32 * 16)
    # Four key ranges: max, sum and D partial floats per (token, head, range), the plan,
    # then each query token's chunk.
    n = 2048 * 8 * 4
    assert g(2048, 4, 8, 1, 256, 512, 4096) == (2 * a256(n * 4) + a256(n * 256 * 4) + 256
                                                + a256(4 * 32 * 4 * 16) + a256(2048 * 4))
    assert g(2048, 4, 8, 3, 256, 512, 4096) == 0  # heads not a multiple of KV heads


def prefill(lib, out=P, q=P, qsl=P, nq=64, maxq=32, kc=P, vc=P, bt=P, mbps=8, cl=P, s=2, hq=8,
            hkv=1, d=256, bs=16, nb=64, maxc=100, scale=0.1, cap=0.0, win=0, ws=P, wsb=1 << 30,
            dt=BF16):
    return lib.pa_prefill_chunk(out, q, qsl, nq, maxq, kc, vc, bt, mbps, cl, s, hq, hkv, d, bs, nb,
                                maxc, scale, cap, win, ws, wsb, dt, N)


def test_prefill_validation(lib):
    assert prefill(lib, dt=F32) == UNSUP
    assert prefill(lib, cap=-0.5) == SHAPE
    assert prefill(lib, win=-3) == SHAPE
    assert prefill(lib, hq=256, hkv=1) == UNSUP     # group larger than a tile
    assert prefill(lib, nq=-1) == SHAPE
    assert prefill(lib, hkv=3) == SHAPE
    assert prefill(lib, d=32) == UNSUP
    assert prefill(lib, qsl=N) == NULLP
    assert prefill(lib, out=N) == NULLP
    assert prefill(lib, maxc=5000, mbps=400, ws=N) == NULLP
    assert prefill(lib, maxc=5000, mbps=400, wsb=16) == WS
    assert prefill(lib, nq=0, out=N, q=N, qsl=N) == OK
