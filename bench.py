#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

One step = one pass of the whole path over one batch: the slot-mapped cache
write of the step's new tokens, then decode (partition kernel + reduce
kernel) and, for the mixed workload, the prefill chunk.  The headline line is
the Llama-2-7B-like decode workload (128 sequences, 32/32 heads, head_dim 128,
fp16, contexts U[512, 4096], 512-token partitions); the other four workloads
are measured the same way and reported under "workloads".

Timing: HIP events on the stream the kernels run on (torch's current stream),
K timed steps after W warm-up steps, in three passes of K steps each: the
whole step between two events, in its one-call form (pa_decode_fused_write:
the step's cache write done in the decode's plan launch; then the prefill
chunks of a mixed step) -- the step time and the headline; the step as
separate calls with one more event where the decode begins (the decode
call's time, plan + partitions + reduce, as one span); and the separate
calls with one event after every phase (the per-phase breakdown: write,
prefill, partitions, reduce).  An event
recorded between two launches adds to the time around it, so no figure
spans an event it does not end on.  Per figure: the mean, and the median,
p10 and p90 over the steps.  Between steps, and outside the events, a 512 MiB
fill evicts the L2s and the 256 MB last-level cache so that every step reads
its K/V from HBM, and a ~300 us GPU spin lets the host queue the step's calls
before the GPU reaches them.

Figures:
  value          algorithmic bytes of one step / step time (GB/s); algorithmic
                 bytes count every attended K/V token of each physical block
                 once, plus Q, output, block-table entries, context lengths and
                 the cache write (new K/V read + written, slots);
  roofline       the decode partition kernel alone: its algorithmic bytes / its
                 average event-timed duration, against 8 TB/s;
  cpu_baseline   the fp64 oracle (tests' reference implementation, untuned) on a
                 bounded sample of the same workload, over up to 8 host processes;
  stream_probe   a bare streaming read (the library's probe kernel) and a torch
                 copy on the same box, against the spec, and the partition
                 kernel's rate against the read probe.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
       python bench.py --profile-kernel NAME    (a few launches, for rocprofv3;
                                                 NAME_fp8: the decode over E4M3 copies
                                                 of the pools, as fp8_kv_cache runs it)
       python bench.py --copy-probe              (1 GiB device copy, counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix, published
HEADLINE = "llama2_7b"
METRIC = "paged-attn decode achieved HBM GB/s (% of MI355X peak) + attended tokens/s"
FLUSH_BYTES = 512 << 20
DTYPE_NAME = {"fp32": "f32", "fp16": "f16", "bf16": "bf16"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic work of one step (host arithmetic on the workload's tables).
# ---------------------------------------------------------------------------
def _attended_slots(w, rows):
    bs = w.block_size
    parts = []
    for s in rows:
        C = int(w.context_lens[s])
        t = np.arange(C, dtype=np.int64)
        parts.append(w.block_tables[s, t // bs].astype(np.int64) * bs + t % bs)
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def work(w):
    """Bytes and flops of one step, split by kernel."""
    eb = w.elem_bytes
    row_kv = w.num_kv_heads * w.head_dim * eb * 2  # K + V of one token, all KV heads
    qrow = w.num_heads * w.head_dim * eb
    bs = w.block_size
    out = {}
    dec = w.decode_rows
    ctx = w.context_lens.astype(np.int64)
    if len(dec):
        uniq = len(np.unique(_attended_slots(w, dec)))
        logical = int(ctx[dec].sum())
        tbl = int(((ctx[dec] + bs - 1) // bs).sum()) * 4 + len(dec) * 4
        single = int((ctx[dec] <= w.partition_size).sum())
        out["decode_kv_bytes"] = uniq * row_kv
        out["decode_logical_kv_bytes"] = logical * row_kv
        out["decode_bytes"] = uniq * row_kv + 2 * len(dec) * qrow + tbl
        out["partition_kernel_bytes"] = uniq * row_kv + len(dec) * qrow + tbl + single * qrow
        out["decode_attended_tokens"] = logical
    if len(w.prefill_rows):
        pre = w.prefill_rows
        uniq = len(np.unique(_attended_slots(w, pre)))
        nq = int(w.query_start_loc[-1])
        pairs = 0
        for i, r in enumerate(pre):
            L = int(w.query_start_loc[i + 1] - w.query_start_loc[i])
            C = int(ctx[r])
            pairs += L * (C - L) + L * (L + 1) // 2
        out["prefill_bytes"] = uniq * row_kv + 2 * nq * qrow
        out["prefill_flops"] = pairs * w.num_heads * 4 * w.head_dim
        out["prefill_attended_pairs"] = pairs
    n_new = len(w.slot_mapping)
    out["write_bytes"] = 2 * n_new * row_kv + 8 * n_new
    out["step_bytes"] = out.get("decode_bytes", 0) + out.get("prefill_bytes", 0) + out["write_bytes"]
    return out


# ---------------------------------------------------------------------------
# Device state of one workload and its step.
# ---------------------------------------------------------------------------
class Step:
    def __init__(self, w, dev):
        import paged_kv_cache_179_amd as pa

        self.pa = pa
        self.w = w
        self.dev = dev
        self.kc0 = w.key_cache.to(dev)
        self.vc0 = w.value_cache.to(dev)
        self.kc = self.kc0  # the step writes into the pool in place (same slots every step)
        self.vc = self.vc0
        self.nk = w.new_key.to(dev)
        self.nv = w.new_value.to(dev)
        self.slots = torch.from_numpy(w.slot_mapping).to(dev)
        bt = torch.from_numpy(w.block_tables)
        cl = torch.from_numpy(w.context_lens)
        dr = torch.from_numpy(w.decode_rows)
        pr = torch.from_numpy(w.prefill_rows)
        self.bt_d = bt[dr].contiguous().to(dev)
        self.cl_d = cl[dr].contiguous().to(dev)
        self.bt_p = bt[pr].contiguous().to(dev)
        self.cl_p = cl[pr].contiguous().to(dev)
        self.q_d = w.query_decode.to(dev)
        self.q_p = w.query_prefill.to(dev)
        self.qsl = torch.from_numpy(w.query_start_loc).to(dev)
        self.out_d = torch.empty_like(self.q_d)
        self.out_p = torch.empty_like(self.q_p)
        self.has_dec = len(w.decode_rows) > 0
        self.has_pre = len(w.prefill_rows) > 0
        self.maxc_d = int(w.context_lens[w.decode_rows].max()) if self.has_dec else 0
        self.maxc_p = int(w.context_lens[w.prefill_rows].max()) if self.has_pre else 0
        self.maxq = int(np.diff(w.query_start_loc).max()) if self.has_pre else 0
        nb = pa.decode_workspace_bytes(len(w.decode_rows), w.num_heads, w.head_dim,
                                       self.maxc_d, w.partition_size) if self.has_dec else 0
        self.ws_d = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        nbp = pa.prefill_workspace_bytes(int(w.query_start_loc[-1]), len(w.prefill_rows),
                                         w.num_heads, w.num_kv_heads, w.head_dim, self.maxq,
                                         self.maxc_p) if self.has_pre else 0
        self.ws_p = torch.empty(max(nbp, 256), dtype=torch.uint8, device=dev)

    def write(self):
        self.pa.reshape_and_cache(self.nk, self.nv, self.kc, self.vc, self.slots)

    def one_call_step(self):
        """The step in the fewest launches: every new token's cache write done
        in the decode call's plan launch (pa_decode_fused_write), then, for a
        mixed step, the prefill chunks."""
        w = self.w
        if self.has_dec:
            self.pa.decode_fused_write(self.out_d, self.q_d, self.nk, self.nv, self.slots, self.kc,
                                       self.vc, self.bt_d, self.cl_d, w.scale, self.maxc_d,
                                       partition_size=w.partition_size, workspace=self.ws_d)
        else:
            self.write()
        if self.has_pre:
            self.prefill()

    def partitions(self):
        self.pa.decode_partitions(self.out_d, self.q_d, self.kc, self.vc, self.bt_d, self.cl_d,
                                  self.w.scale, self.maxc_d, partition_size=self.w.partition_size,
                                  workspace=self.ws_d)

    def reduce(self):
        w = self.w
        self.pa.decode_reduce(self.out_d, self.cl_d, w.num_heads, w.head_dim,
                              w.max_blocks_per_seq, w.block_size, self.maxc_d, w.partition_size,
                              self.ws_d)

    def prefill(self):
        self.pa.prefill_chunk(self.out_p, self.q_p, self.qsl, self.kc, self.vc, self.bt_p,
                              self.cl_p, self.w.scale, self.maxq, self.maxc_p, workspace=self.ws_p)

    def phases(self):
        ph = [("write", self.write)]
        if self.has_pre:
            ph.append(("prefill", self.prefill))
        if self.has_dec:
            ph += [("partitions", self.partitions), ("reduce", self.reduce)]
        return ph


def decode_plan_counts(st):
    """The decode work plan's counts in the step's workspace after a call
    (the layout pa_decode_workspace_bytes documents): items, log2 of the
    partitions an item joins, units taken from the queue, items of shared
    partitions."""
    w = st.w
    P = max(1, -(-min(st.maxc_d, w.max_blocks_per_seq * w.block_size) // w.partition_size))
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n = len(w.decode_rows) * w.num_heads * P
    off = 2 * al(n * 4) + al(n * w.head_dim * 4) if P > 1 else 0
    return [int(x) for x in st.ws_d[off:off + 16].cpu().view(torch.int32).tolist()]


_LEAD_CYCLES = None


def evict(flush_buf):
    """Before a timed region, outside its events: the 512 MiB fill that evicts
    the L2s and the last-level cache, then a ~300 us GPU spin, so that the
    host has queued the region's calls before the GPU reaches it (without
    it, small steps whose few-microsecond kernels outrun the Python calls
    that launch them showed the host's pauses: TinyLlama-shaped decode median
    24.8 us, p90 62.5 us)."""
    global _LEAD_CYCLES
    if _LEAD_CYCLES is None:  # clock ticks per 300 us, measured once
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _LEAD_CYCLES = max(1000, int(1_000_000 * 0.3 / max(e0.elapsed_time(e1), 1e-3)))
    flush_buf.zero_()
    torch.cuda._sleep(_LEAD_CYCLES)


def measure(step, steps, warmup, flush_buf):
    """Event-timed steps over `steps` steps (after `warmup`), in three passes:
    the one-call step between two events ("step"), the step as separate calls
    with an event where the decode begins ("decode": plan + partitions +
    reduce as one span; "step_separate": the whole of it), and one event
    after every phase (the phases by name).  Returns ms lists."""
    phases = step.phases()
    for _ in range(warmup):
        flush_buf.zero_()
        for _, fn in phases:
            fn()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    res = {name: [] for name, _ in phases}
    res["step"] = []
    # 1. The whole step, in its one-call form (the write in the decode's plan launch).
    for _ in range(warmup):
        flush_buf.zero_()
        step.one_call_step()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        evict(flush_buf)
        e = [ev(), ev()]
        e[0].record()
        step.one_call_step()
        e[1].record()
        evs.append(e)
    torch.cuda.synchronize()
    res["_wall_s"] = time.perf_counter() - t0
    res["step"] = [e[0].elapsed_time(e[1]) for e in evs]
    # 2. The decode call as one span (the phases before it, then one event).
    if step.has_dec:
        first_dec = [name for name, _ in phases].index("partitions")
        evs = []
        for _ in range(steps):
            evict(flush_buf)
            e = [ev(), ev(), ev()]
            e[0].record()
            for i, (_, fn) in enumerate(phases):
                if i == first_dec:
                    e[1].record()
                fn()
            e[2].record()
            evs.append(e)
        torch.cuda.synchronize()
        res["decode"] = [e[1].elapsed_time(e[2]) for e in evs]
        res["step_separate"] = [e[0].elapsed_time(e[2]) for e in evs]
    # 3. Every phase.
    evs = []
    for _ in range(steps):
        evict(flush_buf)
        e = [ev() for _ in range(len(phases) + 1)]
        e[0].record()
        for i, (_, fn) in enumerate(phases):
            fn()
            e[i + 1].record()
        evs.append(e)
    torch.cuda.synchronize()
    for e in evs:
        for i, (name, _) in enumerate(phases):
            res[name].append(e[i].elapsed_time(e[i + 1]))
    return res


def summarize(name, w, wk, t, steps):
    mean = {k: float(np.mean(v)) for k, v in t.items() if not k.startswith("_")}
    r = {"workload": name, "dtype": DTYPE_NAME[w.dtype], "num_seqs": w.num_seqs,
         "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
         "block_size": w.block_size, "partition_size": w.partition_size,
         "ms": {k: round(v, 5) for k, v in mean.items()},
         "ms_median": {k: round(float(np.median(v)), 5) for k, v in t.items() if not k.startswith("_")},
         "ms_p10": {k: round(float(np.percentile(v, 10)), 5) for k, v in t.items() if not k.startswith("_")},
         "ms_p90": {k: round(float(np.percentile(v, 90)), 5) for k, v in t.items() if not k.startswith("_")},
         "step_bytes": wk["step_bytes"],
         "step_gbs": wk["step_bytes"] / (mean["step"] * 1e-3) / 1e9}
    if "partitions" in mean:
        dec_ms = mean["decode"]
        r["decode_ms"] = dec_ms
        r["decode_gbs"] = wk["decode_bytes"] / (dec_ms * 1e-3) / 1e9
        r["decode_hbm_frac"] = r["decode_gbs"] / HBM_PEAK_GBS
        r["decode_effective_gbs"] = (wk["decode_logical_kv_bytes"] + wk["decode_bytes"]
                                     - wk["decode_kv_bytes"]) / (dec_ms * 1e-3) / 1e9
        r["decode_attended_tokens_per_s"] = wk["decode_attended_tokens"] / (dec_ms * 1e-3)
        r["partition_kernel_gbs"] = wk["partition_kernel_bytes"] / (mean["partitions"] * 1e-3) / 1e9
        r["decode_bytes"] = wk["decode_bytes"]
    if "prefill" in mean:
        r["prefill_tflops"] = wk["prefill_flops"] / (mean["prefill"] * 1e-3) / 1e12
        r["prefill_mfma_frac"] = r["prefill_tflops"] / MFMA_BF16_PEAK_TFLOPS
        r["prefill_flops"] = wk["prefill_flops"]
    r["write_gbs"] = wk["write_bytes"] / (mean["write"] * 1e-3) / 1e9
    return r


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample, over the host's cores.
# ---------------------------------------------------------------------------
CPU_WORKERS_MAX = 8  # worker processes (each one thread); the rest of the box's share stays free


def _widen(raw, dtype_name):
    """float64 copy of raw cache bits (exact for every storage type)."""
    if dtype_name == "bf16":
        return (raw.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype_name == "fp16":
        return raw.view(np.float16).astype(np.float64)
    return raw.view(np.float32).astype(np.float64)


def _cpu_worker(job):
    """One host process of the CPU baseline: the oracle, one thread, over its
    share of the sampled sequences (each sequence's blocks widened to float64
    inside the timed region, as one oracle call would).  Returns seconds."""
    kpath, vpath, dtype_name, items, scale, bs = job
    from threadpoolctl import threadpool_limits

    import oracle

    K = np.load(kpath, mmap_mode="r")
    V = np.load(vpath, mmap_mode="r")
    used = 0.0
    with threadpool_limits(limits=1):
        for q, b0, nblk, C in items:
            t0 = time.perf_counter()
            oracle.paged_decode(q, _widen(np.asarray(K[b0:b0 + nblk]), dtype_name),
                                _widen(np.asarray(V[b0:b0 + nblk]), dtype_name),
                                np.arange(nblk)[None], [C], scale, bs)
            used += time.perf_counter() - t0
    return used


def cpu_baseline(w, max_kv_bytes=6 << 30):
    """The oracle as it stands (fp64 numpy) on the host: the decode rows of
    the workload in order, up to max_kv_bytes of attended K/V, spread over
    worker processes (one thread each) by size; value = sampled bytes / the
    slowest worker's compute time."""
    import concurrent.futures as cf
    import multiprocessing as mp

    import oracle

    raw = {torch.float16: torch.int16, torch.bfloat16: torch.int16, torch.float32: torch.int32}[
        w.key_cache.dtype]
    # Caches after the step's write, as the oracle computes it (raw bits).
    kc, vc = oracle.reshape_and_cache(w.new_key.view(raw).numpy(), w.new_value.view(raw).numpy(),
                                      w.key_cache.view(raw).numpy(), w.value_cache.view(raw).numpy(),
                                      w.slot_mapping, w.block_size)
    eb = w.elem_bytes
    row_kv = w.num_kv_heads * w.head_dim * eb * 2
    qrow = w.num_heads * w.head_dim * eb
    rows, blocks, items, kv = [], [], [], 0
    for i, s in enumerate(w.decode_rows):
        C = int(w.context_lens[s])
        if rows and kv + C * row_kv > max_kv_bytes:
            break
        nblk = (C + w.block_size - 1) // w.block_size
        q = w.query_decode[i:i + 1].to(torch.float64).numpy()
        items.append((q, sum(len(b) for b in blocks), nblk, C))
        blocks.append(w.block_tables[s, :nblk].astype(np.int64))
        rows.append(int(s))
        kv += C * row_kv
    idx = np.concatenate(blocks)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(CPU_WORKERS_MAX, cores, len(items)))
    shares = [[] for _ in range(workers)]
    load = [0] * workers
    for it in sorted(items, key=lambda x: -x[3]):  # longest first onto the least loaded
        j = int(np.argmin(load))
        shares[j].append(it)
        load[j] += it[3]
    tag = f"/dev/shm/pa_cpu_baseline_{os.getpid()}"
    paths = (tag + "_k.npy", tag + "_v.npy")
    try:
        np.save(paths[0], kc[idx])
        np.save(paths[1], vc[idx])
        del kc, vc
        jobs = [(paths[0], paths[1], w.dtype, sh, w.scale, w.block_size) for sh in shares]
        with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
            secs = list(ex.map(_cpu_worker, jobs))
    finally:
        for pth in paths:
            if os.path.exists(pth):
                os.remove(pth)
    wall = max(secs)
    toks = int(w.context_lens[rows].astype(np.int64).sum())
    nbytes = toks * row_kv + 2 * len(rows) * qrow
    return {"value": nbytes / wall / 1e9, "unit": "GB/s", "cores": workers, "kind": "oracle",
            "attended_tokens_per_s": toks / wall, "seconds": round(wall, 3),
            "cpu_seconds": round(sum(secs), 3),
            "sample": f"oracle decode of the first {len(rows)} of {len(w.decode_rows)} sequences "
                      f"({toks} attended tokens), fp64 numpy, {workers} processes of one thread "
                      f"(longest first onto the least loaded); GB/s = sampled bytes / the slowest "
                      f"process's compute time",
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# Counter-derived traffic (committed rocprofv3 summaries).
# ---------------------------------------------------------------------------
def partition_kernel_name(w):
    """Symbol of the decode partition kernel that serves workload w."""
    if w.dtype == "fp32":
        g = min(8, w.num_heads // w.num_kv_heads)
        return f"decode_partition_kernel<F32,{w.head_dim},{g}>"
    # The last argument says whether the launch's plan searched for shared
    # partitions: not for TinyLlama, whose calls take the static plan.
    groups = "false" if w.name == "tinyllama" else "true"
    return f"decode_mfma_kernel<{w.dtype.upper().replace('FP', 'F')},{w.head_dim},ScoreMap<false,false,false>,false,{groups}>"


def kernel_source_hash():
    """Hash of the library's sources without their // comments and blank
    lines: a change to the code invalidates the committed counters, a change
    to a comment does not."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "paged_kv_cache_179_amd", "csrc"))):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(ROOT, "paged_kv_cache_179_amd", "csrc", f), encoding="utf-8") as fh:
                code = [line.split("//", 1)[0].rstrip() for line in fh]
            h.update(f.encode() + "\n".join(x for x in code if x).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload):
    """HBM bytes per partition-kernel launch from the committed counter summary,
    or None if there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_decode_partition_{workload}.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
def profile_kernel(name, launches=5):
    from paged_kv_cache_179_amd import workloads as W

    fp8 = name.endswith("_fp8")
    w = W.make(name[: -len("_fp8")] if fp8 else name)
    st = Step(w, torch.device("cuda:0"))
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    st.write()
    if fp8:  # the decode over E4M3 copies of the pools (per-tensor scale 1/64), as fp8_kv runs it
        scale = 1.0 / 64
        kc8 = (st.kc.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
        vc8 = (st.vc.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
        torch.cuda.synchronize()
        for _ in range(launches):
            flush.zero_()
            st.pa.decode(st.out_d, st.q_d, kc8, vc8, st.bt_d, st.cl_d, w.scale, st.maxc_d,
                         partition_size=w.partition_size, workspace=st.ws_d, k_scale=scale,
                         v_scale=scale)
        torch.cuda.synchronize()
        log(f"profiled {launches} fp8 decode launches of {w.name}")
        return
    for _ in range(launches):
        flush.zero_()
        if st.has_dec:
            st.partitions()
            st.reduce()
        if st.has_pre:
            st.prefill()
    torch.cuda.synchronize()
    log(f"profiled {launches} launches of {name}")


def copy_probe(nbytes=1 << 30, launches=3):
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(launches):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {nbytes} bytes x {launches}")


def stream_probe(dev, reps=5):
    """What this machine's HBM gives a bare streaming read, for context beside the
    8 TB/s spec: the library's read probe over 4 GiB (non-temporal 16-byte
    loads, eight per lane in flight), and torch's 2 GiB -> 2 GiB copy (read +
    write bytes); each the best of `reps` event-timed launches after one
    warm-up."""
    import paged_kv_cache_179_amd as pa

    x = torch.empty(1 << 30, dtype=torch.int32, device=dev).fill_(1)
    sink = torch.empty((x.numel() * 4 + (256 << 10) - 1) // (256 << 10), dtype=torch.int32, device=dev)
    a = torch.empty(1 << 31, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)

    def best(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    t_read = best(lambda: pa.stream_read_probe(x, sink))
    t_copy = best(lambda: b.copy_(a))
    out = {"read_gbs": x.numel() * 4 / t_read / 1e9, "copy_gbs": 2 * a.numel() / t_copy / 1e9}
    out["read_frac_of_spec"] = out["read_gbs"] / HBM_PEAK_GBS
    out["copy_frac_of_spec"] = out["copy_gbs"] / HBM_PEAK_GBS
    del x, sink, a, b
    torch.cuda.empty_cache()
    return out


def block_ops(dev, reps=10):
    """Block-pool copies on Llama-2-7B-like blocks (32 KV heads x 16 tokens x
    128 dims, fp16: 128 KiB per block and pool): copy-on-write of 1024 blocks
    inside a 4096-block pool (K and V), and a swap of 256 blocks to a pinned
    host pool and back.  Bytes count each copied byte once read and once
    written."""
    import paged_kv_cache_179_amd as pa

    g = torch.Generator(device="cpu").manual_seed(7)
    nb, hkv, bs, d = 4096, 32, 16, 128
    kc = torch.randn((nb, hkv, bs, d), generator=g, dtype=torch.float32).to(torch.float16).to(dev)
    vc = torch.randn((nb, hkv, bs, d), generator=g, dtype=torch.float32).to(torch.float16).to(dev)
    ids = torch.randperm(nb, generator=g)
    pairs = torch.stack([ids[:1024], ids[1024:2048]], dim=1).to(torch.int64).to(dev)
    block = hkv * bs * d * 2
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def timed(fn):
        ts = []
        for i in range(reps + 2):
            evict(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1))
        return float(np.mean(ts))

    ms_copy = timed(lambda: pa.copy_blocks(kc, vc, pairs))
    host = torch.empty((512, hkv, bs, d), dtype=torch.float16).pin_memory()
    out_pairs = torch.stack([ids[:256], torch.arange(256)], dim=1).to(torch.int64).to(dev)
    in_pairs = torch.stack([torch.arange(256), ids[2048:2304]], dim=1).to(torch.int64).to(dev)
    ms_out = timed(lambda: pa.swap_blocks(kc, host, out_pairs))
    ms_in = timed(lambda: pa.swap_blocks(host, kc, in_pairs))
    copy_bytes = 2 * 2 * 1024 * block
    swap_bytes = 256 * block
    return {"copy_blocks": {"pairs": 1024, "block_bytes": block, "ms": round(ms_copy, 5),
                            "gbs": copy_bytes / (ms_copy * 1e-3) / 1e9,
                            "hbm_frac": copy_bytes / (ms_copy * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "swap_out_to_pinned_host": {"pairs": 256, "ms": round(ms_out, 5),
                                        "gbs_one_way": swap_bytes / (ms_out * 1e-3) / 1e9},
            "swap_in_from_pinned_host": {"pairs": 256, "ms": round(ms_in, 5),
                                         "gbs_one_way": swap_bytes / (ms_in * 1e-3) / 1e9}}


def variants(dev, cap=50.0, window=1024, reps=10):
    """The Gemma-2B-like mixed step with Gemma-2-style logit soft-capping (50)
    and a 1024-token sliding window, decode and prefill timed apart.  Bytes
    and flops count only what the window lets each row attend."""
    from paged_kv_cache_179_amd import workloads as W

    w = W.make("gemma_2b_mixed")
    st = Step(w, dev)
    st.write()
    eb = w.elem_bytes
    row_kv = w.num_kv_heads * w.head_dim * eb * 2
    qrow = w.num_heads * w.head_dim * eb
    ctx = w.context_lens.astype(np.int64)
    dec_tokens = int(np.minimum(ctx[w.decode_rows], window).sum())
    dec_bytes = dec_tokens * row_kv + 2 * len(w.decode_rows) * qrow
    pairs = 0
    for i, r in enumerate(w.prefill_rows):
        L = int(w.query_start_loc[i + 1] - w.query_start_loc[i])
        pos = int(ctx[r]) - L + np.arange(L)
        pairs += int(np.minimum(pos + 1, window).sum())
    flops = pairs * w.num_heads * 4 * w.head_dim
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def dec():
        st.pa.decode(st.out_d, st.q_d, st.kc, st.vc, st.bt_d, st.cl_d, w.scale, st.maxc_d,
                     partition_size=w.partition_size, workspace=st.ws_d, logit_softcap=cap,
                     sliding_window=window)

    def pre():
        st.pa.prefill_chunk(st.out_p, st.q_p, st.qsl, st.kc, st.vc, st.bt_p, st.cl_p, w.scale,
                            st.maxq, st.maxc_p, workspace=st.ws_p, logit_softcap=cap,
                            sliding_window=window)

    def timed(fn):
        ts = []
        for i in range(reps + 2):
            evict(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1))
        return float(np.mean(ts))

    ms_d, ms_p = timed(dec), timed(pre)
    return {"workload": "gemma_2b_mixed", "logit_softcap": cap, "sliding_window": window,
            "decode_ms": round(ms_d, 5), "decode_gbs": dec_bytes / (ms_d * 1e-3) / 1e9,
            "decode_hbm_frac": dec_bytes / (ms_d * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "prefill_ms": round(ms_p, 5), "prefill_tflops": flops / (ms_p * 1e-3) / 1e12,
            "prefill_mfma_frac": flops / (ms_p * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def unified_step(dev, reps=10):
    """The Gemma-2B-like mixed step as one fused call (pa_prefill_chunk_fused
    over the 4 chunks and the 124 decode rows as one-token chunks, with all
    2,172 new tokens' cache writes), beside the separate path (write, prefill,
    decode partitions and reduce) on the same data."""
    from paged_kv_cache_179_amd import workloads as W

    w = W.make("gemma_2b_mixed")
    st = Step(w, dev)
    st.write()
    rows = np.concatenate([w.prefill_rows, w.decode_rows])
    lens = np.concatenate([np.diff(w.query_start_loc), np.ones(len(w.decode_rows), dtype=np.int64)])
    qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    q = torch.cat([st.q_p, st.q_d]).contiguous()
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.block_tables[rows]).to(dev)
    cl = torch.from_numpy(w.context_lens[rows]).to(dev)
    maxq, maxc = int(lens.max()), int(w.context_lens[rows].max())
    ws = torch.empty(max(256, st.pa.prefill_workspace_bytes(int(lens.sum()), len(rows), w.num_heads,
                                                            w.num_kv_heads, w.head_dim, maxq, maxc)),
                     dtype=torch.uint8, device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def fused():
        st.pa.prefill_chunk_fused(out, q, st.nk, st.nv, st.slots, qsl, st.kc, st.vc, bt, cl,
                                  w.scale, maxq, maxc, workspace=ws)

    def separate():
        for _, fn in st.phases():
            fn()

    ts = {}
    for label, fn in (("fused", fused), ("separate", separate)):
        v = []
        for i in range(reps + 2):
            evict(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                v.append(e0.elapsed_time(e1))
        ts[label] = float(np.mean(v))
    step_bytes = work(w)["step_bytes"]
    return {"workload": "gemma_2b_mixed", "fused_call_ms": round(ts["fused"], 5),
            "separate_ms": round(ts["separate"], 5), "fused_step_gbs": step_bytes / (ts["fused"] * 1e-3) / 1e9,
            "launches_fused": 3, "launches_separate": 7}


def fp8_kv(dev, names=("llama2_7b", "qwen25_7b", "gemma_2b_mixed"), reps=10):
    """Decode (and, for the mixed workload, the prefill chunks) over E4M3 (fp8)
    copies of the workloads' caches: the same step with half the cache bytes.
    The pools are converted once, outside the timing (per-tensor scale 1/64:
    N(0, 1) values stay inside E4M3's range).  Bytes count each unique
    attended token's fp8 K and V once, plus Q, output and table entries, as for
    the 16-bit line; prefill is counted in flops, as for the 16-bit line."""
    from paged_kv_cache_179_amd import workloads as W

    out = {}
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    scale = 1.0 / 64
    for name in names:
        w = W.make(name)
        st = Step(w, dev)
        st.write()
        kc8 = (st.kc.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
        vc8 = (st.vc.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
        wk = work(w)
        fp8_bytes = wk["decode_bytes"] - wk["decode_kv_bytes"] // 2  # K/V at one byte per element

        def dec():
            st.pa.decode(st.out_d, st.q_d, kc8, vc8, st.bt_d, st.cl_d, w.scale, st.maxc_d,
                         partition_size=w.partition_size, workspace=st.ws_d, k_scale=scale,
                         v_scale=scale)

        def dec16():
            st.pa.decode(st.out_d, st.q_d, st.kc, st.vc, st.bt_d, st.cl_d, w.scale, st.maxc_d,
                         partition_size=w.partition_size, workspace=st.ws_d)

        def pre():
            st.pa.prefill_chunk(st.out_p, st.q_p, st.qsl, kc8, vc8, st.bt_p, st.cl_p, w.scale,
                                st.maxq, st.maxc_p, workspace=st.ws_p, k_scale=scale, v_scale=scale)

        def pre16():
            st.prefill()

        fns = [("fp8", dec), ("16bit", dec16)]
        if st.has_pre:
            fns += [("pre_fp8", pre), ("pre_16bit", pre16)]
        ts = {}
        for label, fn in fns:
            v = []
            for i in range(reps + 2):
                evict(flush)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                if i >= 2:
                    v.append(e0.elapsed_time(e1))
            ts[label] = float(np.mean(v))
        out[name] = {"decode_ms": round(ts["fp8"], 5), "decode_gbs": fp8_bytes / (ts["fp8"] * 1e-3) / 1e9,
                     "decode_hbm_frac": fp8_bytes / (ts["fp8"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "decode_bytes": fp8_bytes, "decode_ms_16bit_same_run": round(ts["16bit"], 5),
                     "speedup_vs_16bit": ts["16bit"] / ts["fp8"]}
        if st.has_pre:
            tf = wk["prefill_flops"] / (ts["pre_fp8"] * 1e-3) / 1e12
            out[name].update({"prefill_ms": round(ts["pre_fp8"], 5), "prefill_tflops": tf,
                              "prefill_mfma_frac": tf / MFMA_BF16_PEAK_TFLOPS,
                              "prefill_ms_16bit_same_run": round(ts["pre_16bit"], 5)})
        del st, kc8, vc8
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default=None, help="measure one workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernel", default=None)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode shards by sequence or KV head with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import paged_kv_cache_179_amd as pa

    if not pa.library_path().exists():
        from paged_kv_cache_179_amd.build import build

        build()
    pa.library()
    if args.copy_probe:
        copy_probe()
        return
    if args.profile_kernel:
        profile_kernel(args.profile_kernel)
        return

    from paged_kv_cache_179_amd import workloads as W

    dev = torch.device("cuda:0")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    names = [args.only] if args.only else W.NAMES
    if HEADLINE not in names:
        names = names + [HEADLINE]
    results = {}
    headline = None
    for name in names:
        t0 = time.perf_counter()
        w = W.make(name)
        log(f"{name}: generated in {time.perf_counter() - t0:.1f}s")
        st = Step(w, dev)
        wk = work(w)
        t = measure(st, args.steps, args.warmup, flush)
        r = summarize(name, w, wk, t, args.steps)
        if st.has_dec:
            cnt = decode_plan_counts(st)
            r["decode_plan"] = {"items": cnt[0], "item_partitions": 1 << cnt[1],
                                "item_tokens_max": w.partition_size << cnt[1],
                                "shared_partition_items": cnt[3],
                                "units": cnt[0] * w.num_kv_heads * -(-(w.num_heads // w.num_kv_heads) // 16)}
        r["wall_ms_per_step_incl_flush"] = t["_wall_s"] / args.steps * 1e3
        results[name] = r
        log(f"{name}: " + json.dumps({k: r[k] for k in r if k.endswith(("gbs", "frac", "_ms", "tflops"))}))
        if name == HEADLINE:
            headline = (w, wk, t, r)
            if not args.no_cpu_baseline:
                log("cpu baseline ...")
                results["_cpu"] = cpu_baseline(w)
        del st
        torch.cuda.empty_cache()

    extras, variant, fp8, unified, probe = {}, None, None, None, None
    if not args.only:
        extras = block_ops(dev)
        log("block ops: " + json.dumps(extras))
        variant = variants(dev)
        log("variants: " + json.dumps(variant))
        fp8 = fp8_kv(dev)
        log("fp8 kv: " + json.dumps(fp8))
        unified = unified_step(dev)
        log("unified step: " + json.dumps(unified))
        probe = stream_probe(dev)
        log("stream probe: " + json.dumps(probe))
    w, wk, t, r = headline
    part_ms = float(np.mean(t["partitions"]))
    achieved = wk["partition_kernel_bytes"] / (part_ms * 1e-3) / 1e9
    if probe:
        probe["headline_partition_kernel_frac_of_read_probe"] = achieved / probe["read_gbs"]
    traffic = counter_traffic(HEADLINE)
    line = {
        "metric": METRIC,
        "value": round(r["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"]["step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[w.dtype],
        "data": "synthetic",
        "config": {"workload": "llama2_7b_decode_step", "num_seqs": w.num_seqs,
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size,
                   "context_lens": "uniform[512,4096]", "partition_size": w.partition_size,
                   "reduce_kernel": True, "step_calls": "pa_decode_fused_write (cache write in the plan launch)",
                   "decode_item_partitions": r.get("decode_plan", {}).get("item_partitions"),
                   "num_blocks": w.num_blocks},
        "hbm_frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4),
        "attended_tokens_per_s": round(r["decode_attended_tokens_per_s"], 1),
        "roofline": {"kernel": partition_kernel_name(w), "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(part_ms, 5),
                     "algorithmic_bytes_per_launch": wk["partition_kernel_bytes"]},
        "cpu_baseline": results.get("_cpu"),
        "workloads": {k: v for k, v in results.items() if not k.startswith("_")},
        "block_ops": extras or None,
        "variants": variant,
        "fp8_kv_cache": fp8,
        "fused_mixed_step": unified,
        "stream_probe": probe,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
