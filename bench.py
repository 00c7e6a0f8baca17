"""Benchmark: paged decode attention on one MI355X.

Workload (seeded synthetic, no dataset): the GQA decode batch — 64
sequences with context lengths U[512, 4096], 32 query heads over 8 KV heads
(group 4), head_dim 128, 16-token blocks in the page's token-major KVBlock
layout (``--v-layout dim`` for dim-major V), bf16 K/V/q, a pool of all blocks
plus 10% spare with shuffled physical ids. ``--layers`` attention layers
(default 4) each hold their own K/V pool and share one block table, as the
layers of a model do; four layers keep the working set (~2.4 GB) far above
the 256 MB Infinity Cache, so every timed decode reads K/V from HBM.

One step = one decode step of the whole path: the host block manager
allocates one slot per sequence (pa_alloc_batch; copy-on-write pairs, none
here), packs the tables, one pinned host-to-device copy carries slots /
pairs / tables / lengths (on a copy stream, overlapping the previous step's
kernels), then per layer pa_copy_blocks (if pairs) -> pa_decode_append: the
new token's K/V written into its slot and the balanced-split attention over
the sequence including it, in one launch (one persistent kernel over the
resident workgroups, then the log-sum-exp merge of sequences cut between
them). ``--separate-write`` runs pa_reshape_and_cache then pa_decode
instead. Inputs are resident in HBM before timing starts.

Printed: one JSON line. ``value`` = KV bytes the decode calls of the timed
steps must read (2 * L * Hkv * D * 2 per sequence and layer, valid tokens
only) / wall time of those steps. ``roofline`` = the same bytes per pa_decode
call / its mean duration from HIP events recorded around the first layer's
pa_decode call of every timed step, on the stream it runs on. The events
are created with hipEventDisableSystemFence (see HipTimingEvent): default
events add a cache write-back and invalidate, ~5 us of idle queue each.
``cpu_baseline`` = the fp64 oracle on the host cores.

``--workload gqa-calls|long|mixed|prefix`` times decode calls instead (the
GQA batch through plain pa_decode, the long-context batch, the mixed-length
batch with ``--kv`` and ``--block-size``, the prefix-sharing batch, with
``--shared`` through pa_decode_shared): ``--layers`` pools whose K/V are
drawn on the device (torch's seeded generator; fp8 pools take the scale
6/448, about the amax of that many N(0,1) draws) and written through
pa_reshape_and_cache, then ``--steps`` rounds of one call per layer, back to
back, timed with HIP events (also around layer 0's call of each round, for
the median and minimum). ``value`` = KV bytes per call / mean call time (no
host work in the timed region); no cpu_baseline. ``--cold`` adds single
calls each preceded by a 1 GiB read (cold L2 and Infinity Cache; a write
instead, ``--cold-write``, leaves dirty lines whose write-back competes
with the timed call).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak) + decode tokens/s"
HBM_PEAK_GBS = 8000.0
# sources of the kernels a bf16 pa_decode call runs (balanced split and partitions)
KERNEL_SOURCES = ["decode_sk_kernel.h", "decode_vt_kernel.h", "decode_common.h", "decode_dispatch.h", "decode.hip",
                  "device_common.h", "decode_sk_bf16.hip", "decode_sk_bf16_tv.hip", "decode_vt_bf16.hip"]


def kernel_hash() -> str:
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_49_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_profile():
    """The committed profile of the GQA decode step (profiles/decode_gqa_profile.json:
    rocprofv3 kernel-trace durations of the balanced kernel (K1) and its merge
    (K2), calibrated FETCH_SIZE / WRITE_SIZE per call, and the algorithmic
    bytes per call of the profiled run), or None when the kernel sources
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "decode_gqa_profile.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_hash") == kernel_hash() else None


def algorithmic_bytes(lens, block_size: int, hq: int, hkv: int, d: int, kv_bytes: int, out_bytes: int,
                      appended: bool) -> int:
    """Bytes one decode call must move at the least: per sequence the K and V
    rows of its valid tokens, its block-table entries, its q rows and its
    output rows, plus (a call that appends) the new token's row written
    into the cache, and the lengths (and slots) arrays."""
    lens = np.asarray(lens, np.int64)
    kv = 2 * int(lens.sum()) * hkv * d * kv_bytes
    tables = 4 * int((-(-lens // block_size)).sum())
    qo = len(lens) * hq * d * (2 + out_bytes)
    new_rows = len(lens) * 2 * hkv * d * kv_bytes if appended else 0
    return kv + tables + qo + new_rows + 4 * len(lens) + (8 * len(lens) if appended else 0)


class HipTimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence. Recording
    a default event makes the queue perform a system-scope cache write-back
    and invalidate, which shows up as several microseconds of idle queue
    around the timed call and slows the work after it; this flag skips that
    (the event then only orders the timestamp, which is all a timer needs).
    The HIP runtime is the one the process already runs (looked up through
    libpagedattn's dependencies)."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self):
        import ctypes

        import paged_kv_cache_49_amd as pa
        if HipTimingEvent._hip is None:
            hip = pa.lib()
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipTimingEvent._hip = hip
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        rc = self._hip.hipEventRecord(self.h, self._ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "HipTimingEvent") -> float:
        """Milliseconds from this event to ``end`` (waits for ``end``)."""
        ms = self._ct.c_float()
        if self._hip.hipEventSynchronize(end.h) != 0 or \
                self._hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if getattr(self, "h", None) is not None and self.h.value and self._hip is not None:
            self._hip.hipEventDestroy(self.h)
            self.h = None


def step_timeline(tms, origin, t0: float, wall: float, layers: int) -> dict:
    """Per-step timeline of timed PagedBatch steps: host phase stamps
    (relative to t0, microseconds), the device span of each step on the
    compute stream (from ``origin``, recorded at t0), layer 0's call time,
    and the device idle gap before each step; plus a summary."""
    rows = []
    prev_end = 0.0
    for i, tm in enumerate(tms):
        h = {k: round((v - t0) * 1e6, 1) for k, v in tm.host.items()}
        g0 = origin.elapsed_time(tm.start) * 1e3
        g1 = origin.elapsed_time(tm.end) * 1e3
        call = tm.calls[0][0].elapsed_time(tm.calls[0][1]) * 1e3
        rows.append({"step": i, "host_us": h, "gpu_start_us": round(g0, 1), "gpu_end_us": round(g1, 1),
                     "gpu_span_us": round(g1 - g0, 1), "gap_before_us": round(g0 - prev_end, 1),
                     "call0_us": round(call, 1)})
        prev_end = g1
    span = np.array([r["gpu_span_us"] for r in rows])
    gap = np.array([r["gap_before_us"] for r in rows])
    host = np.array([r["host_us"]["launched"] - r["host_us"]["enter"] for r in rows])
    bm = np.array([r["host_us"]["block_manager"] - r["host_us"]["staging_free"] for r in rows])
    wait = np.array([r["host_us"]["staging_free"] - r["host_us"]["enter"] for r in rows])
    launch = np.array([r["host_us"]["launched"] - r["host_us"]["upload"] for r in rows])
    summary = {
        "wall_us_per_step": round(wall / len(rows) * 1e6, 1),
        "gpu_span_us_mean": round(float(span.mean()), 1),
        "gpu_gap_us_mean": round(float(gap[1:].mean()) if len(gap) > 1 else 0.0, 1),
        "first_step_gap_us": round(float(gap[0]), 1),
        "host_us_per_step_mean": round(float(host.mean()), 1),
        "host_staging_wait_us_mean": round(float(wait.mean()), 1),
        "host_block_manager_us_mean": round(float(bm.mean()), 1),
        "host_launch_us_mean": round(float(launch.mean()), 1),
        "note": "gpu span: compute-stream events at a step's start (after its upload wait) and end, "
                f"{layers} layers; gap: device idle between steps; host: Python time inside step()",
    }
    return {"summary": summary, "steps": rows}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=4)
    p.add_argument("--partition-size", type=int, default=-1,
                   help="-1: balanced split (default); 0: no split; >0: partitions of that many tokens")
    p.add_argument("--v-layout", choices=["dim", "token"], default="token",
                   help="in-block V layout: token-major (the KVBlock layout; default) or dim-major")
    p.add_argument("--separate-write", action="store_true",
                   help="write the new token with pa_reshape_and_cache, then pa_decode (default with the balanced "
                        "split: pa_decode_append, both in one launch)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
    p.add_argument("--workload", choices=["gqa", "gqa-calls", "long", "mixed", "prefix"], default="gqa",
                   help="gqa: the decode step on the GQA batch (default); others: decode calls on that workload "
                        "(gqa-calls: pa_decode on the GQA batch)")
    p.add_argument("--cold", action="store_true",
                   help="decode-call workloads: also time --steps single calls, each after reading a 1 GiB buffer "
                        "(evicts L2 and the Infinity Cache), reported under 'cold'")
    p.add_argument("--cold-write", action="store_true",
                   help="with --cold: write the 1 GiB buffer instead of reading it (its dirty lines are then written "
                        "back during the timed call)")
    p.add_argument("--kv", choices=["bf16", "fp8"], default="bf16", help="KV dtype of the mixed workload")
    p.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32], help="block size of the mixed workload")
    p.add_argument("--shared", action="store_true",
                   help="prefix workload: pa_decode_shared with groups of sequences sharing their prefix blocks "
                        "(--partition-size > 0, default 256)")
    p.add_argument("--stream-ref", action="store_true",
                   help="only time a plain streaming read of 4 GiB (pa_ref_stream_read), the attainable read "
                        "bandwidth the decode is compared with, and exit")
    p.add_argument("--timeline", default=None,
                   help="GQA step: write the per-step host and device timeline (JSON) to this file")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration) and exit")
    return p.parse_args()


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}))


def stream_ref(steps: int):
    """GB/s of a plain streaming read of 4 GiB (pa_ref_stream_read: 16-byte
    non-temporal loads, grid-stride, 8192 workgroups of 256 threads), mean
    over ``steps`` passes: the attainable read bandwidth."""
    import torch
    import paged_kv_cache_49_amd as pa
    n = 4 << 30
    grid = 8192
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pa.ref_stream_read(x, sink, grid)
    torch.cuda.synchronize()
    e0, e1 = HipTimingEvent(), HipTimingEvent()
    e0.record()
    for _ in range(steps):
        pa.ref_stream_read(x, sink, grid)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / steps
    print(json.dumps({"stream_ref_bytes": n, "passes": steps, "grid": grid, "us_per_pass": round(s * 1e6, 1),
                      "gbs": round(n / s / 1e9, 1), "pct_of_hbm_peak": round(100 * n / s / 1e9 / HBM_PEAK_GBS, 2)}))


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle (gather through its own block tables + naive softmax
    attention), unchanged, over all sequences of one layer, repeated until
    ``seconds``. The host cores run it side by side: a pool of threads, one
    per core this process may use, each calls the oracle on its own subset
    of sequences (round-robin, so lengths balance) with one BLAS thread
    (NumPy releases the interpreter lock inside the gathers, conversions,
    products and exponentials). The same work on one thread is timed too."""
    import concurrent.futures as cf

    import threadpoolctl

    from oracle import allocator as oalloc
    from oracle import attention as oatt
    from oracle import cache_ops as ocache

    B = wl.batch
    alloc = oalloc.BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
    kp = ocache.empty_pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    vp = ocache.empty_pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype)
    for s in range(B):
        slots, _ = alloc.alloc(s, int(wl.lengths[s]))
        k, v = wl.kv(s)
        ocache.write(kp, vp, k, v, slots, wl.kv_dtype)
    mb = max(oalloc.blocks_for(int(n), wl.block_size) for n in wl.lengths)
    tables, lens = alloc.pack(list(range(B)), mb, -1)
    tables, lens = np.asarray(tables), np.asarray(lens)
    q = wl.q()
    nbytes = 2 * int(lens.sum()) * wl.num_kv_heads * wl.head_dim * 2
    affinity = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:
        pass

    def one_pass(threads: int, pool) -> None:
        if threads == 1:
            oatt.paged_decode(q, kp, vp, tables, lens, wl.scale, wl.block_size, wl.kv_dtype)
            return
        subsets = [list(range(i, B, threads)) for i in range(threads)]
        list(pool.map(lambda ss: oatt.paged_decode(q, kp, vp, tables, lens, wl.scale, wl.block_size,
                                                   wl.kv_dtype, seqs=ss), subsets))

    def timed(threads: int, budget: float):
        with cf.ThreadPoolExecutor(max_workers=threads) as pool:
            one_pass(threads, pool)  # untimed: first-touch page faults of the working arrays
            reps, t0 = 0, time.perf_counter()
            while True:
                one_pass(threads, pool)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget or reps >= 200:
                    return reps, el

    threads = max(1, min(affinity, B))
    with threadpoolctl.threadpool_limits(1):
        reps, el = timed(threads, seconds)
        reps1, el1 = timed(1, seconds / 3)
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle paged_decode over all {B} sequences of one layer "
                      f"({int(lens.sum())} tokens, {nbytes / 1e6:.0f} MB of bf16 K/V) on {threads} threads "
                      f"(one subset of sequences each, one BLAS thread), {reps} passes in {el:.1f} s; "
                      f"tokens/s {B * reps / el:.1f}",
            "one_core_value": round(nbytes * reps1 / el1 / 1e9, 4),
            "speedup_over_one_core": round((reps / el) / (reps1 / el1), 2),
            "cpu_model": cpu_model, "affinity_cores": affinity}


def bench_decode_calls(args):
    """Back-to-back decode calls on the long-context, mixed-length or
    prefix-sharing workload; prints one JSON line."""
    import torch
    import paged_kv_cache_49_amd as pa
    import synth
    from paged_kv_cache_49_amd.runner import PagedBatch, workspace_for

    dev = "cuda"
    layers, K, W = args.layers, args.steps, args.warmup
    ps = args.partition_size
    gen = torch.Generator(device=dev).manual_seed(4903)
    extra = {}
    if args.workload == "prefix":
        wl = synth.prefix_sharing(partial_tail=True)
        P, S = wl.prompts, wl.samples
        B, Hq, Hkv, D, bs, kv = P * S, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, "bf16"
        bm = pa.BlockManager(wl.num_blocks, bs, wl.free_order)
        caches = [pa.KVCache.allocate(wl.num_blocks, bs, Hkv, D, kv, device=dev, v_layout=args.v_layout)
                  for _ in range(layers)]
        mb = int(-(-(int(wl.prefix_len.max() + wl.tail_len.max()) + 2) // bs))
        batch = PagedBatch(bm, caches, mb, B, device=dev)
        rnd = lambda n: [torch.randn(n, Hkv, D, generator=gen, device=dev).bfloat16() for _ in range(layers)]
        for p in range(P):
            n = int(wl.prefix_len[p])
            batch.prefill(p * S, rnd(n), rnd(n))
            for i in range(1, S):
                batch.fork(p * S, p * S + i)
        for p in range(P):
            for i in range(S):
                n = int(wl.tail_len[p, i]) + 1  # tail + the new token
                batch.prefill(p * S + i, rnd(n), rnd(n))
        tables, lens, max_ctx = batch.tables(list(range(B)))
        L = lens.cpu().numpy().astype(np.int64)
        unique_tokens = int(wl.prefix_len.sum()) + int((wl.tail_len + 1).sum())
        desc = (f"prefix sharing: {P} prompts x {S} samples, shared prefix 2048 + U[1,15] tokens, tails U[0,256] "
                f"+ 1 new token, 32 q heads / 8 KV heads, head_dim 128, block 16, bf16")
        if args.shared:
            ps = ps if ps > 0 else 256
            sp = bm.shared_prefixes(list(range(B)), ps)
            i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
            sargs = (i32(sp.offsets), i32(sp.members), i32(sp.shared_len), sp.num_groups, sp.max_group_size,
                     sp.max_shared_len, sp.min_shared_len)
            extra["groups"] = sp.num_groups
    else:
        wl = (synth.long_context() if args.workload == "long" else synth.gqa_decode() if args.workload == "gqa-calls"
              else synth.mixed_lengths(block_size=args.block_size, kv_dtype=args.kv))
        B, Hq, Hkv, D, bs, kv = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.kv_dtype
        sc = 6.0 / 448.0 if kv == "fp8" else 1.0
        bm = pa.BlockManager(wl.num_blocks, bs, wl.free_order)
        caches = [pa.KVCache.allocate(wl.num_blocks, bs, Hkv, D, kv, device=dev, v_layout=args.v_layout, k_scale=sc,
                                      v_scale=sc) for _ in range(layers)]
        for s in range(B):
            n = int(wl.lengths[s])
            slots, _ = bm.alloc(s, n)
            sd = torch.from_numpy(slots).to(dev)
            for c in caches:
                k = torch.randn(n, Hkv, D, generator=gen, device=dev).bfloat16()
                v = torch.randn(n, Hkv, D, generator=gen, device=dev).bfloat16()
                pa.reshape_and_cache(c, k, v, sd)
        mb = int(-(-int(wl.lengths.max()) // bs))
        t, l = bm.pack(list(range(B)), mb, -1)
        tables, lens, max_ctx = torch.from_numpy(t).to(dev), torch.from_numpy(l).to(dev), int(l.max())
        L = l.astype(np.int64)
        desc = ("long context: 8 seqs, context U[32768,131072], 32 q heads / 8 KV heads, head_dim 128, block 16, "
                "bf16" if args.workload == "long" else
                "GQA decode batch: 64 seqs, context U[512,4096], 32 q heads / 8 KV heads, head_dim 128, block 16, bf16"
                if args.workload == "gqa-calls" else
                f"mixed lengths: 256 seqs, context clip(lognormal(ln 1024, 1), 16, 16384), 64 q heads / 8 KV heads, "
                f"head_dim 128, block {bs}, KV {kv}, q bf16")
    b = 1 if kv == "fp8" else 2
    call_bytes = 2 * int(L.sum()) * Hkv * D * b
    alg_call = algorithmic_bytes(L, bs, Hq, Hkv, D, b, 2, False)
    q = torch.randn(B, Hq, D, generator=gen, device=dev).bfloat16()
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    shared = args.workload == "prefix" and args.shared
    ws = workspace_for(B, Hq, Hkv, D, max_ctx, ps, device=dev, shared=shared)
    if shared:
        call = lambda c: pa.decode_shared(c, q, tables, lens, max_ctx, wl.scale, ps, *sargs, out=out, workspace=ws)
        kernel = ("pa_decode_shared (token-major V or fp8: the cascade, paged_decode_sk_kernel<..., cascade> + "
                  "decode_cascade_merge_kernel; dim-major 16-bit V: paged_decode_shared_kernel + "
                  f"decode_reduce_kernel; PA_SHARED_PATH={os.environ.get('PA_SHARED_PATH', 'auto')})")
    else:
        call = lambda c: pa.decode(c, q, tables, lens, max_ctx, wl.scale, ps, out=out, workspace=ws)
        kernel = ("pa_decode (paged_decode_sk_kernel + decode_sk_merge_kernel)" if ps < 0 else
                  f"pa_decode (partitions of {ps} tokens: the staged kernel in partition mode + "
                  f"decode_sk_merge_kernel, or the one-wave partition kernel + decode_reduce_kernel; "
                  f"PA_PARTITION_PATH={os.environ.get('PA_PARTITION_PATH', 'auto')})" if ps > 0
                  else "pa_decode (one partition)")
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: B={B} tokens={int(L.sum())} layers={layers} KV {call_bytes / 1e6:.0f} MB/call",
          file=sys.stderr, flush=True)
    for _ in range(W):
        for c in caches:
            call(c)
    torch.cuda.synchronize()
    e0, e1 = HipTimingEvent(), HipTimingEvent()
    per = [(HipTimingEvent(), HipTimingEvent()) for _ in range(K)]
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        for li, c in enumerate(caches):
            if li == 0:
                per[i][0].record()
            call(c)
            if li == 0:
                per[i][1].record()
    e1.record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    call_s = e0.elapsed_time(e1) * 1e-3 / (K * layers)
    value = call_bytes / call_s / 1e9
    durs = np.array([a.elapsed_time(b) for a, b in per]) * 1e-3
    print(f"[bench] {K * layers} calls: {call_s * 1e6:.1f} us/call (layer 0: median {np.median(durs) * 1e6:.1f}, "
          f"min {durs.min() * 1e6:.1f})", file=sys.stderr, flush=True)
    extra["pa_decode_us_median"] = round(float(np.median(durs)) * 1e6, 2)
    extra["pa_decode_us_min"] = round(float(durs.min()) * 1e6, 2)
    if args.cold:
        scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        sink = torch.empty((), dtype=torch.float32, device=dev)
        cold = []
        for i in range(K):
            if args.cold_write:
                scratch.fill_(float(i))
            else:
                torch.sum(scratch, dim=0, out=sink)
            a, b2 = HipTimingEvent(), HipTimingEvent()
            a.record()
            call(caches[i % layers])
            b2.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b2) * 1e-3)
        cold = np.array(cold)
        extra["cold"] = {"calls": K, "median_us": round(float(np.median(cold)) * 1e6, 2),
                         "min_us": round(float(cold.min()) * 1e6, 2),
                         "gbs_median": round(call_bytes / float(np.median(cold)) / 1e9, 2),
                         "note": f"each call after a 1 GiB device {'write' if args.cold_write else 'read'} "
                                 f"(cold L2 and Infinity Cache), timed alone"}
        print(f"[bench] cold calls: median {np.median(cold) * 1e6:.1f} us", file=sys.stderr, flush=True)
    if args.workload == "prefix":
        extra["unique_kv_gbs"] = round(2 * unique_tokens * Hkv * D * b / call_s / 1e9, 2)
        extra["unique_kv_note"] = "KV bytes of distinct tokens (shared prefix counted once per prompt) / call time"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(el / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": kv,
        "data": "synthetic (seeded lengths and block ids; K/V/q drawn N(0,1) on the device)",
        "config": {"workload": desc, "batch": B, "layers": layers, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": bs, "partition_size": ps, "v_layout": args.v_layout,
                   "step": f"{layers} decode calls back to back (one per layer)",
                   "mean_context": round(float(L.mean()), 1)},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B / call_s, 1),
        "decode_tokens_per_s_note": "sequences per second of one layer's call",
        "pa_decode_us": round(call_s * 1e6, 2),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(alg_call / call_s / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(alg_call / call_s / 1e9 / HBM_PEAK_GBS, 4),
                     "frac_events": round(alg_call / call_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_call": alg_call,
                     "algorithmic_note": "K/V rows of the valid tokens (logical: shared blocks counted per "
                                         "sequence), table entries, q and out rows, lengths"},
        "cpu_baseline": None,
        **extra,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (this path has no "
              f"multi-GPU leg: each GPU would run its own share with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.stream_ref:
        stream_ref(max(args.steps, 5))
        return

    if args.workload != "gqa":
        bench_decode_calls(args)
        return

    import paged_kv_cache_49_amd as pa
    import synth
    from paged_kv_cache_49_amd.runner import PagedBatch, StepTiming, workspace_for

    pa.lib()
    torch.cuda.set_device(0)
    dev = "cuda"
    wl = synth.gqa_decode()
    B, Hq, Hkv, D, bs = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    layers, K, W = args.layers, args.steps, args.warmup
    L0 = wl.lengths.astype(np.int64)
    grow = W + K + 1
    max_blocks = int(-(-(int(L0.max()) + grow) // bs))
    num_blocks = wl.num_blocks
    print(f"[bench] gqa decode: B={B} Hq={Hq} Hkv={Hkv} D={D} bs={bs} layers={layers} "
          f"tokens={int(L0.sum())} pool={num_blocks} blocks", file=sys.stderr, flush=True)

    # ---- setup: every layer's pool written through the library
    bm = pa.BlockManager(num_blocks, bs, wl.free_order)
    caches = [pa.KVCache.allocate(num_blocks, bs, Hkv, D, "bf16", device=dev, v_layout=args.v_layout)
              for _ in range(layers)]
    batch = PagedBatch(bm, caches, max_blocks, B, device=dev, pad=0)
    gen = torch.Generator(device=dev).manual_seed(4902)
    for s in range(B):
        k, v = wl.kv(s)
        kd, vd = k.to(dev), v.to(dev)
        ks = [kd] + [torch.randn(kd.shape, generator=gen, device=dev).bfloat16() for _ in range(layers - 1)]
        vs = [vd] + [torch.randn(vd.shape, generator=gen, device=dev).bfloat16() for _ in range(layers - 1)]
        batch.prefill(s, ks, vs)
    q = [wl.q().to(dev)] + [torch.randn(B, Hq, D, generator=gen, device=dev).bfloat16() for _ in range(layers - 1)]
    k_new = [torch.randn(B, Hkv, D, generator=gen, device=dev).bfloat16() for _ in range(layers)]
    v_new = [torch.randn(B, Hkv, D, generator=gen, device=dev).bfloat16() for _ in range(layers)]
    outs = [torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    ws = workspace_for(B, Hq, Hkv, D, max_blocks * bs, args.partition_size, device=dev)
    ids = np.arange(B, dtype=np.int64)
    ones = np.ones(B, np.int32)
    torch.cuda.synchronize()
    print("[bench] setup done", file=sys.stderr, flush=True)

    fused = args.partition_size == pa.BALANCED and not args.separate_write
    # every timing event (warm-up and timed steps) exists before the first
    # step: the warm-up runs exactly the timed path, events included, and no
    # event is created inside the timed region
    warm_tm = [StepTiming(HipTimingEvent) for _ in range(W)]
    step_tm = [StepTiming(HipTimingEvent) for _ in range(K)]
    origin = HipTimingEvent()
    for tm in warm_tm:
        batch.step(ids, k_new, v_new, q, outs, wl.scale, args.partition_size, ws, ones, timing=tm, fused=fused)
    torch.cuda.synchronize()
    lens_before = L0 + W

    batch.host_seconds, batch.host_steps = 0.0, 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    origin.record()
    for tm in step_tm:
        batch.step(ids, k_new, v_new, q, outs, wl.scale, args.partition_size, ws, ones, timing=tm, fused=fused)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    el = t1 - t0
    timeline = step_timeline(step_tm, origin, t0, el, layers)
    if args.timeline:
        with open(args.timeline, "w") as fh:
            json.dump(timeline, fh, indent=1)

    kv_row = 2 * Hkv * D * 2  # K and V bytes of one token of one sequence (bf16)
    step_bytes = [layers * kv_row * int((lens_before + i + 1).sum()) for i in range(K)]
    total_bytes = float(sum(step_bytes))
    durs = np.array([tm.calls[0][0].elapsed_time(tm.calls[0][1]) for tm in step_tm]) * 1e-3  # seconds
    per_call_bytes = total_bytes / (K * layers)  # every layer of a step reads the same bytes
    # all bytes a call moves at the least (K/V, tables, q, out, the appended row), mean over the timed calls
    alg_call = float(np.mean([algorithmic_bytes(lens_before + i + 1, bs, Hq, Hkv, D, 2, 2, fused)
                              for i in range(K)]))
    call_s = float(durs.mean())
    achieved = alg_call / call_s / 1e9
    prof = load_profile()
    value = total_bytes / el / 1e9
    print(f"[bench] {K} steps in {el * 1e3:.2f} ms; pa_decode mean {call_s * 1e6:.1f} us "
          f"(min {durs.min() * 1e6:.1f}, max {durs.max() * 1e6:.1f})", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(el / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q, lengths U[512,4096], shuffled block ids)",
        "config": {
            "workload": "GQA decode batch: 64 seqs, context U[512,4096], 32 q heads / 8 KV heads, head_dim 128, "
                        "block 16, bf16; one decode step per layer, layers share block tables",
            "batch": B, "layers": layers, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": bs, "partition_size": args.partition_size, "v_layout": args.v_layout,
            "step": "pa_decode_append (write + attention, one launch)" if fused else
                    "pa_reshape_and_cache + pa_decode",
            "mean_context": round(float(lens_before.mean()) + (K + 1) / 2, 1),
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(B * layers * K / el, 1),
        "decode_tokens_per_s_note": "sequences x layers per second (one query token per sequence per layer)",
        "decode_tokens_per_s_call": round(B / call_s, 1),
        "decode_tokens_per_s_call_note": "B / mean pa_decode call time (sequences one call decodes per second)",
        "pa_decode_us": round(call_s * 1e6, 2),
        "pa_decode_us_median": round(float(np.median(durs)) * 1e6, 2),
        "pa_decode_us_min": round(float(durs.min()) * 1e6, 2),
        "host_block_manager_us_per_step": round(batch.host_seconds / max(batch.host_steps, 1) * 1e6, 2),
        "host_block_manager_note": "pa_alloc_batch + pa_bm_pack of the whole batch on the host, inside each step",
        "setup_upload_stalls_s": batch.warm_stalls,
        "gpu_busy_frac": round(layers * call_s / (el / K), 4),
        "gpu_busy_note": "layers x mean pa_decode call time / step wall time",
        "step_timeline": timeline["summary"],
        "roofline": {
            "bound": "hbm",
            "kernel": (("pa_decode_append" if fused else "pa_decode") +
                       (" (paged_decode_sk_kernel + decode_sk_merge_kernel)" if args.partition_size < 0
                        else " (partition kernel + decode_reduce_kernel)")),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": prof["traffic"]["bytes_per_call"] if prof else None,
            "traffic_unit": "HBM bytes per call (FETCH_SIZE + WRITE_SIZE of K1 + K2, calibrated on a 1 GiB copy)",
            "traffic_per_algorithmic_byte": prof["traffic"]["per_algorithmic_byte"] if prof else None,
            "algorithmic_bytes_per_call": round(alg_call),
            "algorithmic_note": "per call: K/V rows of the valid tokens, block-table entries, q and out rows, "
                                "the appended token's K/V row, lengths and slots; achieved = that / the mean "
                                "HIP-event duration of layer 0's call (both launches and the gap between them)",
            "frac_events": round(achieved / HBM_PEAK_GBS, 4),
            "frac_kernel": prof["frac_kernel"] if prof else None,
            "frac_kernel_note": ("algorithmic bytes per call of the profiled run / the rocprofv3 average duration "
                                 "of K1 (paged_decode_sk_kernel) and of K1 + K2 (+ decode_sk_merge_kernel), "
                                 "from profiles/decode_gqa_profile.json" if prof else
                                 "kernel sources changed since the committed profile: not recomputed"),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
