"""Benchmark: paged decode attention on one MI355X.

Workload (seeded synthetic, no dataset): the GQA decode batch — 64
sequences with context lengths U[512, 4096], 32 query heads over 8 KV heads
(group 4), head_dim 128, 16-token blocks, bf16 K/V/q, a pool of all blocks
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
KERNEL_SOURCES = ["decode_sk_kernel.h", "decode_vt_kernel.h", "decode_kernel.h", "decode_dispatch.h", "decode.hip",
                  "device_common.h", "decode_sk_bf16.hip", "decode_vt_bf16.hip"]


def kernel_hash() -> str:
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_49_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes (read + written) of one pa_decode call from the committed
    counter summary, and their ratio to the algorithmic bytes of the counted
    calls; (None, None) when the kernel sources changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", "decode_gqa_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    if t.get("kernel_hash") != kernel_hash():
        return None, None
    hbm, alg = t.get("hbm_bytes_per_call"), t.get("algorithmic_bytes_per_call_of_counted_run")
    return hbm, (round(hbm / alg, 4) if hbm and alg else None)


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


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=4)
    p.add_argument("--partition-size", type=int, default=-1,
                   help="-1: balanced split (default); 0: no split; >0: partitions of that many tokens")
    p.add_argument("--v-layout", choices=["dim", "token"], default="dim",
                   help="in-block V layout: dim-major (matrix-core PV) or the token-major KVBlock layout")
    p.add_argument("--separate-write", action="store_true",
                   help="write the new token with pa_reshape_and_cache, then pa_decode (default with the balanced "
                        "split: pa_decode_append, both in one launch)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for cpu_baseline")
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


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle (gather through its own block tables + naive softmax
    attention) over all sequences of one layer, repeated until ``seconds``."""
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
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    reps, t0 = 0, time.perf_counter()
    while True:
        oatt.paged_decode(q, kp, vp, tables, lens, wl.scale, wl.block_size, wl.kv_dtype)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 200:
            break
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"fp64 oracle paged_decode over all {B} sequences of one layer "
                      f"({int(lens.sum())} tokens, {nbytes / 1e6:.0f} MB of bf16 K/V), {reps} repeats in "
                      f"{el:.1f} s; tokens/s {B * reps / el:.1f}"}


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

    import paged_kv_cache_49_amd as pa
    import synth
    from paged_kv_cache_49_amd.runner import PagedBatch, workspace_for

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

    fused = args.partition_size == pa.BALANCED and args.v_layout == "dim" and not args.separate_write
    for _ in range(W):
        batch.step(ids, k_new, v_new, q, outs, wl.scale, args.partition_size, ws, ones, fused=fused)
    torch.cuda.synchronize()
    lens_before = L0 + W

    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        batch.step(ids, k_new, v_new, q, outs, wl.scale, args.partition_size, ws, ones, decode_events=events,
                   event_layers=(0,), make_event=HipTimingEvent, fused=fused)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    el = t1 - t0

    kv_row = 2 * Hkv * D * 2  # K and V bytes of one token of one sequence (bf16)
    step_bytes = [layers * kv_row * int((lens_before + i + 1).sum()) for i in range(K)]
    total_bytes = float(sum(step_bytes))
    durs = np.array([a.elapsed_time(b) for a, b in events]) * 1e-3  # seconds
    per_call_bytes = total_bytes / (K * layers)  # every layer of a step reads the same bytes
    call_s = float(durs.mean())
    achieved = per_call_bytes / call_s / 1e9
    traffic, traffic_ratio = load_traffic()
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
        "pa_decode_us": round(call_s * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": (("pa_decode_append" if fused else "pa_decode") +
                       (" (paged_decode_sk_kernel + decode_sk_merge_kernel)" if args.partition_size < 0
                        else " (partition kernel + decode_reduce_kernel)")),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per pa_decode call (FETCH_SIZE + WRITE_SIZE, calibrated)",
            "traffic_per_algorithmic_byte": traffic_ratio,
            "algorithmic_bytes_per_call": round(per_call_bytes),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
