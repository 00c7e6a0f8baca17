"""Host-side sequencing of library calls for a batch of sequences.

``PagedBatch`` ties one BlockManager (host tables) to one or more KVCache
pools (e.g. one per attention layer, all indexed by the same block tables)
and runs the serving loop's steps through the C ABI:

  prefill(seq, K, V)   allocate L slots, write every layer's K/V rows
  fork(parent, child)  share all blocks (refcounts)
  step(...)            one decode step for a batch: allocate one slot per
                       sequence (copy-on-write pairs included), upload the
                       slot mapping / pairs / tables / lengths in a single
                       host-to-device copy from pinned memory, then per layer
                       pa_copy_blocks -> pa_reshape_and_cache -> pa_decode,
                       or with ``fused=True`` pa_copy_blocks ->
                       pa_decode_append (the write and the attention in one
                       launch; balanced split, 16-bit pools), or with
                       ``shared=True`` ... -> pa_decode_shared (each group
                       of forks reads its shared prefix once)

The metadata staging area is double-buffered: a buffer is refilled only
after the copy issued from it two steps earlier has completed (HIP event),
so the host can run ahead of the device without overwriting data in flight.
By default the upload runs on a copy stream of its own (default priority):
it overlaps the previous step's kernels, and the step's first kernel waits
only for an event that has long fired. The copy into a device buffer waits
for the kernels of the step that last read it (two steps earlier).
"""
from __future__ import annotations

import time
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import (BALANCED, BlockManager, KVCache, copy_blocks, decode_shared_workspace_size, decode_workspace_size,
               prepare_decode, prepare_decode_append, prepare_decode_shared, reshape_and_cache)


class _Staging:
    """Pinned host buffer + device buffer with the step metadata layout:
    slots int64[B] | cow int32[B][2] | lens int32[B] | tables int32[B][W] |
    shared-prefix groups: offsets int32[B/2+1] | members int32[B] |
    shared_len int32[B]."""

    def __init__(self, batch: int, max_blocks: int, device):
        self.B, self.W = batch, max_blocks
        ng = batch // 2 + 1
        n32 = 2 * batch + 2 * batch + batch + batch * max_blocks + ng + 2 * batch
        self.host = torch.empty(n32, dtype=torch.int32, pin_memory=True)
        self.dev = torch.empty(n32, dtype=torch.int32, device=device)
        h = self.host.numpy()
        self.slots_np = h[: 2 * batch].view(np.int64)
        self.cow_np = h[2 * batch: 4 * batch].reshape(batch, 2)
        self.lens_np = h[4 * batch: 5 * batch]
        t_end = 5 * batch + batch * max_blocks
        self.tables_np = h[5 * batch:t_end].reshape(batch, max_blocks)
        self.goff_np = h[t_end:t_end + ng]
        self.gmem_np = h[t_end + ng:t_end + ng + batch]
        self.shl_np = h[t_end + ng + batch:t_end + ng + 2 * batch]
        d = self.dev
        self.slots = d[: 2 * batch].view(torch.int64)
        self.cow = d[2 * batch: 4 * batch].view(batch, 2)
        self.lens = d[4 * batch: 5 * batch]
        self.tables = d[5 * batch:t_end].view(batch, max_blocks)
        self.goff = d[t_end:t_end + ng]
        self.gmem = d[t_end + ng:t_end + ng + batch]
        self.shl = d[t_end + ng + batch:t_end + ng + 2 * batch]
        self.copied: Optional[torch.cuda.Event] = None    # after the upload into `dev`
        self.consumed: Optional[torch.cuda.Event] = None  # after the last kernel that read `dev`


class PagedBatch:
    def __init__(self, bm: BlockManager, caches: Sequence[KVCache], max_blocks: int, batch: int,
                 device="cuda", pad: int = -1, upload_stream: bool = True):
        self.bm = bm
        self.caches = list(caches)
        self.max_blocks = int(max_blocks)
        self.device = device
        self.pad = int(pad)
        self._stage = [_Staging(batch, self.max_blocks, device) for _ in range(2)]
        self._turn = 0
        self._copy_stream = torch.cuda.Stream(device=device) if upload_stream else None
        if self._copy_stream is not None:
            self._warm_upload_path()
        self.last_cow_count = 0
        # host time of the block-manager work of the steps (alloc_batch,
        # pack, shared_prefixes), seconds, and the number of steps it covers
        self.host_seconds = 0.0
        self.host_steps = 0

    def _warm_upload_path(self, rounds: int = 16) -> None:
        """Queue ``rounds`` metadata uploads on the copy stream, each behind
        compute-stream work that is certain to be still running (1 GiB of
        fills, ~0.2 ms), and wait for all.

        Measured on MI355X (ROCm 7.2): besides the first pinned
        host-to-device copy of a process, one of the first few copies queued
        on a second stream behind unfinished work of the compute stream
        blocks the calling thread for ~6 ms while the GPU idles (plain
        hipMemcpyAsync behaves the same); whether a copy meets unfinished
        work depends on timing, so a short warm-up can miss it and leave the
        stall to a later decode step. Taking it here keeps it out of the
        steps. ``warm_stalls`` records the enqueue times above 1 ms (seconds).
        The staging buffers' contents are overwritten by every step."""
        compute = torch.cuda.current_stream(self.device)
        cs = self._copy_stream
        busy = torch.empty(64 << 20, dtype=torch.int32, device=self.device)
        ready = [torch.cuda.Event(), torch.cuda.Event()]
        copied = [torch.cuda.Event(), torch.cuda.Event()]
        self.warm_stalls = []
        for i in range(rounds):
            st = self._stage[i % 2]
            for _ in range(4):
                busy.fill_(i)  # work the upload waits for, still running when it is queued
            ready[i % 2].record(compute)
            cs.wait_event(ready[i % 2])
            t0 = time.perf_counter()
            with torch.cuda.stream(cs):
                st.dev.copy_(st.host, non_blocking=True)
            dt = time.perf_counter() - t0
            if dt > 1e-3:
                self.warm_stalls.append(round(dt, 4))
            copied[i % 2].record(cs)
            compute.wait_event(copied[i % 2])
        torch.cuda.synchronize(self.device)

    # -- setup ---------------------------------------------------------------
    def prefill(self, seq_id: int, ks: Sequence[torch.Tensor], vs: Sequence[torch.Tensor]) -> np.ndarray:
        """Append len(ks[0]) tokens to ``seq_id`` and write layer i's rows
        ks[i], vs[i] ([L][Hkv][D]). Returns the slots (host)."""
        L = int(ks[0].shape[0])
        slots, cows = self.bm.alloc(seq_id, L)
        if cows:
            pairs = torch.tensor(cows, dtype=torch.int32, device=self.device)
            for c in self.caches:
                copy_blocks(c, pairs)
        if L:
            sd = torch.from_numpy(slots).to(self.device)
            for c, k, v in zip(self.caches, ks, vs):
                reshape_and_cache(c, k.to(self.device, non_blocking=False).contiguous(),
                                  v.to(self.device, non_blocking=False).contiguous(), sd)
        return slots

    def fork(self, parent: int, child: int) -> None:
        self.bm.fork(parent, child)

    def tables(self, seq_ids: Sequence[int]):
        """Device (tables, lens) of ``seq_ids`` (synchronous upload)."""
        t, l = self.bm.pack(seq_ids, self.max_blocks, self.pad)
        return (torch.from_numpy(t).to(self.device), torch.from_numpy(l).to(self.device), int(l.max(initial=0)))

    # -- one decode step -----------------------------------------------------
    def step(self, seq_ids: np.ndarray, k_new: Sequence[torch.Tensor], v_new: Sequence[torch.Tensor],
             q: Sequence[torch.Tensor], outs: Sequence[torch.Tensor], scale: float, partition_size: int,
             workspace: Optional[torch.Tensor] = None, ones: Optional[np.ndarray] = None,
             timing: Optional["StepTiming"] = None, fused: bool = False, shared: bool = False) -> int:
        """Append one token to each of ``seq_ids`` in every layer and run
        decode attention for it. Returns the batch's max context length.
        With ``timing`` (a StepTiming, its events created beforehand), the
        step records host timestamps of its phases and device events at its
        start and end on the compute stream and around the decode call of
        each layer the StepTiming names.

        ``shared=True``: the rows whose tables start with the same blocks
        (forks of one prompt) are grouped (pa_bm_shared_prefixes, granule =
        ``partition_size``) and decoded with pa_decode_shared, which reads
        each group's shared partitions once."""
        tm = timing
        if tm is not None:
            tm.host["enter"] = time.perf_counter()
        st = self._stage[self._turn]
        self._turn ^= 1
        if st.copied is not None:
            st.copied.synchronize()  # the pinned buffer's previous upload is done
        if tm is not None:
            tm.host["staging_free"] = time.perf_counter()
        B = len(seq_ids)
        if ones is None:
            ones = np.ones(B, np.int32)
        t_host = time.perf_counter()
        _, cows = self.bm.alloc_batch(seq_ids, ones, slot_out=st.slots_np, cow_out=st.cow_np)
        ncow = len(cows)
        self.bm.pack(seq_ids, self.max_blocks, self.pad, tables=st.tables_np, context_lens=st.lens_np)
        max_ctx = int(st.lens_np[:B].max(initial=0))
        groups = None
        if shared:
            if fused or partition_size <= 0:
                raise ValueError("shared steps need partition_size > 0 and fused=False")
            groups = self.bm.shared_prefixes(seq_ids, partition_size, group_offsets=st.goff_np,
                                             group_members=st.gmem_np, shared_len=st.shl_np)
        t_bm = time.perf_counter()
        self.host_seconds += t_bm - t_host
        self.host_steps += 1
        if tm is not None:
            tm.host["block_manager"] = t_bm
        compute = torch.cuda.current_stream(self.device)
        if st.copied is None:
            st.copied, st.consumed = torch.cuda.Event(), torch.cuda.Event()
        if self._copy_stream is None:
            st.dev.copy_(st.host, non_blocking=True)
            st.copied.record(compute)
        else:
            cs = self._copy_stream
            cs.wait_event(st.consumed)  # kernels of the step that last read st.dev (no-op before any record)
            with torch.cuda.stream(cs):
                st.dev.copy_(st.host, non_blocking=True)
            st.copied.record(cs)
            compute.wait_event(st.copied)
        if tm is not None:
            tm.host["upload"] = time.perf_counter()
            tm.start.record()  # on the compute stream, after the wait for the upload
        self.last_cow_count = ncow
        tables = st.tables if B == st.B else st.tables[:B]
        lens = st.lens[:B]
        for i, c in enumerate(self.caches):
            if ncow:
                copy_blocks(c, st.cow[:ncow])
            if not fused:
                reshape_and_cache(c, k_new[i], v_new[i], st.slots[:B])
            ev = tm.calls.get(i) if tm is not None else None
            # arguments marshalled before the start event, so the timed
            # interval holds the launch alone (no host work)
            if fused:
                if partition_size != BALANCED:
                    raise ValueError("fused steps use the balanced split (partition_size = BALANCED)")
                launch = prepare_decode_append(c, k_new[i], v_new[i], st.slots[:B], q[i], tables, lens, max_ctx,
                                               scale, out=outs[i], workspace=workspace)
            elif groups is not None:
                launch = prepare_decode_shared(c, q[i], tables, lens, max_ctx, scale, partition_size, st.goff,
                                               st.gmem[:B], st.shl[:B], groups.num_groups, groups.max_group_size,
                                               groups.max_shared_len, groups.min_shared_len, out=outs[i],
                                               workspace=workspace)
            else:
                launch = prepare_decode(c, q[i], tables, lens, max_ctx, scale, partition_size, out=outs[i],
                                        workspace=workspace)
            if ev is not None:
                ev[0].record()
            launch()
            if ev is not None:
                ev[1].record()
        st.consumed.record(compute)
        if tm is not None:
            tm.end.record()
            tm.host["launched"] = time.perf_counter()
        return max_ctx


class StepTiming:
    """Timing of one PagedBatch.step, its events created up front (so that
    creating them costs nothing inside a timed region): ``start`` / ``end``
    recorded on the compute stream at the step's start (after its wait for
    the metadata upload) and end, ``calls[layer]`` = (start, end) around
    that layer's decode launch, and ``host`` = perf_counter() stamps of the
    step's phases (enter, staging_free, block_manager, upload, launched).
    ``make_event()`` returns an object with ``record()`` (on the current
    stream) and ``elapsed_time(other)`` in milliseconds."""

    def __init__(self, make_event, call_layers: Sequence[int] = (0,)):
        self.start, self.end = make_event(), make_event()
        self.calls = {int(i): (make_event(), make_event()) for i in call_layers}
        self.host: dict = {}


def workspace_for(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                  partition_size: int, device="cuda", shared: bool = False) -> Optional[torch.Tensor]:
    """A workspace for decode calls of these sizes (shared=True: one that
    also serves decode_shared)."""
    size = decode_shared_workspace_size if shared else decode_workspace_size
    with torch.cuda.device(device):
        n = size(batch, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None
