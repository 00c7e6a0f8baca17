"""Python binding for libpagedattn: paged KV cache and PagedAttention decode
on AMD MI355X (gfx950).

The functions here only marshal arguments (tensor pointers, dtype codes,
the current HIP stream) into the C ABI declared in include/libpagedattn.h;
every step of the path runs in the library's host C++ and HIP kernels.
Device tensors come from PyTorch (memory and streams only). A missing
library raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib
from ._lib import PaBmStats, PaKvCache, lib

__all__ = [
    "PagedAttnError", "OutOfBlocks", "UnknownSeq", "SeqExists", "Unsupported", "InvalidArgument",
    "DeviceError", "BlockManager", "KVCache", "reshape_and_cache", "copy_blocks", "decode",
    "decode_workspace_size", "decode_shared_workspace_size", "decode_append", "prepare_decode", "prepare_decode_append", "prepare_decode_shared", "decode_shared", "SharedPrefixes", "copy_blocks_between", "lib",
    "BALANCED",
]


class PagedAttnError(RuntimeError):
    status = -1

    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class InvalidArgument(PagedAttnError):
    pass


class OutOfBlocks(PagedAttnError):
    pass


class UnknownSeq(PagedAttnError):
    pass


class SeqExists(PagedAttnError):
    pass


class Unsupported(PagedAttnError):
    pass


class DeviceError(PagedAttnError):
    pass


class OutOfHostMemory(PagedAttnError):
    pass


_ERRORS = {
    _lib.PA_ERR_INVALID_ARGUMENT: InvalidArgument,
    _lib.PA_ERR_OUT_OF_BLOCKS: OutOfBlocks,
    _lib.PA_ERR_UNKNOWN_SEQ: UnknownSeq,
    _lib.PA_ERR_SEQ_EXISTS: SeqExists,
    _lib.PA_ERR_UNSUPPORTED: Unsupported,
    _lib.PA_ERR_DEVICE: DeviceError,
    _lib.PA_ERR_OUT_OF_HOST_MEMORY: OutOfHostMemory,
}


def _status_name(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _check(status: int) -> None:
    if status != _lib.PA_OK:
        msg = lib().pa_last_error().decode()
        raise _ERRORS.get(status, PagedAttnError)(status, msg)


_DTYPE_CODES = {
    torch.float16: _lib.PA_F16,
    torch.bfloat16: _lib.PA_BF16,
    torch.float32: _lib.PA_F32,
    torch.uint8: _lib.PA_FP8_E4M3,
    torch.float8_e4m3fn: _lib.PA_FP8_E4M3,
}
_NAMES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPE_CODES[t.dtype]
    except KeyError:
        raise Unsupported(_lib.PA_ERR_UNSUPPORTED, f"tensor dtype {t.dtype}") from None


def _dev(t: Optional[torch.Tensor], name: str) -> int:
    """Device pointer of a GPU tensor (never copies host data to the device)."""
    if t is None:
        return 0
    if not t.is_cuda:
        raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT, f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _host_i64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _host_i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------------------
# host block manager


@dataclasses.dataclass
class SharedPrefixes:
    """Output of BlockManager.shared_prefixes (host arrays): group gi's batch
    rows are members[offsets[gi]:offsets[gi + 1]]; shared_len[row] tokens."""
    offsets: np.ndarray
    members: np.ndarray
    shared_len: np.ndarray
    num_groups: int
    max_group_size: int
    max_shared_len: int
    min_shared_len: int = 0  # smallest shared_len over the batch rows

    def groups(self) -> list:
        return [self.members[self.offsets[g]:self.offsets[g + 1]].tolist() for g in range(self.num_groups)]


class BlockManager:
    """Owns a pa_bm handle (see include/libpagedattn.h for the semantics)."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        h = ctypes.c_void_p()
        order = None if initial_free_order is None else _host_i32(initial_free_order)
        _check(lib().pa_bm_create(int(num_blocks), int(block_size), None if order is None else _ptr(order),
                                  ctypes.byref(h)))
        self._h = h
        # held here so that destruction at interpreter exit does not depend
        # on module globals, which may already be gone then
        self._destroy = lib().pa_bm_destroy
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    def alloc(self, seq_id: int, num_new_tokens: int) -> Tuple[np.ndarray, list]:
        slots = np.empty(max(int(num_new_tokens), 0), dtype=np.int64)
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_alloc(self._h, int(seq_id), int(num_new_tokens), _ptr(slots) if slots.size else None,
                              ctypes.byref(src), ctypes.byref(dst), ctypes.byref(n)))
        return slots, ([(src.value, dst.value)] if n.value else [])

    def alloc_batch(self, seq_ids, num_new_tokens, slot_out: Optional[np.ndarray] = None,
                    cow_out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Returns (slots int64[sum], cow pairs int32[k][2]). ``slot_out`` /
        ``cow_out`` may be preallocated (e.g. numpy views of pinned memory)."""
        ids = _host_i64(seq_ids)
        nt = _host_i32(num_new_tokens)
        total = int(np.clip(nt, 0, None).sum())
        slots = np.empty(total, np.int64) if slot_out is None else slot_out
        cows = np.empty((max(len(ids), 1), 2), np.int32) if cow_out is None else cow_out
        n = ctypes.c_int32()
        _check(lib().pa_alloc_batch(self._h, _ptr(ids), len(ids), _ptr(nt), _ptr(slots) if total else None,
                                    _ptr(cows), ctypes.byref(n)))
        return slots[:total], cows[: n.value]

    def free(self, seq_id: int) -> None:
        _check(lib().pa_free(self._h, int(seq_id)))

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(lib().pa_fork(self._h, int(parent_id), int(child_id)))

    def seq_info(self, seq_id: int) -> Tuple[int, int]:
        L, nb = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_seq_info(self._h, int(seq_id), ctypes.byref(L), ctypes.byref(nb)))
        return L.value, nb.value

    def seq_blocks(self, seq_id: int) -> list:
        _, nb = self.seq_info(seq_id)
        out = np.empty(max(nb, 1), np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_seq_blocks(self._h, int(seq_id), _ptr(out), nb, ctypes.byref(n)))
        return out[: n.value].tolist()

    def pack(self, seq_ids, max_blocks: int, pad: int = -1, tables: Optional[np.ndarray] = None,
             context_lens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        ids = _host_i64(seq_ids)
        if tables is None:
            tables = np.empty((len(ids), max_blocks), np.int32)
        if context_lens is None:
            context_lens = np.empty(len(ids), np.int32)
        _check(lib().pa_pack_block_tables(self._h, _ptr(ids), len(ids), int(max_blocks), int(pad),
                                          _ptr(tables), _ptr(context_lens)))
        return tables, context_lens

    def shared_prefixes(self, seq_ids, granule: int, group_offsets: Optional[np.ndarray] = None,
                        group_members: Optional[np.ndarray] = None, shared_len: Optional[np.ndarray] = None):
        """pa_bm_shared_prefixes: groups of the rows of ``seq_ids`` whose
        tables start with the same blocks. Returns a SharedPrefixes of host
        arrays (written into the given ones when provided)."""
        ids = _host_i64(seq_ids)
        n = len(ids)
        if group_offsets is None:
            group_offsets = np.zeros(n // 2 + 1, np.int32)
        if group_members is None:
            group_members = np.zeros(max(n, 1), np.int32)
        if shared_len is None:
            shared_len = np.zeros(max(n, 1), np.int32)
        ng, gmax, smax = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_bm_shared_prefixes(self._h, _ptr(ids) if n else None, n, int(granule), _ptr(group_offsets),
                                           _ptr(group_members), _ptr(shared_len), ctypes.byref(ng),
                                           ctypes.byref(gmax), ctypes.byref(smax)))
        smin = int(shared_len[:n].min()) if n else 0
        return SharedPrefixes(group_offsets, group_members, shared_len, ng.value, gmax.value, smax.value, smin)

    # -- prefix caching -------------------------------------------------
    def set_prefix_cache(self, enable: bool) -> None:
        _check(lib().pa_bm_set_prefix_cache(self._h, 1 if enable else 0))

    def alloc_prompt(self, seq_id: int, token_ids) -> Tuple[np.ndarray, int]:
        """pa_alloc_prompt: (slots of all tokens, tokens covered by reused
        cached blocks)."""
        toks = _host_i32(token_ids)
        slots = np.empty(max(len(toks), 1), np.int64)
        nc = ctypes.c_int32()
        _check(lib().pa_alloc_prompt(self._h, int(seq_id), _ptr(toks) if len(toks) else None, len(toks),
                                     _ptr(slots), ctypes.byref(nc)))
        return slots[: len(toks)], nc.value

    def prefix_cache_stats(self) -> dict:
        a, b = ctypes.c_int32(), ctypes.c_int32()
        c, d, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_bm_prefix_cache_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                              ctypes.byref(d), ctypes.byref(e)))
        return dict(num_cached_blocks=a.value, num_evictable=b.value, hits=c.value, misses=d.value,
                    evictions=e.value)

    def evictable(self) -> list:
        out = np.empty(self.num_blocks, np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_bm_evictable(self._h, _ptr(out), self.num_blocks, ctypes.byref(n)))
        return out[: n.value].tolist()

    # -- swapping (host pool) -------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        _check(lib().pa_bm_set_host_pool(self._h, int(num_host_blocks)))

    def _swap(self, fn, seq_id: int) -> np.ndarray:
        n_blocks = self.seq_info(seq_id)[1]
        pairs = np.empty((max(n_blocks, 1), 2), np.int32)
        n = ctypes.c_int32()
        _check(fn(self._h, int(seq_id), _ptr(pairs), n_blocks, ctypes.byref(n)))
        return pairs[: n.value]

    def swap_out(self, seq_id: int) -> np.ndarray:
        """pa_swap_out: (device block, host block) pairs [n][2]."""
        return self._swap(lib().pa_swap_out, seq_id)

    def swap_in(self, seq_id: int) -> np.ndarray:
        """pa_swap_in: (host block, device block) pairs [n][2]."""
        return self._swap(lib().pa_swap_in, seq_id)

    def is_swapped(self, seq_id: int) -> bool:
        v = ctypes.c_int32()
        _check(lib().pa_bm_swap_state(self._h, int(seq_id), ctypes.byref(v)))
        return bool(v.value)

    def host_stats(self) -> dict:
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        d, e = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_bm_host_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), ctypes.byref(d),
                                      ctypes.byref(e)))
        return dict(num_host_blocks=a.value, num_host_free=b.value, num_swapped=c.value, swap_outs=d.value,
                    swap_ins=e.value)

    def host_free_stack(self) -> list:
        cap = max(self.host_stats()["num_host_blocks"], 1)
        out = np.empty(cap, np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_bm_host_free_stack(self._h, _ptr(out), cap, ctypes.byref(n)))
        return out[: n.value].tolist()

    def usage(self, max_context_len: int) -> dict:
        """pa_bm_usage_get: KV usage, paged and naive waste, capacity."""
        u = _lib.PaBmUsage()
        _check(lib().pa_bm_usage_get(self._h, int(max_context_len), ctypes.byref(u)))
        return {f: getattr(u, f) for f, _ in _lib.PaBmUsage._fields_}

    def stats(self) -> dict:
        s = PaBmStats()
        _check(lib().pa_bm_stats(self._h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in PaBmStats._fields_ if f != "reserved"}

    def refcounts(self) -> list:
        out = np.empty(self.num_blocks, np.int32)
        _check(lib().pa_bm_refcounts(self._h, _ptr(out)))
        return out.tolist()

    def free_stack(self) -> list:
        out = np.empty(self.num_blocks, np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_bm_free_stack(self._h, _ptr(out), self.num_blocks, ctypes.byref(n)))
        return out[: n.value].tolist()


# ---------------------------------------------------------------------------
# device pool


_V_LAYOUTS = {"token": _lib.PA_LAYOUT_TOKEN_MAJOR, "dim": _lib.PA_LAYOUT_DIM_MAJOR}


@dataclasses.dataclass
class KVCache:
    """A paged KV pool in device memory: K and V tensors whose block b starts
    at element b * block_stride. K blocks are [block_size][num_kv_heads]
    [head_dim]; V blocks are that too (``v_layout="token"``) or
    [num_kv_heads][head_dim][block_size] (``v_layout="dim"``)."""

    k: torch.Tensor
    v: torch.Tensor
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    block_stride: int
    k_scale: float = 1.0
    v_scale: float = 1.0
    v_layout: str = "token"

    @classmethod
    def allocate(cls, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 kv_dtype: str = "bf16", device="cuda", layout: str = "split", k_scale: float = 1.0,
                 v_scale: float = 1.0, fill: Optional[float] = None, v_layout: str = "token") -> "KVCache":
        """``layout="split"``: separate K and V pools; ``"interleaved"``: one
        buffer of blocks each holding K then V."""
        dt = _NAMES[kv_dtype]
        be = block_size * num_kv_heads * head_dim
        pinned = str(device) == "pinned"  # a host pool the device addresses directly (swap target)
        if pinned:
            device = "cpu"
        if layout == "split":
            k = torch.empty(num_blocks * be, dtype=dt, device=device, pin_memory=pinned)
            v = torch.empty(num_blocks * be, dtype=dt, device=device, pin_memory=pinned)
            stride = be
        elif layout == "interleaved":
            buf = torch.empty(num_blocks * 2 * be, dtype=dt, device=device, pin_memory=pinned)
            k = buf
            v = buf[be:]
            stride = 2 * be
        else:
            raise ValueError(layout)
        if fill is not None:
            k.fill_(fill)
            v.fill_(fill)
        if v_layout not in _V_LAYOUTS:
            raise ValueError(v_layout)
        return cls(k, v, num_blocks, block_size, num_kv_heads, head_dim, stride, k_scale, v_scale, v_layout)

    @property
    def dtype_code(self) -> int:
        return _code(self.k)

    def desc(self) -> PaKvCache:
        if not ((self.k.is_cuda and self.v.is_cuda) or (self.k.is_pinned() and self.v.is_pinned())):
            raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT,
                                  "pool tensors must be on the device (or in pinned host memory for a host pool)")
        return PaKvCache(self.k.data_ptr(), self.v.data_ptr(), int(self.block_stride), int(self.num_blocks),
                         int(self.block_size), int(self.num_kv_heads), int(self.head_dim), self.dtype_code,
                         _V_LAYOUTS[self.v_layout], float(self.k_scale), float(self.v_scale))

    def block_view(self, which: str = "k") -> torch.Tensor:
        """Logical [num_blocks][block_size][num_kv_heads][head_dim] view of K
        or V (a strided view of the pool in either V layout)."""
        t = self.k if which == "k" else self.v
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if which == "v" and self.v_layout == "dim":
            strides = (self.block_stride, 1, self.head_dim * self.block_size, self.block_size)
        else:
            strides = (self.block_stride, self.num_kv_heads * self.head_dim, self.head_dim, 1)
        return t.as_strided(shape, strides)


# ---------------------------------------------------------------------------
# device operations


def reshape_and_cache(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                      stream=None) -> None:
    desc = cache.desc()
    T = int(slot_mapping.numel())
    _check(lib().pa_reshape_and_cache(ctypes.byref(desc), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                      _code(k_new), _dev(slot_mapping, "slot_mapping"), T, _stream(stream)))


def copy_blocks(cache: KVCache, pairs: torch.Tensor, stream=None) -> None:
    desc = cache.desc()
    n = int(pairs.numel() // 2)
    _check(lib().pa_copy_blocks(ctypes.byref(desc), _dev(pairs, "pairs") if n else None, n, _stream(stream)))


#: partition_size value selecting the balanced split (dim-major V pools)
BALANCED = _lib.PA_PARTITION_BALANCED


def decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                          partition_size: int) -> int:
    """Workspace bytes of pa_decode (for BALANCED: on the current device)."""
    return int(lib().pa_decode_workspace_size(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                              int(max_context_len), int(partition_size)))


def decode_shared_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                 max_context_len: int, partition_size: int) -> int:
    """Workspace bytes of pa_decode_shared (on the current device)."""
    return int(lib().pa_decode_shared_workspace_size(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                                     int(max_context_len), int(partition_size)))


def _deferred(fn, args, device: torch.device, out: torch.Tensor, keep):
    """A callable that issues fn(*args) on ``device`` and returns ``out``;
    it holds ``keep``, the objects args point into."""
    def launch() -> torch.Tensor:
        if device.index == torch.cuda.current_device():
            _check(fn(*args))
        else:
            with torch.cuda.device(device):
                _check(fn(*args))
        return out

    launch.keep = keep
    return launch


def prepare_decode(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                   max_context_len: int, scale: float, partition_size: int = 0, out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """decode with its arguments marshalled now and the launch deferred:
    returns a callable that issues pa_decode and returns ``out`` (e.g. to
    time the launch alone). The callable holds the tensors it points into;
    their shapes must not change before it runs."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:  # (a given workspace is sized by the library's own check)
        with torch.cuda.device(q.device):
            need = decode_workspace_size(B, Hq, cache.num_kv_heads, D, max_context_len, partition_size)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    desc = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(desc), _dev(out, "out"), _code(out), _dev(q, "q"), _code(q),
            _dev(block_tables, "block_tables"), int(block_tables.shape[1]), _dev(context_lens, "context_lens"),
            int(B), int(Hq), int(max_context_len), float(scale), int(partition_size), _dev(workspace, "workspace"),
            ws_bytes, _stream(stream))
    return _deferred(lib().pa_decode, args, q.device, out, (desc, workspace, cache, q, block_tables, context_lens))


def decode(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
           max_context_len: int, scale: float, partition_size: int = 0, out: Optional[torch.Tensor] = None,
           out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Paged decode attention; returns ``out`` [B][Hq][D]. A workspace is
    allocated with torch when the split needs one and none is given."""
    return prepare_decode(cache, q, block_tables, context_lens, max_context_len, scale, partition_size, out=out,
                          out_dtype=out_dtype, workspace=workspace, stream=stream)()


def decode_noalloc(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                   max_context_len: int, scale: float, partition_size: int = 0, out: Optional[torch.Tensor] = None,
                   out_dtype: Optional[torch.dtype] = None, stream=None) -> torch.Tensor:
    """pa_decode_noalloc: decode with the library's static per-GPU scratch
    instead of a workspace (the library allocates nothing). Calls that
    overlap on one GPU race on that scratch. Returns ``out``."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    desc = cache.desc()
    args = (ctypes.byref(desc), _dev(out, "out"), _code(out), _dev(q, "q"), _code(q),
            _dev(block_tables, "block_tables"), int(block_tables.shape[1]), _dev(context_lens, "context_lens"),
            int(B), int(Hq), int(max_context_len), float(scale), int(partition_size), _stream(stream))
    return _deferred(lib().pa_decode_noalloc, args, q.device, out, (desc, cache, q, block_tables, context_lens))()


def prepare_decode_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                          q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                          max_context_len: int, scale: float, out: Optional[torch.Tensor] = None,
                          out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None):
    """decode_append with its arguments marshalled now and the launch
    deferred: returns a callable that issues pa_decode_append and returns
    ``out`` (e.g. to time the launch alone). The callable holds the
    tensors it points into; their shapes must not change before it runs."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if slot_mapping.dtype != torch.int64:
        raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT, "slot_mapping must be int64")
    if workspace is None:  # (a given workspace is sized by the library's own check)
        with torch.cuda.device(q.device):
            need = decode_workspace_size(B, Hq, cache.num_kv_heads, D, max_context_len, BALANCED)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    desc = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(desc), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _code(k_new),
            _dev(slot_mapping, "slot_mapping"), _dev(out, "out"), _code(out), _dev(q, "q"), _code(q),
            _dev(block_tables, "block_tables"), int(block_tables.shape[1]), _dev(context_lens, "context_lens"),
            int(B), int(Hq), int(max_context_len), float(scale), _dev(workspace, "workspace"), ws_bytes,
            _stream(stream))
    return _deferred(lib().pa_decode_append, args, q.device, out,
                     (desc, workspace, cache, k_new, v_new, slot_mapping, q, block_tables, context_lens))


def decode_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                  q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                  scale: float, out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode_append: write each sequence's newest token (k_new / v_new
    [B][Hkv][D] at slot_mapping[s], the slot of token context_lens[s] - 1)
    and run the balanced decode that includes it, in one launch. Returns
    ``out`` [B][Hq][D]."""
    return prepare_decode_append(cache, k_new, v_new, slot_mapping, q, block_tables, context_lens, max_context_len,
                                 scale, out=out, out_dtype=out_dtype, workspace=workspace, stream=stream)()


def prepare_decode_shared(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                          max_context_len: int, scale: float, partition_size: int, group_offsets: torch.Tensor,
                          group_members: torch.Tensor, shared_len: torch.Tensor, num_groups: int,
                          max_group_size: int, max_shared_len: int, min_shared_len: int = 0,
                          out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """decode_shared with its arguments marshalled now and the launch
    deferred (see prepare_decode)."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:  # (a given workspace is sized by the library's own check)
        with torch.cuda.device(q.device):
            need = decode_shared_workspace_size(B, Hq, cache.num_kv_heads, D, max_context_len, partition_size)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    for name, t in (("group_offsets", group_offsets), ("group_members", group_members), ("shared_len", shared_len)):
        if t.dtype != torch.int32:
            raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT, f"{name} must be int32")
    desc = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(desc), _dev(out, "out"), _code(out), _dev(q, "q"), _code(q),
            _dev(block_tables, "block_tables"), int(block_tables.shape[1]), _dev(context_lens, "context_lens"),
            int(B), int(Hq), int(max_context_len), float(scale), int(partition_size),
            _dev(group_offsets, "group_offsets"), _dev(group_members, "group_members"), _dev(shared_len, "shared_len"),
            int(num_groups), int(max_group_size), int(max_shared_len), int(min_shared_len),
            _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    return _deferred(lib().pa_decode_shared, args, q.device, out,
                     (desc, workspace, cache, q, block_tables, context_lens, group_offsets, group_members,
                      shared_len))


def decode_shared(cache: KVCache, q: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                  max_context_len: int, scale: float, partition_size: int, group_offsets: torch.Tensor,
                  group_members: torch.Tensor, shared_len: torch.Tensor, num_groups: int, max_group_size: int,
                  max_shared_len: int, min_shared_len: int = 0, out: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """pa_decode_shared: decode with each group's shared prefix read once
    for all its rows (group arrays on the device, int32). Returns ``out``."""
    return prepare_decode_shared(cache, q, block_tables, context_lens, max_context_len, scale, partition_size,
                                 group_offsets, group_members, shared_len, num_groups, max_group_size,
                                 max_shared_len, min_shared_len, out=out, out_dtype=out_dtype, workspace=workspace,
                                 stream=stream)()


def ref_stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int, stream=None) -> None:
    """pa_ref_stream_read (measurement aid): read all of the device tensor
    ``buf`` once with a plain streaming kernel of ``grid`` workgroups;
    ``sink`` = a device int32/uint32 tensor of grid * 256 elements."""
    if sink.numel() < grid * 256 or sink.element_size() != 4:
        raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT, "sink needs grid * 256 32-bit elements")
    _check(lib().pa_ref_stream_read(_dev(buf, "buf"), int(buf.numel() * buf.element_size()), _dev(sink, "sink"),
                                    int(grid), _stream(stream)))


def copy_blocks_between(dst: KVCache, src: KVCache, pairs, stream=None) -> None:
    """pa_copy_blocks_between: dst block pairs[i][1] <- src block
    pairs[i][0] (K and V). ``pairs`` int32 [N][2], a device tensor or host
    data (then uploaded first, synchronously)."""
    if not isinstance(pairs, torch.Tensor):
        pairs = torch.as_tensor(np.asarray(pairs, np.int32).reshape(-1, 2))
    if pairs.numel() == 0:
        return
    if not pairs.is_cuda:
        dev = dst.k.device if dst.k.is_cuda else src.k.device
        pairs = pairs.to(torch.int32).contiguous().to(dev)
    if pairs.dtype != torch.int32:
        raise InvalidArgument(_lib.PA_ERR_INVALID_ARGUMENT, "pairs must be int32")
    d, s_ = dst.desc(), src.desc()
    _check(lib().pa_copy_blocks_between(ctypes.byref(d), ctypes.byref(s_), _dev(pairs, "pairs"), int(pairs.shape[0]),
                                        _stream(stream)))
