"""Cache write and block copy — oracle models on the pools' storage bits.

* Write ([course] §2 primer: decoding adds one token's K/V per step;
  [course] §2 "The insight": blocks of 16 tokens' K and V in a pool; [note]
  最小模型: growing a request only needs one more block): token i's K and V
  rows go to physical block ``slot // bs``, in-block row ``slot % bs``; a
  negative slot means "skip this token".
* Copy ([course] §2 "The bonus: block sharing (copy-on-write)": when
  generations diverge only the differing block is copied; [note] section
  prefix sharing 的边界: copy-on-write happens only when a branch writes):
  for every (src, dst) pair the whole K block and the whole V block of
  ``src`` overwrite those of ``dst``.

Pools are numpy arrays of storage bits, [num_blocks][bs][Hkv][D]:
uint16 for f16 / bf16 (the bits are copied unchanged), uint8 for fp8 (the
E4M3 code of the quantised value).
"""
from __future__ import annotations

import numpy as np
import torch

from . import fp8 as _fp8

_BITS = {"f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


def storage_bits(x: torch.Tensor, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Bits a source tensor occupies in a ``kv_dtype`` cache."""
    if kv_dtype == "fp8":
        return _fp8.quantize(x.detach().to("cpu", torch.float32).numpy(), scale)
    want = {"f16": torch.float16, "bf16": torch.bfloat16}[kv_dtype]
    if x.dtype != want:
        raise ValueError(f"a {kv_dtype} cache takes {kv_dtype} sources, got {x.dtype}")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def empty_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
               kv_dtype: str, fill: int = 0) -> np.ndarray:
    return np.full((num_blocks, block_size, num_kv_heads, head_dim), fill, dtype=_BITS[kv_dtype])


def write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: torch.Tensor, v_new: torch.Tensor,
          slots, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """In place: pool[slot // bs][slot % bs] = enc(row) for every slot >= 0.

    k_new, v_new [T][Hkv][D]; slots [T] (int64)."""
    bs = k_pool.shape[1]
    kb = storage_bits(k_new, kv_dtype, k_scale)
    vb = storage_bits(v_new, kv_dtype, v_scale)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    blk, off = np.divmod(slots[keep], bs)
    k_pool[blk, off] = kb[keep]
    v_pool[blk, off] = vb[keep]


def copy(k_pool: np.ndarray, v_pool: np.ndarray, pairs) -> None:
    """In place: block dst of each pool becomes a copy of block src."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
