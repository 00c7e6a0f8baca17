"""Single-query (decode) attention through a block table — fp64 oracle.

What the paged path computes, as the pages state it:

* [course] §2 "The insight: page the KV cache like OS virtual memory": one
  pool holds the KV cache as blocks of a fixed size; a per-sequence table
  names the physical block behind each logical block, and attention looks
  every key and value up through that table while it computes the scores.
  The block layout the section prints is K[BLOCK][HEADS][HEAD_DIM]
  (token-major inside a block).
* [note] section 最小模型 ("minimal model"): the kernel reads the block table
  and visits the (possibly scattered) physical blocks in logical token order.
* [note] section 它为什么有效 ("why it works"): paging is not an algorithm that
  reduces attention math — so the result is ordinary attention over the
  sequence's tokens in logical order.

Readings where the pages are silent (each listed in the design notes):
* the score is softmax(scale * q . k) with the caller's fp32 ``scale``,
  taken here as float64(scale);
* query head h reads KV head h // G, G = Hq / Hkv (contiguous groups);
* the query attends to every token in [0, L), L = context length;
* L = 0 gives an all-zero output row;
* fp8 K/V enter as decode(code) * scale (the dequantised values).
"""
from __future__ import annotations

import numpy as np
import torch

from . import fp8 as _fp8


def to_f64(x) -> np.ndarray:
    """Storage values -> fp64 (exact for fp16 / bf16 / fp32)."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def gather_sequence(pool: np.ndarray, table_row, length: int, block_size: int) -> np.ndarray:
    """Contiguous rows [L][...] of one sequence, read through its block table.

    Token t of the sequence lives in physical block ``table_row[t // bs]`` at
    in-block row ``t % bs`` ([course] §2 "The insight"; [note] 最小模型).
    ``pool`` is [num_blocks][bs][...]. Table entries past ceil(L/bs) are
    never read."""
    t = np.arange(length)
    n_used = -(-length // block_size)
    row = np.asarray(table_row[:n_used], dtype=np.int64)
    if n_used and (row.min() < 0 or row.max() >= pool.shape[0]):
        raise ValueError("block table entry outside the pool")
    return pool[row[t // block_size], t % block_size]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Naive softmax attention of one query set over contiguous K/V, fp64.

    q [G][D], k [L][D], v [L][D] -> [G][D]:
        z_t = scale * q . k_t,  w_t = exp(z_t - max z),  out = sum w_t v_t / sum w_t
    (subtracting max z changes nothing mathematically; it keeps exp finite).
    L = 0 -> zeros."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    z = np.float64(scale) * (q @ np.asarray(k, np.float64).T)  # [G][L]
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return (w @ np.asarray(v, np.float64)) / w.sum(axis=1, keepdims=True)


def decode_contiguous(q, k_seq, v_seq, scale: float, num_kv_heads: int) -> np.ndarray:
    """One sequence's decode output from its K/V in token order.

    q [Hq][D]; k_seq, v_seq [L][Hkv][D] (already fp64 values) -> [Hq][D].
    Query head h uses KV head h // G."""
    q = to_f64(q)
    hq = q.shape[0]
    g = hq // num_kv_heads
    out = np.empty_like(q)
    for kvh in range(num_kv_heads):
        heads = slice(kvh * g, (kvh + 1) * g)
        out[heads] = attend(q[heads], k_seq[:, kvh, :], v_seq[:, kvh, :], scale)
    return out


def pool_values(pool_bits: np.ndarray, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """fp64 values of a pool given as storage bits (uint16 f16/bf16, uint8 fp8)."""
    if kv_dtype == "fp8":
        return _fp8.dequantize(pool_bits, scale)
    if kv_dtype == "f16":
        return pool_bits.view(np.float16).astype(np.float64)
    if kv_dtype == "bf16":
        as32 = pool_bits.astype(np.uint32) << 16
        return as32.view(np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


def paged_decode(q, k_pool_bits, v_pool_bits, block_tables, context_lens, scale: float,
                 block_size: int, kv_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs=None) -> np.ndarray:
    """Decode attention for a batch through block tables, fp64.

    q [B][Hq][D]; pools [num_blocks][bs][Hkv][D] as storage bits;
    block_tables [B][max_blocks]; context_lens [B]. Returns [B][Hq][D]
    (rows not in ``seqs`` are left zero). Each sequence is rebuilt
    contiguous from the table and then attended naively."""
    q = to_f64(q)
    b, hq, d = q.shape
    hkv = k_pool_bits.shape[2]
    out = np.zeros((b, hq, d), dtype=np.float64)
    for s in (range(b) if seqs is None else seqs):
        length = int(context_lens[s])
        kb = gather_sequence(k_pool_bits, block_tables[s], length, block_size)
        vb = gather_sequence(v_pool_bits, block_tables[s], length, block_size)
        kf = pool_values(kb, kv_dtype, k_scale)
        vf = pool_values(vb, kv_dtype, v_scale)
        out[s] = decode_contiguous(q[s], kf, vf, scale, hkv)
    return out


def source_values(x, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """fp64 values a K/V source tensor has once stored in a ``kv_dtype`` cache.

    16-bit caches store the source bits unchanged; an fp8 cache stores
    quantize(x, scale) and yields decode(code) * scale."""
    if kv_dtype == "fp8":
        xs = x.detach().to("cpu", torch.float32).numpy()
        return _fp8.dequantize(_fp8.quantize(xs, scale), scale)
    return to_f64(x)
