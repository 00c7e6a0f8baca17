"""Test-side glue: builds the oracle's own view of a workload (allocator model
-> slot writes -> pool -> paged decode) using only ``oracle`` and ``synth``,
and small comparison utilities shared by the tests."""
from __future__ import annotations

import numpy as np
import torch

from oracle import allocator as oalloc
from oracle import attention as oatt
from oracle import cache_ops as ocache

# spec tolerance for fp16 / bf16 attention outputs (fp8: same limits,
# against the oracle fed the dequantised values)
MAX_ABS_TOL = 1e-2
REL_L2_TOL = 2e-3


def max_blocks_for(lengths, block_size, extra=0):
    return max(1, max((oalloc.blocks_for(int(n), block_size) for n in lengths), default=1) + extra)


def oracle_setup(wl, max_blocks=None, pad=-1, fill=0):
    """Allocate every sequence of ``wl`` in the allocator model and write its
    K/V through the slot model. Returns (alloc, kpool, vpool, tables, lens)."""
    alloc = oalloc.BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
    kpool = ocache.empty_pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, fill)
    vpool = ocache.empty_pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype, fill)
    ks, vs = wl.kv_scales()
    for s in range(wl.batch):
        slots, cows = alloc.alloc(s, int(wl.lengths[s]))
        assert not cows
        k, v = wl.kv(s)
        ocache.write(kpool, vpool, k, v, slots, wl.kv_dtype, ks, vs)
    if max_blocks is None:
        max_blocks = max_blocks_for(wl.lengths, wl.block_size)
    tables, lens = alloc.pack(list(range(wl.batch)), max_blocks, pad)
    return alloc, kpool, vpool, np.asarray(tables, np.int32), np.asarray(lens, np.int32)


def oracle_paged(wl, **kw):
    alloc, kpool, vpool, tables, lens = oracle_setup(wl, **kw)
    ks, vs = wl.kv_scales()
    return oatt.paged_decode(wl.q(), kpool, vpool, tables, lens, wl.scale, wl.block_size,
                             wl.kv_dtype, ks, vs)


def oracle_contiguous(wl, seqs=None):
    """Expected output rows from the sequences' token-ordered K/V (no table)."""
    q = oatt.to_f64(wl.q())
    ks, vs = wl.kv_scales()
    out = np.zeros_like(q)
    for s in (range(wl.batch) if seqs is None else seqs):
        k, v = wl.kv(s)
        out[s] = oatt.decode_contiguous(q[s], oatt.source_values(k, wl.kv_dtype, ks),
                                        oatt.source_values(v, wl.kv_dtype, vs), wl.scale,
                                        wl.num_kv_heads)
    return out


def errors(got, ref):
    """(max-abs error, relative L2 error) in fp64 over the whole array."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    denom = np.linalg.norm(ref.ravel())
    return float(np.abs(diff).max(initial=0.0)), float(np.linalg.norm(diff.ravel()) / max(denom, 1e-300))


def assert_close(got, ref, max_abs=MAX_ABS_TOL, rel_l2=REL_L2_TOL, what=""):
    ma, rl = errors(got, ref)
    assert np.isfinite(np.asarray(got)).all(), f"{what}: non-finite output"
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max-abs {ma:.3e} (<= {max_abs}), rel-L2 {rl:.3e} (<= {rel_l2})"
    return ma, rl


def sdpa_reference(q, k_seq, v_seq, scale):
    """torch's scaled_dot_product_attention (fp64, CPU, grouped KV heads) for
    one sequence: q [Hq][D], k/v [L][Hkv][D] -> [Hq][D]. An independent
    library routine used only to pin the oracle."""
    qt = torch.as_tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.as_tensor(np.asarray(k_seq, np.float64)).permute(1, 0, 2)[None]
    vt = torch.as_tensor(np.asarray(v_seq, np.float64)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale),
                                                         enable_gqa=True)
    return o[0, :, 0, :].numpy()
