"""Pins for the cache write and block copy models (CPU only): a write
followed by a read through the block table returns the source rows in token
order; negative slots are skipped; a copy duplicates exactly one block; an
fp8 write stores the E4M3 codes of the scaled values."""
import numpy as np
import torch

import synth
from oracle import allocator as A
from oracle import attention as oatt
from oracle import cache_ops as C
from oracle import fp8
from tests import helpers as H


def test_write_then_gather_is_identity():
    wl = synth.random_case(41, [1, 16, 17, 50], 4, 2, 8, 16, "bf16")
    alloc, kp, vp, tables, lens = H.oracle_setup(wl)
    for s in range(wl.batch):
        k, v = wl.kv(s)
        got_k = oatt.gather_sequence(kp, tables[s], int(lens[s]), wl.block_size)
        got_v = oatt.gather_sequence(vp, tables[s], int(lens[s]), wl.block_size)
        assert np.array_equal(got_k, C.storage_bits(k, "bf16"))
        assert np.array_equal(got_v, C.storage_bits(v, "bf16"))


def test_negative_slots_are_skipped():
    kp = C.empty_pool(4, 2, 1, 4, "f16", fill=7)
    vp = C.empty_pool(4, 2, 1, 4, "f16", fill=7)
    rows = torch.randn(3, 1, 4).half()
    C.write(kp, vp, rows, rows, [5, -1, 0], "f16")
    bits = C.storage_bits(rows, "f16")
    assert np.array_equal(kp[2, 1], bits[0]) and np.array_equal(kp[0, 0], bits[2])
    untouched = np.ones(kp.shape[:2], bool)
    untouched[2, 1] = untouched[0, 0] = False
    assert (kp[untouched] == 7).all() and (vp[untouched] == 7).all()


def test_copy_duplicates_whole_blocks_only():
    rng = np.random.default_rng(0)
    kp = rng.integers(0, 2 ** 16, size=(6, 4, 2, 8)).astype(np.uint16)
    vp = rng.integers(0, 2 ** 16, size=(6, 4, 2, 8)).astype(np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    C.copy(kp, vp, [(1, 4), (5, 0)])
    assert np.array_equal(kp[4], k0[1]) and np.array_equal(vp[4], v0[1])
    assert np.array_equal(kp[0], k0[5]) and np.array_equal(vp[0], v0[5])
    for b in (1, 2, 3, 5):
        assert np.array_equal(kp[b], k0[b]) and np.array_equal(vp[b], v0[b])


def test_fp8_write_stores_scaled_codes():
    rows = torch.randn(5, 2, 16).bfloat16()
    kp = C.empty_pool(3, 4, 2, 16, "fp8")
    vp = C.empty_pool(3, 4, 2, 16, "fp8")
    ks, vs = 0.01, 0.02
    C.write(kp, vp, rows, rows * 2, [0, 1, 2, 3, 4], "fp8", ks, vs)
    want_k = fp8.quantize(rows.float().numpy(), ks)
    want_v = fp8.quantize((rows * 2).float().numpy(), vs)
    assert np.array_equal(kp.reshape(12, 2, 16)[:5], want_k)
    assert np.array_equal(vp.reshape(12, 2, 16)[:5], want_v)
    # dequantised values are within half an E4M3 step of the source
    back = fp8.dequantize(kp.reshape(12, 2, 16)[:5], ks)
    assert np.all(np.abs(back - rows.double().numpy()) <= np.abs(rows.double().numpy()) / 16 + ks * 2 ** -9)


def test_copy_on_write_then_write_isolates_the_writer():
    """A fork shares a partial tail; after the writer's copy and write, the
    other holder reads exactly what it read before."""
    wl = synth.random_case(42, [21], 2, 1, 8, 8, "f16", headroom=3.0)
    alloc, kp, vp, tables, lens = H.oracle_setup(wl)
    alloc.fork(0, 1)
    before = oatt.gather_sequence(kp, alloc.table(1), alloc.length(1), 8).copy()
    slots, cows = alloc.alloc(0, 1)
    assert len(cows) == 1
    C.copy(kp, vp, cows)
    new = torch.randn(1, 1, 8).half()
    C.write(kp, vp, new, new, slots, "f16")
    assert np.array_equal(oatt.gather_sequence(kp, alloc.table(1), alloc.length(1), 8), before)
    got0 = oatt.gather_sequence(kp, alloc.table(0), alloc.length(0), 8)
    assert np.array_equal(got0[:21], before) and np.array_equal(got0[21], C.storage_bits(new, "f16")[0])
