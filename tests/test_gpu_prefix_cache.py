"""Prefix caching on the GPU: a later request whose prompt starts like an
earlier (finished) one reuses the earlier request's full blocks and writes
K/V only for the rest; its decode output must match the oracle computed on
its whole prompt.

K/V of position t are a deterministic function of the token prefix
tokens[0..t] (as in a real model), so a reused block holds exactly the rows
the new request would have written."""
import hashlib

import numpy as np
import pytest
import torch

import paged_kv_cache_49_amd as pa
from oracle import attention as oatt
from tests import helpers as H
from tests.gpu_util import poison_fill, say

pytestmark = pytest.mark.gpu

HKV, D, G, BS = 4, 128, 4, 16


def _kv(tokens):
    """K and V rows [len][HKV][D] (bf16), each row a function of its prefix."""
    ks, vs = [], []
    h = hashlib.sha256()
    for t in tokens:
        h.update(int(t).to_bytes(4, "little"))
        rng = np.random.default_rng(int.from_bytes(h.digest()[:8], "little"))
        ks.append(rng.standard_normal((HKV, D)).astype(np.float32))
        vs.append(rng.standard_normal((HKV, D)).astype(np.float32))
    return torch.from_numpy(np.stack(ks)).bfloat16(), torch.from_numpy(np.stack(vs)).bfloat16()


def _decode(cache, bm, seqs, q, mb):
    t, l = bm.pack(seqs, mb, -1)
    out = pa.decode(cache, q.cuda(), torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(), int(l.max()),
                    float(np.float32(1 / np.sqrt(D))), pa.BALANCED, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def test_prompt_blocks_reused_across_requests(gpu):
    say("prefix cache reuse")
    rng = np.random.default_rng(5)
    nb = 400
    bm = pa.BlockManager(nb, BS, rng.permutation(nb).astype(np.int32))
    bm.set_prefix_cache(True)
    cache = pa.KVCache.allocate(nb, BS, HKV, D, "bf16", fill=poison_fill("bf16"), v_layout="dim")
    scale = float(np.float32(1 / np.sqrt(D)))
    mb = 80

    def submit(seq, tokens):
        slots, cached = bm.alloc_prompt(seq, tokens)
        k, v = _kv(tokens)
        if cached < len(tokens):  # only the rows the cache does not hold
            pa.reshape_and_cache(cache, k[cached:].cuda(), v[cached:].cuda(),
                                 torch.from_numpy(slots[cached:]).cuda())
        return cached, k, v

    a = rng.integers(0, 1000, size=700).tolist()
    cached, ka, va = submit(1, a)
    assert cached == 0
    q = torch.from_numpy(rng.standard_normal((3, G * HKV, D)).astype(np.float32)).bfloat16()
    got_a = _decode(cache, bm, [1], q[:1], mb)
    ref_a = oatt.decode_contiguous(oatt.to_f64(q[0]), oatt.to_f64(ka), oatt.to_f64(va), scale, HKV)
    H.assert_close(got_a[0], ref_a, what="request A")
    bm.free(1)

    b = a[:500] + rng.integers(0, 1000, size=300).tolist()
    cached_b, kb, vb = submit(2, b)
    assert cached_b == 496  # the 31 full blocks of the common 500 tokens
    c = a[:200] + rng.integers(0, 1000, size=50).tolist()
    cached_c, kc, vc = submit(3, c)
    assert cached_c == 192
    got = _decode(cache, bm, [2, 3], q[1:], mb)
    for row, (k, v) in enumerate([(kb, vb), (kc, vc)]):
        ref = oatt.decode_contiguous(oatt.to_f64(q[1 + row]), oatt.to_f64(k), oatt.to_f64(v), scale, HKV)
        H.assert_close(got[row], ref, what=f"request {'BC'[row]}")
    st = bm.prefix_cache_stats()
    assert st["hits"] == 31 + 12 and st["misses"] == 43 + 19 + 3
