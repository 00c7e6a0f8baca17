"""pa_decode_noalloc (decode with the library's static per-GPU scratch, for
callers that cannot allocate) against pa_decode with a workspace.

Two calls in a row through the C ABI, the second with a smaller batch (the
scratch then holds the first call's leftovers): each output must equal
pa_decode's on the same inputs bit for bit (the same kernels and grid; only
where the partial results live differs) and meet the oracle tolerance.
A partitioned call whose workspace would exceed the scratch is refused
before any launch.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_49_amd as pa
import synth
from tests import helpers as H
from tests.gpu_util import device_setup, say

pytestmark = pytest.mark.gpu


def _both(wl, partition_size, v_layout):
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout=v_layout)
    q = wl.q().cuda()
    say(f"noalloc {wl.name} B={wl.batch} kv={wl.kv_dtype} G={wl.group} part={partition_size} V={v_layout}")
    want = pa.decode(cache, q, tables, lens, max_ctx, wl.scale, partition_size, out_dtype=torch.float32)
    got = pa.decode_noalloc(cache, q, tables, lens, max_ctx, wl.scale, partition_size, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return got.cpu(), want.cpu()


CASES = [
    # (kv, D, bs, G, partition_size, v_layout)
    ("bf16", 128, 16, 4, pa.BALANCED, "token"),
    ("bf16", 128, 16, 8, pa.BALANCED, "dim"),
    ("fp8", 128, 16, 8, pa.BALANCED, "token"),
    ("f16", 64, 8, 2, 256, "dim"),
    ("bf16", 128, 16, 4, 512, "token"),
]


@pytest.mark.parametrize("kv,D,bs,G,ps,v_layout", CASES, ids=lambda c: str(c))
def test_noalloc_matches_pa_decode_twice(gpu, kv, D, bs, G, ps, v_layout):
    hkv = 8 if G <= 4 else 4
    rng = np.random.default_rng(5150 + D + bs + G + max(ps, 0))
    first = rng.integers(1, 3000, size=24)
    first[:3] = [1, 16, 2049]
    second = rng.integers(1, 900, size=5)
    for i, lengths in enumerate((first, second)):
        wl = synth.random_case(5150 + 10 * i + G, lengths, G * hkv, hkv, D, bs, kv)
        got, want = _both(wl, ps, v_layout)
        assert torch.equal(got, want), f"call {i}: pa_decode_noalloc differs from pa_decode"
        ma, rl = H.assert_close(got.double().numpy(), H.oracle_contiguous(wl), what=f"call {i}")
        say(f"   call {i}: bit-identical to pa_decode; max-abs {ma:.2e} rel-L2 {rl:.2e}")


def test_noalloc_refuses_a_partition_workspace_beyond_the_scratch(gpu):
    """64 seqs x 32 heads x 4096 partitions of 16 tokens needs ~4.3 GB of
    partial results: refused before any launch."""
    B, Hq, hkv, D, bs = 64, 32, 8, 128, 16
    max_blocks = 4096
    cache = pa.KVCache.allocate(8, bs, hkv, D, "bf16")
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(B, max_blocks, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(pa.InvalidArgument, match="scratch"):
        pa.decode_noalloc(cache, q, tables, lens, max_blocks * bs, 0.088, 16)
