"""The balanced decode split (partition_size = pa.BALANCED, dim-major V) on
the GPU against the fp64 oracle.

The split divides the batch's tiles (16 tokens; 32 for fp8 pools) evenly
over the resident
workgroups and merges sequences cut between them. PA_SK_WGS caps the grid,
so small inputs still reach every case of the split: one workgroup walking
many sequences and many unit batches (cap 1), sequences cut between a few
workgroups (small caps), and workgroups with no units at all (more
workgroups than tiles). Tolerance as in test_gpu_decode.py.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_49_amd as pa
import synth
from tests import helpers as H
from paged_kv_cache_49_amd.runner import workspace_for
from tests.gpu_util import device_setup, run_decode, say

pytestmark = pytest.mark.gpu

BAL = pa.BALANCED
LENGTHS = [1, 15, 16, 17, 100, 511, 512, 513, 1100, 2049]


@pytest.fixture
def wgs(monkeypatch):
    """set_wgs(n): cap the balanced grid at n workgroups (None: no cap)."""
    def set_wgs(n):
        if n is None:
            monkeypatch.delenv("PA_SK_WGS", raising=False)
        else:
            monkeypatch.setenv("PA_SK_WGS", str(n))
    return set_wgs


def _check(wl, what="", v_layout="dim", layout="split"):
    say(f"balanced {wl.name} kv={wl.kv_dtype} D={wl.head_dim} bs={wl.block_size} Hkv={wl.num_kv_heads} "
        f"G={wl.group} V {v_layout} {layout} {what}")
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout=v_layout, layout=layout)
    got = run_decode(wl, cache, tables, lens, max_ctx, BAL)
    ma, rl = H.assert_close(got, H.oracle_contiguous(wl), what=f"{wl.name} {what}")
    say(f"   max-abs {ma:.2e}  rel-L2 {rl:.2e}")
    return got


CASES = [
    ("bf16", 128, 16, 4),
    ("f16", 64, 16, 1),
    ("bf16", 128, 8, 8),
    ("bf16", 64, 32, 2),
    ("f16", 128, 32, 4),
    ("fp8", 128, 16, 8),
    ("fp8", 64, 8, 4),
    ("fp8", 128, 32, 1),
]


@pytest.mark.parametrize("cap", [None, 1, 7])
@pytest.mark.parametrize("hkv", [2, 8])
@pytest.mark.parametrize("kv,D,bs,G", CASES, ids=lambda c: str(c))
def test_parity_sweep(gpu, wgs, kv, D, bs, G, hkv, cap):
    wgs(cap)
    wl = synth.random_case(2000 + D + bs + G + hkv, LENGTHS, G * hkv, hkv, D, bs, kv)
    _check(wl, f"cap={cap}")


TOKEN_CASES = [
    ("bf16", 128, 16, 4, "split"),
    ("f16", 64, 16, 1, "interleaved"),
    ("bf16", 128, 8, 8, "split"),
    ("bf16", 64, 32, 2, "interleaved"),
    ("f16", 128, 32, 4, "split"),
]


@pytest.mark.parametrize("cap", [None, 1, 7])
@pytest.mark.parametrize("hkv", [2, 8])
@pytest.mark.parametrize("kv,D,bs,G,layout", TOKEN_CASES, ids=lambda c: str(c))
def test_token_major_v(gpu, wgs, kv, D, bs, G, layout, hkv, cap):
    """The page's token-major V blocks (split pools and the interleaved
    K-then-V block), each unit's V rows transposed through LDS."""
    wgs(cap)
    wl = synth.random_case(2800 + D + bs + G + hkv, LENGTHS, G * hkv, hkv, D, bs, kv)
    _check(wl, f"cap={cap}", v_layout="token", layout=layout)


def test_token_major_v_matches_dim_major(gpu):
    """The same logical data in both V layouts gives the same output up to
    fp32 rounding order (the arithmetic is the same; only the operand path
    differs)."""
    wl = synth.random_case(2900, [300, 1500, 17, 4000], 32, 8, 128, 16, "bf16")
    a = _check(wl, "dim", v_layout="dim")
    b = _check(wl, "token", v_layout="token")
    H.assert_close(b, a, what="token-major vs dim-major")


FP8_LENGTHS = [1, 7, 8, 9, 31, 32, 33, 63, 64, 65, 777, 1601]


@pytest.mark.parametrize("v_layout", ["dim", "token"])
@pytest.mark.parametrize("cap", [None, 1, 5])
@pytest.mark.parametrize("D,bs,G", [(128, 8, 8), (128, 16, 4), (64, 32, 2), (128, 32, 8), (64, 8, 1)])
def test_fp8_32_token_units(gpu, wgs, D, bs, G, cap, v_layout):
    """fp8 pools take 32-token units (two 16-row QK tiles and one 32-deep PV
    step per unit): lengths on both sides of multiples of 8, 16 and 32, and
    units that span 4, 2 or 1 blocks; dim-major V (8-byte runs from the
    stage) and token-major V (rows widened to bf16 in the stage, two
    transposing reads per 16-dim tile)."""
    wgs(cap)
    wl = synth.random_case(2600 + D + bs + G, FP8_LENGTHS, 2 * G, 2, D, bs, "fp8")
    _check(wl, f"cap={cap}", v_layout=v_layout)


@pytest.mark.parametrize("v_layout", ["dim", "token"])
@pytest.mark.parametrize("hkv", [1, 3, 6])
def test_fp8_head_groups(gpu, wgs, hkv, v_layout):
    """32-token fp8 units with one wave (Hkv 1) and workgroups of a power of
    two below Hkv (3 -> 1, 6 -> 2 heads), cut between a few workgroups."""
    wgs(5)
    wl = synth.random_case(2700 + hkv, [33, 700, 1, 1500, 95], 4 * hkv, hkv, 128, 16, "fp8")
    _check(wl, "cap=5", v_layout=v_layout)


@pytest.mark.parametrize("hkv", [1, 3, 6, 16, 24])
@pytest.mark.parametrize("cap", [None, 5])
def test_head_groups(gpu, wgs, hkv, cap):
    """A workgroup serves the largest divisor of Hkv up to 8 KV heads: one
    wave (Hkv 1), odd widths (3, 6) and several head groups (16, 24)."""
    wgs(cap)
    wl = synth.random_case(2100 + hkv, [40, 700, 3, 1500], 2 * hkv, hkv, 128, 16, "bf16")
    _check(wl, f"cap={cap}")


@pytest.mark.parametrize("cap", [None, 1, 2, 3])
def test_empty_and_short_sequences(gpu, wgs, cap):
    """Zero-length sequences give zeros; with the default grid most
    workgroups get no units at all."""
    wgs(cap)
    wl = synth.random_case(2200, [0, 1, 0, 17, 0, 33], 16, 2, 128, 16, "bf16")
    got = _check(wl, f"cap={cap}")
    for s in (0, 2, 4):
        assert np.array_equal(got[s], np.zeros_like(got[s]))


def test_all_sequences_empty(gpu):
    wl = synth.random_case(2201, [0, 0, 0], 16, 2, 128, 16, "bf16", min_blocks=4)
    got = _check(wl)
    assert np.array_equal(got, np.zeros_like(got))


def test_one_long_sequence_over_every_workgroup(gpu):
    """One 20000-token sequence: every workgroup holds a piece of it, and
    the merge combines hundreds of pieces."""
    wl = synth.random_case(2300, [20000], 8, 2, 128, 16, "bf16")
    _check(wl)


@pytest.mark.parametrize("cap", [1, 2, 3])
def test_many_unit_batches_per_workgroup(gpu, wgs, cap):
    """With 1 to 3 workgroups each walks hundreds of units: many 63-unit
    batches, many sequences, pieces at both ends of every range."""
    wgs(cap)
    wl = synth.random_case(2400, [3000, 1500, 700, 1, 16, 250, 4100], 8, 2, 128, 16, "bf16")
    _check(wl, f"cap={cap}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("cap", [None, 3])
def test_16bit_outputs(gpu, wgs, out_dtype, cap):
    wgs(cap)
    wl = synth.random_case(2500, [5, 300, 900, 2000], 16, 2, 128, 16, "bf16")
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout="dim")
    got = run_decode(wl, cache, tables, lens, max_ctx, BAL, out_dtype)
    H.assert_close(got, H.oracle_contiguous(wl), what=f"{out_dtype} cap={cap}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("cap", [None, 3])
def test_staged_segment_ends(gpu, wgs, out_dtype, G, cap):
    """Token-major V (the staged path) stores a segment that ends inside a
    range together with the next unit: through the wave's LDS region, half
    the group's rows a pass (G >= 4), or from the registers (G < 4). Short
    sequences put several ends into one range, the cap cuts segments into
    pieces; every output type."""
    wgs(cap)
    wl = synth.random_case(2600 + G, [5, 300, 17, 900, 1, 40, 2000, 33], 2 * G, 2, 128, 16, "bf16")
    say(f"staged segment ends G={G} out={out_dtype} cap={cap}")
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout="token")
    got = run_decode(wl, cache, tables, lens, max_ctx, BAL, out_dtype)
    H.assert_close(got, H.oracle_contiguous(wl), what=f"G={G} {out_dtype} cap={cap}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("v_layout", ["token", "dim"])
def test_fp8_segment_ends_16bit_outputs(gpu, wgs, out_dtype, v_layout):
    """fp8 pools (32-token units, staged either V layout) with 16-bit
    outputs and many segment ends per range."""
    wgs(5)
    wl = synth.random_case(2700, [5, 300, 17, 900, 1, 40, 2000, 33], 16, 2, 128, 16, "fp8")
    say(f"fp8 segment ends V {v_layout} out={out_dtype}")
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout=v_layout)
    got = run_decode(wl, cache, tables, lens, max_ctx, BAL, out_dtype)
    H.assert_close(got, H.oracle_contiguous(wl), what=f"fp8 {v_layout} {out_dtype}")


def test_agrees_with_partitions_and_is_deterministic(gpu):
    wl = synth.random_case(2600, [3, 129, 700, 1500, 4000], 32, 8, 128, 16, "bf16")
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout="dim")
    a = run_decode(wl, cache, tables, lens, max_ctx, BAL)
    b = run_decode(wl, cache, tables, lens, max_ctx, BAL)
    c = run_decode(wl, cache, tables, lens, max_ctx, 512)
    assert np.array_equal(a, b)  # the split depends only on the lengths and the grid
    H.assert_close(a, c, what="balanced vs partitions")
    H.assert_close(a, H.oracle_contiguous(wl))


def test_lengths_beyond_max_context_are_clamped(gpu):
    wl = synth.random_case(2700, [300, 90], 8, 2, 128, 16, "bf16")
    _, cache, tables, lens, _ = device_setup(wl, v_layout="dim")
    got = run_decode(wl, cache, tables, lens, 128, BAL)
    short = synth.random_case(2700, [300, 90], 8, 2, 128, 16, "bf16")
    k, v = wl.kv(0)
    short._kv_cache[0] = (k[:128], v[:128])
    short._kv_cache[1] = wl.kv(1)
    short.lengths = np.array([128, 90])
    H.assert_close(got, H.oracle_contiguous(short))


def test_needle_follows_logical_order(gpu, wgs):
    """One key per sequence matches the query; the output is that token's V
    row wherever it sits, also when the sequence is cut between workgroups."""
    wgs(5)
    L, hkv, D, G = 96, 1, 128, 4
    wl = synth.random_case(2800, [L] * 8, G * hkv, hkv, D, 16, "bf16", headroom=1.0)
    qv = torch.randn(D)
    q = qv.repeat(8, G, 1).bfloat16()
    wl._q = q
    qd = q.double()[0, 0]
    stars = [0, 1, 15, 16, 17, 47, 80, 95]
    for s, t_star in enumerate(stars):
        k = torch.zeros(L, hkv, D)
        k[t_star, 0] = 30.0 / (wl.scale * float(qd @ qd)) * qv
        v = torch.randn(L, hkv, D)
        wl._kv_cache[s] = (k.bfloat16(), v.bfloat16())
    got = _check(wl, "needle")
    for s, t_star in enumerate(stars):
        want = wl.kv(s)[1][t_star, 0].double().numpy()
        assert np.abs(got[s] - want).max() < 1e-3


def test_workspace_reused_across_batches(gpu, wgs):
    """One workspace serves consecutive calls of different batches and
    grids: nothing a call leaves in it changes a later call's result."""
    wl0 = synth.random_case(2700, [5000, 3, 800, 2500], 32, 8, 128, 16, "bf16")
    B, Hq, D = wl0.batch, wl0.num_q_heads, wl0.head_dim
    ws = workspace_for(8, Hq, 8, D, 9216, BAL)
    cases = [(wl0, None), (synth.random_case(2701, [700, 9000, 1, 64, 1500, 33, 4000, 2], 32, 8, 128, 16, "bf16"), 5),
             (wl0, 3), (wl0, None)]
    for wl, cap in cases:
        wgs(cap)
        say(f"reuse: B={wl.batch} cap={cap}")
        _, cache, tables, lens, max_ctx = device_setup(wl, v_layout="dim")
        q = wl.q().cuda()
        out = pa.decode(cache, q, tables, lens, max_ctx, wl.scale, BAL, out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        H.assert_close(out.cpu().double().numpy(), H.oracle_contiguous(wl), what=f"reuse B={wl.batch} cap={cap}")


def test_batch_at_the_lds_bound(gpu):
    """The largest batch the balanced split takes with token-major V for 8
    KV heads, G = 4, head_dim 128: its tile prefix fills the last bytes of
    the 160 KiB of LDS a workgroup may use next to the stage (B = 20288 is
    refused, see test_abi). Short sequences plus a few longer ones; sampled
    rows against the oracle, every row finite."""
    B = 20287
    rng = np.random.default_rng(31)
    lengths = rng.integers(1, 9, size=B)
    lengths[[0, 7, B // 2, B - 1]] = [1, 200, 65, 33]
    wl = synth.random_case(3300, lengths, 32, 8, 128, 16, "bf16")
    say(f"balanced split at B = {B}")
    _, cache, tables, lens, mx = device_setup(wl, v_layout="token")
    got = run_decode(wl, cache, tables, lens, mx, pa.BALANCED)
    assert np.isfinite(got).all()
    rows = [0, 1, 7, 100, B // 2, B - 2, B - 1]
    ref = H.oracle_contiguous(wl, seqs=rows)
    H.assert_close(got[rows], ref[rows], what="B at the LDS bound")
