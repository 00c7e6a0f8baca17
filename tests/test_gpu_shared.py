"""pa_decode_shared on the GPU: each group's shared prefix read once for all
its rows, against the fp64 oracle and against pa_decode.

Batches are built the way parallel sampling builds them: a prompt is
prefilled, forked into its samples (shared blocks, refcounts), each sample
appends tokens of its own (copy-on-write of a partial shared tail block),
then the groups come from pa_bm_shared_prefixes. Group sizes cover one row
tile and several (more members than 16 / G), groups of one member (left
out) and rows without a prompt of their own sharing anything."""
import numpy as np
import pytest
import torch

import paged_kv_cache_49_amd as pa
import synth
from oracle import attention as oatt
from tests import helpers as H
from tests.gpu_util import poison_fill, say

pytestmark = pytest.mark.gpu

_T = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.bfloat16}  # fp8 pools take bf16 sources
FP8_SCALES = (0.011, 0.013)  # per-tensor K / V scales of the fp8 cases (amax of N(0,1) samples / 448 or so)


def _values(rng, shape, kv):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(_T[kv])


def _build(seed, prompts, samples, tail_max, G, hkv, D, bs, kv, v_layout="dim"):
    """Prefill prompts, fork samples, append tails; returns everything a
    decode call and the oracle need."""
    rng = np.random.default_rng(seed)
    seqs = []  # (prompt, k, v) per batch row, full token-ordered K/V
    for p, (plen, ns) in enumerate(zip(prompts, samples)):
        kp, vp = _values(rng, (plen, hkv, D), kv), _values(rng, (plen, hkv, D), kv)
        for i in range(ns):
            t = int(rng.integers(1, tail_max + 1))
            kt, vt = _values(rng, (t, hkv, D), kv), _values(rng, (t, hkv, D), kv)
            seqs.append((p, kp, vp, kt, vt))
    B = len(seqs)
    total = sum(len(x[1]) + len(x[3]) for x in seqs)
    nb = total // bs + 4 * B + 16
    bm = pa.BlockManager(nb, bs, np.random.default_rng(seed + 1).permutation(nb).astype(np.int32))
    ks, vs = FP8_SCALES if kv == "fp8" else (1.0, 1.0)
    cache = pa.KVCache.allocate(nb, bs, hkv, D, kv, fill=poison_fill(kv), v_layout=v_layout, k_scale=ks, v_scale=vs)
    first_row = {}
    for row, (p, kp, vp, kt, vt) in enumerate(seqs):
        if p in first_row:
            bm.fork(first_row[p], row)
        else:
            first_row[p] = row
            sl, _ = bm.alloc(row, len(kp))
            pa.reshape_and_cache(cache, kp.cuda(), vp.cuda(), torch.from_numpy(sl).cuda())
    cows = []
    for row, (p, kp, vp, kt, vt) in enumerate(seqs):
        sl, cow = bm.alloc(row, len(kt))
        if cow:
            pa.copy_blocks(cache, torch.tensor(cow, dtype=torch.int32).cuda())
            cows += cow
        pa.reshape_and_cache(cache, kt.cuda(), vt.cuda(), torch.from_numpy(sl).cuda())
    mb = max(-(-(len(x[1]) + len(x[3])) // bs) for x in seqs)
    tables, lens = bm.pack(list(range(B)), mb, -1)
    q = _values(rng, (B, G * hkv, D), kv)
    return bm, cache, seqs, tables, lens, q, mb


def _oracle(seqs, q, hkv, scale, kv):
    ks, vs = FP8_SCALES if kv == "fp8" else (1.0, 1.0)
    qd = oatt.to_f64(q)
    out = np.zeros(qd.shape)
    for row, (p, kp, vp, kt, vt) in enumerate(seqs):
        k = oatt.source_values(torch.cat([kp, kt]), kv, ks)
        v = oatt.source_values(torch.cat([vp, vt]), kv, vs)
        out[row] = oatt.decode_contiguous(qd[row], k, v, scale, hkv)
    return out


def _run(seed, prompts, samples, tail_max, G, hkv, D, bs, kv, ps, what="", v_layout="dim"):
    say(f"shared {what}: prompts {prompts} x {samples} G={G} Hkv={hkv} D={D} bs={bs} {kv} ps={ps} V {v_layout}")
    bm, cache, seqs, tables, lens, q, mb = _build(seed, prompts, samples, tail_max, G, hkv, D, bs, kv, v_layout)
    B = len(seqs)
    sp = bm.shared_prefixes(list(range(B)), ps)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    scale = float(np.float32(1.0 / np.sqrt(D)))
    max_ctx = int(lens.max())
    td, ld, qd = dev(tables), dev(lens), q.cuda()
    got = pa.decode_shared(cache, qd, td, ld, max_ctx, scale, ps, dev(sp.offsets), dev(sp.members),
                           dev(sp.shared_len), sp.num_groups, sp.max_group_size, sp.max_shared_len,
                           sp.min_shared_len, out_dtype=torch.float32)
    plain = pa.decode(cache, qd, td, ld, max_ctx, scale, ps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = _oracle(seqs, q, hkv, scale, kv)
    g = got.cpu().double().numpy()
    ma, rl = H.assert_close(g, ref, what=f"shared {what}")
    H.assert_close(g, plain.cpu().double().numpy(), what=f"shared vs pa_decode {what}")
    say(f"   groups {sp.num_groups} (max {sp.max_group_size} rows, {sp.max_shared_len} shared tokens); "
        f"max-abs {ma:.2e} rel-L2 {rl:.2e}")
    return sp


CASES = [
    ("bf16", 128, 16, 4, 8, 512),
    ("bf16", 128, 16, 4, 8, 256),
    ("bf16", 64, 8, 8, 2, 256),
    ("f16", 128, 32, 1, 4, 512),
    ("f16", 64, 16, 2, 3, 128),
    ("fp8", 128, 16, 8, 4, 256),
    ("fp8", 64, 32, 4, 2, 512),
]


@pytest.mark.parametrize("kv,D,bs,G,hkv,ps", CASES, ids=lambda c: str(c))
def test_shared_parity(gpu, kv, D, bs, G, hkv, ps):
    # prompt lengths: several partitions, under one partition, and one with a
    # partial last block; 1-member group, 17-member group (> 16 / G rows)
    sp = _run(4000 + D + bs + G, [1100, 700, 2000, 90, 1301], [3, 1, 17, 4, 5], 80, G, hkv, D, bs, kv, ps,
              what=f"{kv} D{D} bs{bs} G{G}")
    assert sp.num_groups >= 2


@pytest.mark.parametrize("kv,D,bs,G,hkv,ps", [
    ("bf16", 128, 16, 4, 8, 512),
    ("f16", 64, 8, 8, 2, 256),
    ("fp8", 128, 32, 4, 4, 512),
], ids=lambda c: str(c))
def test_shared_token_major_v(gpu, kv, D, bs, G, hkv, ps):
    """The page's token-major V blocks: each tile's V rows go through the
    wave's LDS tile (fp8 widened to bf16) into the PV operand."""
    sp = _run(4200 + D + bs + G, [1100, 700, 2000, 90, 1301], [3, 1, 17, 4, 5], 80, G, hkv, D, bs, kv, ps,
              what=f"{kv} D{D} bs{bs} G{G}", v_layout="token")
    assert sp.num_groups >= 2


# The cascade (the balanced kernel over the groups' prefixes and the rows'
# tails, merged per row): groups of at most 32 / G rows on token-major V or
# fp8 pools, forced with PA_SHARED_PATH=cascade (an error if a case could
# not take it). Shapes: one and two head groups per workgroup set (Hkv 16),
# 1, 2, 4 and 8 KV heads per workgroup (Hkv 3 -> 1), fp8 prefixes rounded
# down to 32-token units (granule 16), short prefixes (a workgroup's range
# then crosses several prefix segments), a batch with fewer units than
# workgroups, block sizes 8 / 16 / 32.
CAS_CASES = [
    # kv, D, bs, G, hkv, ps, V layout, prompt lengths, samples per prompt
    ("bf16", 128, 16, 4, 8, 256, "token", [1100, 700, 2000, 90, 1301], [3, 1, 8, 4, 5]),
    ("f16", 64, 8, 8, 2, 16, "token", [300, 40, 77, 129], [4, 3, 2, 4]),
    ("bf16", 128, 32, 1, 4, 32, "token", [600, 33, 95], [32, 5, 2]),
    ("fp8", 128, 16, 8, 4, 16, "dim", [1100, 48, 400], [4, 3, 2]),
    ("fp8", 64, 32, 4, 16, 64, "token", [700, 200, 65], [8, 2, 3]),
    ("bf16", 128, 16, 2, 16, 16, "token", [50, 20, 33, 17, 64, 18], [16, 2, 3, 5, 2, 7]),
    ("f16", 128, 16, 4, 8, 16, "token", [40], [2]),
    ("fp8", 128, 8, 2, 8, 16, "token", [513, 256, 31], [16, 4, 9]),
    ("bf16", 64, 16, 2, 3, 16, "token", [100, 70], [6, 3]),
]


@pytest.mark.parametrize("kv,D,bs,G,hkv,ps,layout,prompts,samples", CAS_CASES, ids=lambda c: str(c))
def test_shared_cascade(gpu, monkeypatch, kv, D, bs, G, hkv, ps, layout, prompts, samples):
    monkeypatch.setenv("PA_SHARED_PATH", "cascade")
    sp = _run(4300 + D + bs + G + hkv, prompts, samples, 40, G, hkv, D, bs, kv, ps,
              what=f"cascade {kv} D{D} bs{bs} G{G} Hkv{hkv}", v_layout=layout)
    assert sp.num_groups >= 1 and sp.max_group_size * G <= 32


def test_shared_cascade_refuses_large_groups(gpu, monkeypatch):
    """A group of more than 32 / G rows has no cascade: forced, the call
    fails; by default it takes the shared-prefix partition kernels."""
    monkeypatch.setenv("PA_SHARED_PATH", "cascade")
    with pytest.raises(pa.Unsupported):
        _run(4400, [300, 200], [9, 2], 20, 4, 8, 128, 16, "bf16", 16, what="cascade, 9 x 4 rows", v_layout="token")
    monkeypatch.delenv("PA_SHARED_PATH")
    _run(4400, [300, 200], [9, 2], 20, 4, 8, 128, 16, "bf16", 16, what="9 x 4 rows, default", v_layout="token")


def test_shared_cascade_matches_partition_path(gpu, monkeypatch):
    """The same call on both paths (cascade and partition kernels) agrees to
    the parity tolerance on every row."""
    kw = dict(seed=4500, prompts=[900, 333, 1500], samples=[8, 3, 6], tail_max=70, G=4, hkv=8, D=128, bs=16,
              kv="bf16", v_layout="token")
    bm, cache, seqs, tables, lens, q, mb = _build(kw["seed"], kw["prompts"], kw["samples"], kw["tail_max"], kw["G"],
                                                  kw["hkv"], kw["D"], kw["bs"], kw["kv"], kw["v_layout"])
    B = len(seqs)
    sp = bm.shared_prefixes(list(range(B)), 256)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    scale = float(np.float32(1.0 / np.sqrt(kw["D"])))
    args = (cache, q.cuda(), dev(tables), dev(lens), int(lens.max()), scale, 256, dev(sp.offsets), dev(sp.members),
            dev(sp.shared_len), sp.num_groups, sp.max_group_size, sp.max_shared_len, sp.min_shared_len)
    outs = {}
    for path in ("cascade", "partition"):
        monkeypatch.setenv("PA_SHARED_PATH", path)
        say(f"shared: {path} path")
        outs[path] = pa.decode_shared(*args, out_dtype=torch.float32)
    torch.cuda.synchronize()
    H.assert_close(outs["cascade"].cpu().double().numpy(), outs["partition"].cpu().double().numpy(),
                   what="cascade vs partition path")


@pytest.mark.parametrize("layout", ["dim", "token"])
def test_shared_prefix_sharing_workload(gpu, layout):
    """The 16 prompts x 8 samples workload (2048 + r shared tokens, tails
    U[0, 256], one new token), partitions of 512, all rows vs the oracle
    (token-major V: the cascade)."""
    wl = synth.prefix_sharing(partial_tail=True)
    P, S, hkv, D, bs = wl.prompts, wl.samples, wl.num_kv_heads, wl.head_dim, wl.block_size
    say(f"shared: prefix-sharing workload, V {layout}")
    bm = pa.BlockManager(wl.num_blocks, bs, wl.free_order)
    cache = pa.KVCache.allocate(wl.num_blocks, bs, hkv, D, "bf16", fill=float("nan"), v_layout=layout)
    for p in range(P):
        k, v = wl.prefix_kv(p)
        sl, _ = bm.alloc(p * S, len(k))
        pa.reshape_and_cache(cache, k.cuda(), v.cuda(), torch.from_numpy(sl).cuda())
        for i in range(1, S):
            bm.fork(p * S, p * S + i)
    for p in range(P):
        for i in range(S):
            kt, vt = wl.tail_kv(p, i)
            sl, cow = bm.alloc(p * S + i, len(kt))
            if cow:
                pa.copy_blocks(cache, torch.tensor(cow, dtype=torch.int32).cuda())
            pa.reshape_and_cache(cache, kt.cuda(), vt.cuda(), torch.from_numpy(sl).cuda())
    B = P * S
    mb = int(-(-(int(wl.prefix_len.max() + wl.tail_len.max()) + 2) // bs))
    tables, lens = bm.pack(list(range(B)), mb, -1)
    sp = bm.shared_prefixes(list(range(B)), 512)
    assert sp.num_groups == P and sp.max_group_size == S and sp.max_shared_len == 2048
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
    q = wl.q().cuda()
    got = pa.decode_shared(cache, q, dev(tables), dev(lens), int(lens.max()), wl.scale, 512, dev(sp.offsets),
                           dev(sp.members), dev(sp.shared_len), sp.num_groups, sp.max_group_size, sp.max_shared_len,
                           sp.min_shared_len, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qd = oatt.to_f64(wl.q())
    ref = np.zeros(qd.shape)
    for p in range(P):
        k, v = wl.prefix_kv(p)
        for i in range(S):
            kt, vt = wl.tail_kv(p, i)
            ref[p * S + i] = oatt.decode_contiguous(qd[p * S + i], oatt.to_f64(torch.cat([k, kt])),
                                                    oatt.to_f64(torch.cat([v, vt])), wl.scale, hkv)
    ma, rl = H.assert_close(got.cpu().double().numpy(), ref, what="prefix-sharing workload")
    say(f"   max-abs {ma:.2e} rel-L2 {rl:.2e}")


def test_no_groups_is_plain_decode(gpu):
    """With no group (num_groups = 0) the call is pa_decode."""
    wl = synth.random_case(4100, [300, 1200, 5], 16, 4, 128, 16, "bf16")
    from tests.gpu_util import device_setup, run_decode
    _, cache, tables, lens, max_ctx = device_setup(wl, v_layout="dim")
    z = torch.zeros(wl.batch + 1, dtype=torch.int32, device="cuda")
    got = pa.decode_shared(cache, wl.q().cuda(), tables, lens, max_ctx, wl.scale, 256, z, z, z, 0, 0, 0, 0,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    H.assert_close(got.cpu().double().numpy(), H.oracle_contiguous(wl), what="no groups")


@pytest.mark.parametrize("layout", ["dim", "token"])
def test_runner_shared_steps(gpu, layout):
    """PagedBatch.step(shared=True): groups computed from the block manager
    at every step, uploaded with the step's metadata; two steps in a row
    against the oracle."""
    from paged_kv_cache_49_amd.runner import PagedBatch, workspace_for
    wl = synth.prefix_sharing(prompts=4, samples=5, prefix=1024, partial_tail=True, max_tail=60)
    P, S, hkv, D, bs = wl.prompts, wl.samples, wl.num_kv_heads, wl.head_dim, wl.block_size
    say(f"shared: runner steps, V {layout}")
    bm = pa.BlockManager(wl.num_blocks + 64, bs, None)
    cache = pa.KVCache.allocate(wl.num_blocks + 64, bs, hkv, D, "bf16", fill=float("nan"), v_layout=layout)
    mb = int(-(-(int(wl.prefix_len.max() + wl.tail_len.max()) + 4) // bs))
    batch = PagedBatch(bm, [cache], mb, P * S)
    for p in range(P):
        k, v = wl.prefix_kv(p)
        batch.prefill(p * S, [k], [v])
        for i in range(1, S):
            batch.fork(p * S, p * S + i)
    own_k, own_v = {}, {}
    for p in range(P):
        for i in range(S):
            kt, vt = wl.tail_kv(p, i)
            n = int(wl.tail_len[p, i])
            batch.prefill(p * S + i, [kt[:n]], [vt[:n]])
            own_k[p * S + i], own_v[p * S + i] = [kt[:n]], [vt[:n]]
    B = P * S
    rng = np.random.default_rng(11)
    ws = workspace_for(B, wl.num_q_heads, hkv, D, mb * bs, 512, shared=True)
    for step in range(2):
        kn = _values(rng, (B, hkv, D), "bf16")
        vn = _values(rng, (B, hkv, D), "bf16")
        q = _values(rng, (B, wl.num_q_heads, D), "bf16")
        out = torch.empty(B, wl.num_q_heads, D, dtype=torch.float32, device="cuda")
        batch.step(np.arange(B), [kn.cuda()], [vn.cuda()], [q.cuda()], [out], wl.scale, 512, ws, shared=True)
        torch.cuda.synchronize()
        qd = oatt.to_f64(q)
        ref = np.zeros(qd.shape)
        for p in range(P):
            k, v = wl.prefix_kv(p)
            for i in range(S):
                r = p * S + i
                own_k[r].append(kn[r:r + 1])
                own_v[r].append(vn[r:r + 1])
                ref[r] = oatt.decode_contiguous(qd[r], oatt.to_f64(torch.cat([k] + own_k[r])),
                                                oatt.to_f64(torch.cat([v] + own_v[r])), wl.scale, hkv)
        H.assert_close(out.cpu().double().numpy(), ref, what=f"runner shared step {step}")
    sp = bm.shared_prefixes(list(range(B)), 512)
    assert sp.num_groups == P and sp.max_shared_len == 1024
