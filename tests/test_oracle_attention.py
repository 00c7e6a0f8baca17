"""Pins for the attention oracle (CPU only).

The oracle is checked against things other than itself: torch's
scaled_dot_product_attention (an independent library routine, fp64), closed
forms (L = 1, equal keys, zero scale, constant values, a "needle" key), the
log-sum-exp merge identity, the worked block table of the "PagedAttention"
LLM note (section 最小模型), invariance under the physical placement of
blocks, and a set of planted mistakes that the pins must catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import allocator as oalloc
from oracle import attention as oatt
from oracle import cache_ops as ocache
from tests import helpers as H

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _source_f64(wl, s):
    k, v = wl.kv(s)
    ks, vs = wl.kv_scales()
    return oatt.source_values(k, wl.kv_dtype, ks), oatt.source_values(v, wl.kv_dtype, vs)


def _sdpa_all(wl):
    q = oatt.to_f64(wl.q())
    out = np.zeros_like(q)
    for s in range(wl.batch):
        k, v = _source_f64(wl, s)
        if k.shape[0]:
            out[s] = H.sdpa_reference(q[s], k, v, wl.scale)
    return out


def _random_cases():
    """Random tiny cases over block sizes and group sizes, each with an f16
    and a bf16 pool (the two 16-bit storage formats decode differently)."""
    cases = []
    rng = np.random.default_rng(7)
    for i, (bs, g, hkv, d) in enumerate([(1, 1, 2, 16), (2, 2, 2, 8), (4, 4, 2, 16), (16, 4, 1, 32),
                                         (16, 1, 3, 8), (4, 2, 2, 24), (8, 8, 1, 16)]):
        lengths = rng.integers(1, 41, size=3)
        for dt in ("f16", "bf16"):
            cases.append(synth.random_case(100 + i, lengths, g * hkv, hkv, d, bs, dt))
    return cases


def test_tiny_workload_matches_sdpa():
    wl = synth.tiny_decode()
    got = H.oracle_paged(wl)
    ref = _sdpa_all(wl)
    assert np.abs(got - ref).max() <= 1e-12


@pytest.mark.parametrize("wl", _random_cases(), ids=lambda w: f"{w.name}-{w.kv_dtype}-bs{w.block_size}-g{w.group}")
def test_random_cases_match_sdpa(wl):
    got = H.oracle_paged(wl)
    ref = _sdpa_all(wl)
    assert np.abs(got - ref).max() <= 1e-12
    # the table route and the token-order route agree exactly in value
    assert np.abs(got - H.oracle_contiguous(wl)).max() <= 1e-13


def test_fp8_cache_matches_sdpa_on_dequantised_values():
    wl = synth.random_case(11, [5, 33, 16], 8, 2, 32, 8, "fp8")
    got = H.oracle_paged(wl)
    ref = _sdpa_all(wl)
    assert np.abs(got - ref).max() <= 1e-12


def test_bf16_pool_bits_decode_by_hand():
    """bf16 storage is the top half of an IEEE binary32: sign, 8 exponent
    bits (bias 127), 7 fraction bits. Values worked out by hand."""
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x0080, 0x7F7F, 0x8000, 0x4049, 0x3E00], np.uint16)
    want = np.array([1.0, -2.0, 1.5,
                     2.0 ** -133,                      # smallest subnormal: 2^-126 * 2^-7
                     2.0 ** -126,                      # smallest normal
                     (2.0 - 2.0 ** -7) * 2.0 ** 127,   # largest finite
                     -0.0, 3.140625,                   # 1.5703125 * 2
                     0.125])
    got = oatt.pool_values(bits, "bf16")
    assert np.array_equal(got, want)
    assert np.signbit(got[6])


def test_bf16_pool_matches_sdpa_on_the_source_values():
    """A bf16 pool written through the slot model and decoded by the oracle
    gives SDPA's result on the source tensors' own values (torch's bf16 ->
    fp64 conversion, a route that does not use the oracle's decoder)."""
    wl = synth.random_case(12, [1, 16, 17, 40], 8, 2, 32, 16, "bf16")
    assert np.abs(H.oracle_paged(wl) - _sdpa_all(wl)).max() <= 1e-12


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((1, 2, 16))
    v = rng.standard_normal((1, 2, 16))
    out = oatt.decode_contiguous(q, k, v, 0.7, 2)
    assert np.array_equal(out[:2], np.repeat(v[0, :1], 2, 0))
    assert np.array_equal(out[2:], np.repeat(v[0, 1:], 2, 0))


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    L = 37
    q = rng.standard_normal((3, 8))
    k = np.repeat(rng.standard_normal((1, 1, 8)), L, axis=0)
    v = rng.standard_normal((L, 1, 8))
    out = oatt.decode_contiguous(q, k, v, 0.5, 1)
    assert np.abs(out - v[:, 0].mean(axis=0)).max() <= 1e-14


def test_zero_scale_gives_mean_of_values():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 8))
    k = rng.standard_normal((20, 1, 8))
    v = rng.standard_normal((20, 1, 8))
    out = oatt.decode_contiguous(q, k, v, 0.0, 1)
    assert np.abs(out - v[:, 0].mean(axis=0)).max() <= 1e-14


def test_constant_values_pass_through():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 8))
    k = rng.standard_normal((20, 1, 8)) * 3
    c = rng.standard_normal(8)
    v = np.broadcast_to(c, (20, 1, 8)).copy()
    out = oatt.decode_contiguous(q, k, v, 0.9, 1)
    assert np.abs(out - c).max() <= 1e-14


@pytest.mark.parametrize("t_star", [0, 1, 15, 16, 17, 40, 63])
def test_needle_selects_its_value(t_star):
    """K_t = 0 except K_{t*} = c q (c = 30/(scale |q|^2)): the logit gap is
    30, so the output is V_{t*} up to about L e^-30."""
    rng = np.random.default_rng(5)
    L, D, scale = 64, 16, 0.25
    qv = rng.standard_normal(D)
    q = np.stack([qv, qv])  # both heads of the group share q
    k = np.zeros((L, 1, D))
    k[t_star, 0] = 30.0 / (scale * qv @ qv) * qv
    v = rng.standard_normal((L, 1, D))
    out = oatt.decode_contiguous(q, k, v, scale, 1)
    bound = L * math.exp(-30.0) * np.abs(v).max() * 2
    assert np.abs(out - v[t_star, 0]).max() <= bound


def test_lse_merge_identity():
    """Attention over a sequence equals the log-sum-exp merge of attention
    over any split of it into consecutive parts (the split-K reduction)."""
    rng = np.random.default_rng(6)
    L, D = 300, 16
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    scale = 0.3
    whole = oatt.attend(q, k, v, scale)
    for cuts in ([0, 100, 200, 300], [0, 1, 299, 300], [0, 150, 300], [0, 64, 128, 192, 256, 300]):
        ms, ls, os_ = [], [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            z = scale * (q @ k[a:b].T)[0]
            m = z.max()
            w = np.exp(z - m)
            ms.append(m)
            ls.append(w.sum())
            os_.append(w @ v[a:b] / w.sum())
        mstar = max(ms)
        wts = np.array([l * math.exp(m - mstar) for m, l in zip(ms, ls)])
        merged = (wts[:, None] * np.array(os_)).sum(0) / wts.sum()
        assert np.abs(merged - whole[0]).max() <= 1e-13


def test_note_minimal_model_gather_order():
    """The worked table of the LLM note's minimal model: logical blocks
    0, 1, 2 live in physical blocks 7, 2, 9 of a 10-block pool."""
    with open(os.path.join(GOLDEN, "note_minimal_model.json")) as f:
        g = json.load(f)
    bs = 4
    pool = np.zeros((g["pool_blocks"], bs, 1, 2))
    for blk in range(g["pool_blocks"]):
        for off in range(bs):
            pool[blk, off, 0] = (blk, off)  # tag every row with its location
    rows = oatt.gather_sequence(pool, g["block_table"], 3 * bs, bs)
    got = [(int(r[0, 0]), int(r[0, 1])) for r in rows]
    want = [(b, o) for b in g["block_table"] for o in range(bs)]
    assert got == want
    # the printed physical row: A<i> sits at the position the table names
    for i, phys in enumerate(g["block_table"]):
        assert g["physical_row"][phys] == f"A{i}"


def test_physical_placement_does_not_change_result():
    base = synth.random_case(21, [33, 7, 48, 1], 8, 2, 16, 4, "bf16", headroom=2.0)
    out0 = H.oracle_paged(base)
    for seed in range(3):
        wl = synth.random_case(21, [33, 7, 48, 1], 8, 2, 16, 4, "bf16", headroom=2.0)
        wl.free_order = np.random.default_rng(seed).permutation(wl.num_blocks).astype(np.int32)
        assert np.array_equal(H.oracle_paged(wl), out0)


def test_empty_sequence_gives_zeros():
    wl = synth.random_case(22, [0, 5], 4, 2, 8, 4, "f16")
    out = H.oracle_paged(wl)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.abs(out[1]).max() > 0


def test_table_entries_past_the_length_are_not_read():
    wl = synth.random_case(23, [9, 16], 4, 2, 8, 4, "f16")
    alloc, kp, vp, tables, lens = H.oracle_setup(wl, max_blocks=8, pad=10 ** 6)
    out = oatt.paged_decode(wl.q(), kp, vp, tables, lens, wl.scale, wl.block_size, "f16")
    assert np.isfinite(out).all()


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant is a plausible bug in the oracle; the SDPA
# pin must reject every one of them.

def _mut_gather_swapped(pool, table_row, length, bs):
    t = np.arange(length)
    row = np.asarray(table_row[: -(-length // bs)], np.int64)
    return pool[row[(t % bs) % len(row)], (t // bs) % bs]


def _mut_gather_short(pool, table_row, length, bs):
    return oatt.__dict__["_orig_gather"](pool, table_row, max(length - 1, 1), bs)


def _mut_attend_noscale(q, k, v, scale):
    return oatt.__dict__["_orig_attend"](q, k, v, 1.0)


def _mut_attend_v_is_k(q, k, v, scale):
    return oatt.__dict__["_orig_attend"](q, k, k, scale)


def _mut_attend_unnormalised(q, k, v, scale):
    z = scale * (q @ k.T)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return w @ v


def _mut_attend_wrong_axis(q, k, v, scale):
    z = scale * (k @ q.T)  # [L][G], softmax over heads instead of tokens
    w = np.exp(z - z.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return (w.T @ v) / w.shape[0]


def _mut_decode_head_mod(q, k_seq, v_seq, scale, num_kv_heads):
    q = oatt.to_f64(q)
    out = np.empty_like(q)
    for h in range(q.shape[0]):
        kvh = h % num_kv_heads
        out[h] = oatt.attend(q[h:h + 1], k_seq[:, kvh], v_seq[:, kvh], scale)[0]
    return out


def _mut_pool_values_bf16_shift(pool_bits, kv_dtype, scale=1.0):
    if kv_dtype == "bf16":
        return (pool_bits.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    return oatt.__dict__["_orig_pool_values"](pool_bits, kv_dtype, scale)


MUTANTS = {
    "gather-block-offset-swapped": ("gather_sequence", _mut_gather_swapped),
    "gather-drops-last-token": ("gather_sequence", _mut_gather_short),
    "scale-dropped": ("attend", _mut_attend_noscale),
    "value-is-key": ("attend", _mut_attend_v_is_k),
    "softmax-unnormalised": ("attend", _mut_attend_unnormalised),
    "softmax-wrong-axis": ("attend", _mut_attend_wrong_axis),
    "head-group-modulo": ("decode_contiguous", _mut_decode_head_mod),
    "bf16-decode-shift": ("pool_values", _mut_pool_values_bf16_shift),
}


@pytest.mark.parametrize("kv_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, kv_dtype, monkeypatch):
    attr, fn = MUTANTS[name]
    if name.startswith("bf16") and kv_dtype != "bf16":
        pytest.skip("a bf16-only mistake")
    monkeypatch.setitem(oatt.__dict__, "_orig_gather", oatt.gather_sequence)
    monkeypatch.setitem(oatt.__dict__, "_orig_attend", oatt.attend)
    monkeypatch.setitem(oatt.__dict__, "_orig_pool_values", oatt.pool_values)
    wl = synth.random_case(31, [19, 40, 6], 8, 2, 16, 4, kv_dtype)
    ref = _sdpa_all(wl)
    monkeypatch.setattr(oatt, attr, fn)
    got = H.oracle_paged(wl)
    assert np.abs(got - ref).max() > 1e-6, f"mutant {name} not caught"
