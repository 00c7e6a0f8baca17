"""The seeded generators are deterministic and match the stated shapes."""
import numpy as np
import torch

import synth


def test_generators_are_deterministic():
    a, b = synth.gqa_decode(), synth.gqa_decode()
    assert np.array_equal(a.lengths, b.lengths) and np.array_equal(a.free_order, b.free_order)
    assert torch.equal(a.q(), b.q())
    # per-sequence streams: drawing seq 5 alone gives the same values
    assert torch.equal(a.kv(5)[0], b.kv(5)[0]) and torch.equal(a.kv(5)[1], b.kv(5)[1])


def test_workload_shapes():
    t = synth.tiny_decode()
    assert t.lengths.tolist() == [1, 17, 33, 100] and t.num_blocks == 64 and t.head_dim == 64
    assert sorted(t.free_order.tolist()) == list(range(64)) and t.kv_dtype == "f16"
    g = synth.gqa_decode()
    assert g.batch == 64 and g.lengths.min() >= 512 and g.lengths.max() <= 4096 and g.group == 4
    used = sum(-(-int(n) // 16) for n in g.lengths)
    assert g.num_blocks == int(np.ceil(used * 1.1))
    lc = synth.long_context()
    assert lc.batch == 8 and lc.lengths.min() >= 32768 and lc.lengths.max() <= 131072
    for bs in (8, 16, 32):
        m = synth.mixed_lengths(bs)
        assert m.batch == 256 and m.lengths.min() >= 16 and m.lengths.max() <= 16384 and m.group == 8
    assert np.array_equal(synth.mixed_lengths(8).lengths, synth.mixed_lengths(32).lengths)
    p = synth.prefix_sharing()
    assert p.prefix_len.min() >= 2049 and p.prefix_len.max() <= 2063 and p.tail_len.max() <= 256
    p0 = synth.prefix_sharing(partial_tail=False)
    assert (p0.prefix_len == 2048).all()


def test_fp8_scale_is_amax_over_448():
    wl = synth.random_case(3, [10, 20], 4, 2, 16, 8, "fp8")
    ks, vs = wl.kv_scales()
    amax = max(float(wl.kv(s)[0].float().abs().max()) for s in range(2))
    assert ks == float(np.float32(amax / 448.0))
