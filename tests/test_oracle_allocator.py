"""Pins for the allocator model (CPU only): the pages' worked examples, the
capacity closed forms of the course page's verification questions, and
invariants under random operation sequences (hypothesis)."""
import json
import os
from collections import Counter

import pytest
from hypothesis import given, settings, strategies as st

from oracle import allocator as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def check_invariants(m: A.BlockAllocatorModel):
    rc = m.refcnt
    refs = Counter(b for s in m.seqs() for b in m.table(s))
    assert all(rc[b] == refs.get(b, 0) for b in range(m.num_blocks)), "refcount != references"
    stack = m.free_stack
    assert len(set(stack)) == len(stack)
    assert sorted(stack) == [b for b in range(m.num_blocks) if rc[b] == 0], "free stack != unreferenced"
    for s in m.seqs():
        L = m.length(s)
        assert len(m.table(s)) == A.blocks_for(L, m.block_size)  # ceil(L/bs): <= 1 partial block
        assert A.paged_waste_tokens(L, m.block_size) <= m.block_size - 1


def test_note_minimal_model_table():
    g = _golden("note_minimal_model.json")
    bs = 16
    order = g["block_table"] + [b for b in range(g["pool_blocks"]) if b not in g["block_table"]]
    m = A.BlockAllocatorModel(g["pool_blocks"], bs, order)
    slots, cows = m.alloc(0, 3 * bs)
    assert m.table(0) == g["block_table"] and not cows
    assert slots[:2] == [7 * bs, 7 * bs + 1] and slots[bs] == 2 * bs and slots[-1] == 9 * bs + bs - 1
    # growth is one block at a time: the 49th token takes one more block
    m.alloc(0, 1)
    assert len(m.table(0)) == 4
    check_invariants(m)


def test_course_mental_model_sharing():
    g = _golden("course_mental_model_sharing.json")
    order = [3, 7, 1, 9] + [b for b in range(12) if b not in (3, 7, 1, 9)]
    m = A.BlockAllocatorModel(12, 16, order)
    m.alloc("A", 16)          # the shared prefix fills b3
    m.fork("A", "B")          # B points at the same physical block
    m.alloc("A", 32)          # A grows: b7, b1 (b3 is full, nothing copied)
    _, cows = m.alloc("B", 16)  # B grows: b9
    assert not cows
    assert m.table("A") == g["seq_a"] and m.table("B") == g["seq_b"]
    assert m.refcnt[g["shared_block"]] == g["shared_refcount"]
    assert m.stats()["num_shared"] == 1
    check_invariants(m)


def test_course_capacity_examples():
    g = _golden("course_capacity.json")
    bs = g["block_size"]
    assert A.blocks_for(g["request_tokens"], bs) == g["printed_blocks_approx"] == 7
    w = A.naive_waste(g["request_tokens"], g["slab_tokens"])
    assert round(w, 2) in (0.98, 0.99) and abs(w - (1 - 100 / 8192)) < 1e-15
    assert A.paged_waste_tokens(100, bs) == 12


@pytest.mark.parametrize("ctx", [4096, 2048])
def test_course_q4_q5_capacity(ctx):
    g = _golden("course_capacity.json")
    nb, bs = g["q4_pool_blocks"], g["block_size"]
    m = A.BlockAllocatorModel(nb, bs)
    fits = 0
    while True:
        try:
            m.alloc(fits, ctx)
        except A.OutOfBlocks:
            break
        fits += 1
    assert fits == A.capacity(nb, ctx, bs) == nb // (ctx // bs)
    assert m.stats()["num_free"] == nb - fits * (ctx // bs) == 16
    assert {4096: 39, 2048: 78}[ctx] == fits  # halving the context doubles concurrency


def test_copy_on_write_gives_writer_a_copy():
    m = A.BlockAllocatorModel(8, 4, list(range(8)))
    m.alloc("p", 6)                       # blocks [0, 1], block 1 half full
    m.fork("p", "c1")
    m.fork("p", "c2")
    assert m.refcnt[1] == 3
    slots, cows = m.alloc("c1", 1)        # c1 writes into shared block 1
    assert cows == [(1, 2)] and m.table("c1") == [0, 2] and slots == [2 * 4 + 2]
    assert m.table("p") == [0, 1] and m.table("c2") == [0, 1]  # others keep the original
    _, cows = m.alloc("c2", 3)            # copies again; then grows one block
    assert cows == [(1, 3)] and m.table("c2") == [0, 3, 4]
    slots, cows = m.alloc("p", 1)         # last holder writes in place
    assert cows == [] and slots == [1 * 4 + 2] and m.refcnt[1] == 1
    assert m.stats()["cow_copies"] == 2
    check_invariants(m)


def test_full_shared_block_is_never_copied():
    m = A.BlockAllocatorModel(8, 4)
    m.alloc(0, 8)
    m.fork(0, 1)
    _, cows = m.alloc(1, 1)
    assert cows == [] and m.table(1)[:2] == m.table(0)
    check_invariants(m)


def test_exhaustion_changes_nothing():
    m = A.BlockAllocatorModel(6, 4, [5, 4, 3, 2, 1, 0])
    m.alloc(0, 10)
    m.fork(0, 1)
    before = (m.free_stack, m.refcnt, {s: m.table(s) for s in m.seqs()})
    with pytest.raises(A.OutOfBlocks):
        m.alloc_batch([0, 1, 2], [1, 1, 9])   # 1 copy (seq 1 then writes in place) + 3 new > 3 free
    m2 = A.BlockAllocatorModel(6, 4, [5, 4, 3, 2, 1, 0])
    m2.alloc(0, 10)
    m2.fork(0, 1)
    m2.alloc_batch([0, 1, 2], [1, 1, 8])      # exactly 3 blocks: fits
    with pytest.raises(A.OutOfBlocks):
        m.alloc(7, 13)                        # an unknown seq is not created on failure
    assert (m.free_stack, m.refcnt, {s: m.table(s) for s in m.seqs()}) == before
    assert 7 not in m.seqs()


def test_batch_copy_on_write_counts_in_order():
    m = A.BlockAllocatorModel(16, 4, list(range(16)))
    m.alloc(0, 5)
    m.fork(0, 1)
    m.fork(0, 2)
    slots, cows = m.alloc_batch([2, 0, 1], [1, 1, 1])
    assert cows == [(1, 2), (1, 3)]           # seqs 2 and 0 copy, seq 1 writes in place
    assert m.table(1) == [0, 1] and m.refcnt[1] == 1
    assert slots == [2 * 4 + 1, 3 * 4 + 1, 1 * 4 + 1]


def test_error_paths():
    m = A.BlockAllocatorModel(4, 4)
    with pytest.raises(A.UnknownSeq):
        m.free(3)
    with pytest.raises(A.UnknownSeq):
        m.fork(1, 2)
    m.alloc(1, 1)
    with pytest.raises(A.SeqExists):
        m.fork(1, 1)
    with pytest.raises(A.InvalidArgument):
        m.alloc_batch([1, 1], [1, 1])
    with pytest.raises(A.InvalidArgument):
        A.BlockAllocatorModel(3, 4, [0, 1, 1])


def test_free_returns_every_block_and_reuses_last_first():
    m = A.BlockAllocatorModel(10, 2, list(range(10)))
    m.alloc(0, 5)   # blocks 0, 1, 2
    m.free(0)
    assert m.stats()["num_free"] == 10
    slots, _ = m.alloc(1, 1)
    assert slots == [2 * 2]  # the freed sequence's last block is popped first


_ops = st.lists(
    st.one_of(
        st.tuples(st.just("alloc"), st.integers(0, 5), st.integers(0, 9)),
        st.tuples(st.just("fork"), st.integers(0, 5), st.integers(0, 5)),
        st.tuples(st.just("free"), st.integers(0, 5), st.just(0)),
        st.tuples(st.just("batch"), st.lists(st.integers(0, 5), max_size=4, unique=True),
                  st.lists(st.integers(0, 5), min_size=4, max_size=4)),
    ),
    max_size=40,
)


@settings(max_examples=300, deadline=None)
@given(ops=_ops, bs=st.sampled_from([1, 2, 4]), nb=st.integers(1, 24))
def test_invariants_under_random_operations(ops, bs, nb):
    m = A.BlockAllocatorModel(nb, bs)
    for op in ops:
        before = (m.free_stack, m.refcnt, {s: (m.table(s), m.length(s)) for s in m.seqs()})
        shared_before = {s: list(m.table(s)) for s in m.seqs()}
        try:
            if op[0] == "alloc":
                _, cows = m.alloc(op[1], op[2])
                for src, dst in cows:  # the other holders are untouched
                    for s, t in shared_before.items():
                        if s != op[1]:
                            assert m.table(s) == t
            elif op[0] == "fork":
                m.fork(op[1], op[2])
            elif op[0] == "free":
                m.free(op[1])
            else:
                m.alloc_batch(op[1], op[2][: len(op[1])])
        except A.AllocError:
            assert (m.free_stack, m.refcnt, {s: (m.table(s), m.length(s)) for s in m.seqs()}) == before
        check_invariants(m)
    for s in m.seqs():
        m.free(s)
    assert sorted(m.free_stack) == list(range(nb)) and m.stats()["num_used"] == 0
