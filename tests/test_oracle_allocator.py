"""Pins for the allocator model (CPU only): the pages' worked examples, the
capacity closed forms of the course page's verification questions,
invariants under random operation sequences (hypothesis), and hand-built
cases for swapping and prefix caching (what a swap must move and free,
which blocks a repeated or diverging prompt gets back, eviction order)."""
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


# ---- swapping ([course] §4 and §8: a preempted sequence's blocks can be
# swapped out and brought back later). Pins: plain counting of what a swap
# must move and free, on hand-built states.

def _snapshot(m):
    return (m.seqs(), [m.table(s) for s in m.seqs()], m.free_stack, m.host_free_stack, m.refcnt,
            m.evictable, m.host_stats())


def test_swap_round_trip_restores_the_sequence_and_both_pools():
    bs = 16
    m = A.BlockAllocatorModel(40, bs)
    m.set_host_pool(10)
    m.alloc(1, 100)  # 7 blocks
    m.alloc(2, 20)   # 2 blocks
    t1 = m.table(1)
    pairs = m.swap_out(1)
    assert [d for d, _ in pairs] == t1                 # every block, in logical order
    assert len({h for _, h in pairs}) == 7             # each to its own host block
    assert len(m.free_stack) == 40 - 2                 # its 7 device blocks are free again
    assert len(m.host_free_stack) == 3
    assert m.is_swapped(1) and m.length(1) == 100
    back = m.swap_in(1)
    assert [h for h, _ in back] == [h for _, h in pairs]
    assert len(m.table(1)) == 7 and all(m.refcnt[b] == 1 for b in m.table(1))
    assert len(m.host_free_stack) == 10 and not m.is_swapped(1)
    assert m.host_stats()["swap_outs"] == 1 and m.host_stats()["swap_ins"] == 1
    check_invariants(m)


def test_swapping_out_a_fork_leaves_the_shared_blocks_to_the_others():
    m = A.BlockAllocatorModel(20, 16)
    m.set_host_pool(8)
    m.alloc(1, 40)
    m.fork(1, 2)  # 3 blocks at refcount 2
    shared = m.table(1)
    free_before = len(m.free_stack)
    pairs = m.swap_out(2)
    assert [d for d, _ in pairs] == shared             # the data still moves (the copy is the swapped one's)
    assert m.table(1) == shared and all(m.refcnt[b] == 1 for b in shared)
    assert len(m.free_stack) == free_before            # nothing freed: sequence 1 still holds them
    m.swap_in(2)
    assert not set(m.table(2)) & set(shared)           # fresh blocks; the sharing is not restored
    check_invariants(m)


def test_swap_out_and_in_are_all_or_nothing():
    m = A.BlockAllocatorModel(20, 16)
    m.set_host_pool(2)
    m.alloc(1, 40)  # 3 blocks, host pool of 2
    snap = _snapshot(m)
    with pytest.raises(A.OutOfBlocks):
        m.swap_out(1)
    assert _snapshot(m) == snap and not m.is_swapped(1)
    m2 = A.BlockAllocatorModel(4, 16)
    m2.set_host_pool(4)
    m2.alloc(1, 48)      # 3 of 4 blocks
    m2.swap_out(1)       # all 4 free
    m2.alloc(2, 32)      # 2 taken: 2 left < 3
    snap = _snapshot(m2)
    with pytest.raises(A.OutOfBlocks):
        m2.swap_in(1)
    assert _snapshot(m2) == snap and m2.is_swapped(1)


def test_swapped_sequence_refuses_growth_fork_and_pack_and_frees_to_the_host_pool():
    m = A.BlockAllocatorModel(20, 16)
    m.set_host_pool(5)
    m.alloc(1, 33)
    m.swap_out(1)
    for op in (lambda: m.alloc(1, 1), lambda: m.fork(1, 2), lambda: m.pack([1], 8), lambda: m.swap_out(1)):
        with pytest.raises(A.InvalidArgument):
            op()
    with pytest.raises(A.InvalidArgument):
        m.set_host_pool(9)  # host blocks in use
    m.free(1)
    assert len(m.host_free_stack) == 5 and len(m.free_stack) == 20
    with pytest.raises(A.UnknownSeq):
        m.swap_in(1)


# ---- prefix caching ([course] §4: sharing across requests needs an
# identical prefix; §9 and §11). Pins: which blocks an identical or
# diverging prompt must get back, and the eviction order, on hand-built
# prompts.

def check_cache_invariants(m: A.BlockAllocatorModel):
    rc = m.refcnt
    refs = Counter(b for s in m.seqs() for b in m.table(s))
    assert all(rc[b] == refs.get(b, 0) for b in range(m.num_blocks))
    free = m.free_stack + m.evictable
    assert len(set(free)) == len(free)
    assert sorted(free) == [b for b in range(m.num_blocks) if rc[b] == 0]


def test_prefix_cache_reuses_exactly_the_common_full_blocks():
    bs = 4
    m = A.BlockAllocatorModel(64, bs)
    m.set_prefix_cache(True)
    a = list(range(100, 118))  # 18 tokens: 4 full blocks and 2 tokens
    slots, c = m.alloc_prompt(1, a)
    ta = m.table(1)
    assert c == 0 and slots == [ta[t // bs] * bs + t % bs for t in range(18)]
    # the same prompt: its 4 full blocks, never the partial fifth
    _, c = m.alloc_prompt(2, a)
    assert c == 16 and m.table(2)[:4] == ta[:4] and m.table(2)[4] != ta[4]
    # first difference at token 9 (block 2): blocks 0 and 1 only
    b = a[:9] + [7] + a[10:]
    _, c = m.alloc_prompt(3, b)
    assert c == 8 and m.table(3)[:2] == ta[:2] and m.table(3)[2] not in ta
    # block 1's tokens behind another block 0: nothing (the key is the whole prefix)
    _, c = m.alloc_prompt(4, [9, 9, 9, 9] + a[4:])
    assert c == 0 and not set(m.table(4)) & set(ta)
    # a prompt that ends on a block boundary reuses all of its blocks
    _, c = m.alloc_prompt(5, a[:8])
    assert c == 8 and m.table(5) == ta[:2]
    st = m.prefix_cache_stats()
    assert st["hits"] == 4 + 2 + 0 + 2 and st["misses"] == 4 + 0 + 2 + 4 + 0
    assert [m.refcnt[x] for x in ta[:4]] == [4, 4, 2, 2]
    check_cache_invariants(m)


def test_prefix_cache_evicts_the_least_recently_released_block_first():
    bs = 2
    m = A.BlockAllocatorModel(7, bs)
    m.set_prefix_cache(True)
    m.alloc_prompt(1, [1, 2, 3, 4, 5, 6])  # 3 full blocks
    m.alloc_prompt(2, [7, 8, 9, 10])       # 2 full blocks
    ta, tb = m.table(1), m.table(2)
    m.free(1)
    m.free(2)
    assert m.evictable == ta[::-1] + tb[::-1]  # a prefix leaves the cache from its end
    assert len(m.free_stack) == 2
    m.alloc(3, 6)  # 3 blocks: the 2 free ones, then ta[2] evicted
    assert ta[2] in m.table(3) and m.evictable == ta[1::-1] + tb[::-1]
    assert m.prefix_cache_stats()["evictions"] == 1
    _, c = m.alloc_prompt(4, [1, 2, 3, 4, 5, 6])
    assert c == 4 and m.table(4)[:2] == ta[:2]  # blocks 0 and 1 still cached, block 2 gone
    check_cache_invariants(m)


def test_prefix_cache_off_is_a_plain_allocation():
    tokens = list(range(37))
    on, off = A.BlockAllocatorModel(30, 8, list(range(29, -1, -1))), A.BlockAllocatorModel(30, 8, list(range(29, -1, -1)))
    ref = A.BlockAllocatorModel(30, 8, list(range(29, -1, -1)))
    off_slots, c = off.alloc_prompt(1, tokens)
    ref_slots, cows = ref.alloc(1, len(tokens))
    assert c == 0 and off_slots == ref_slots and not cows and off.table(1) == ref.table(1)
    _, c = off.alloc_prompt(2, tokens)
    assert c == 0
    on.set_prefix_cache(True)
    on.alloc_prompt(1, tokens)
    on.free(1)
    on.set_prefix_cache(False)  # forgets every registration; the blocks go back to the stack
    assert on.evictable == [] and len(on.free_stack) == 30
    _, c = on.alloc_prompt(2, tokens)
    assert c == 0
