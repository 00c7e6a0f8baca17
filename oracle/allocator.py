"""Block manager model — oracle for the host allocator.

What the pages fix:
* [course] §2 "The insight": physical blocks, all of one size, form a
  pool; a sequence takes a new block only when its tokens overflow the
  blocks it holds, and hands its blocks back the moment it is done; a
  per-sequence table says which physical block holds each logical block.
  Only a sequence's last block can be partly empty.
* [note] 最小模型 ("minimal model"): growing a request only allocates one more
  block; a finished request releases its own blocks.
* [note] section "block size 是容量与 kernel 的共同参数": a request of
  ``seq_len`` tokens needs ceil(seq_len / block_size) blocks.
* [course] §2 "The bonus: block sharing (copy-on-write)" and §3 "Mental
  Model": sequences with a common prefix point at the same physical blocks
  (seq A -> [b3][b7][b1], seq B -> [b3][b9]); only the differing block is
  copied when they diverge.
* [note] section prefix sharing 的边界: sharing is governed by reference
  counts and copy-on-write happens only when a branch writes.
* [course] §4 "Hitchhiker's Guide" and §11: the pool is finite; at the
  limit the caller queues or rejects.

Readings where the pages leave the choice open:
* Which free block is handed out: a LIFO stack whose first pop returns
  ``free_order[0]``; released blocks are pushed back, the sequence's blocks
  in logical order (so its last block is the next one popped).
* Copy-on-write: when a sequence writes into its partially filled last
  block while that block's refcount is above 1, the WRITER gets a fresh
  block (popped before its growth blocks) and the pair (old, new) is
  reported for a whole-block copy; the other holders keep the old block;
  the last holder writes in place. Full blocks are never written.
* Pool exhaustion: the whole request fails and nothing changes.
* Swapping ([course] §4 and §8: under memory pressure a sequence may be
  preempted by swapping its blocks out): a host pool with its own LIFO free
  stack whose first pop is host block 0. Swap-out moves the sequence's
  blocks in logical order to freshly popped host blocks, reporting (device,
  host) pairs; each device block loses that reference (back on the device
  stack at 0). Swap-in pops fresh device blocks in logical order, reporting
  (host, device) pairs, and pushes the host blocks back in logical order.
  A swapped sequence can only be swapped in, freed (its host blocks go back
  on the host stack) or queried. Both are all-or-nothing.
* Prefix caching ([course] §4: sharing across users needs an identical
  prefix and prefix caching enabled; §11: enable it for common prompts):
  with the cache on, each full block a prompt fills is registered under its
  whole token prefix (here the exact prefix itself is the key). A prompt
  reuses registered blocks for its leading full blocks while the prefixes
  match; its other full blocks are registered unless their prefix already
  is. A registered block whose refcount drops to 0 keeps its data in an
  evictable LRU, which a released sequence's registered blocks enter in
  reverse logical order; unregistered ones go onto the free stack in
  logical order as before. Every allocation pops the free stack first, then
  evicts (and unregisters) the LRU's oldest block. Turning the cache off
  forgets all registrations and moves the LRU, oldest first, onto the free
  stack.
* A batch of allocations is all-or-nothing and may not name a sequence
  twice; requests are applied in the given order.

This model applies a request to a copy of the state and commits only if it
completes — all-or-nothing by construction.
"""
from __future__ import annotations

import copy
from typing import Dict, List, Sequence, Tuple


class AllocError(Exception):
    code = "error"


class OutOfBlocks(AllocError):
    code = "out_of_blocks"


class UnknownSeq(AllocError):
    code = "unknown_seq"


class SeqExists(AllocError):
    code = "seq_exists"


class InvalidArgument(AllocError):
    code = "invalid_argument"


def blocks_for(length: int, block_size: int) -> int:
    """ceil(length / block_size) ([note] block size section)."""
    return -(-int(length) // int(block_size))


def capacity(pool_blocks: int, context_len: int, block_size: int) -> int:
    """Concurrent sequences of ``context_len`` tokens a pool holds:
    pool_blocks // blocks_per_seq ([course] §4 and §11: seqs ~ pool
    blocks / blocks per sequence)."""
    return int(pool_blocks) // blocks_for(context_len, block_size)


def naive_waste(used_tokens: int, reserved_tokens: int) -> float:
    """Fraction of a contiguous max-context reservation left unused
    ([course] §2 primer, internal fragmentation)."""
    return 1.0 - used_tokens / reserved_tokens


def paged_waste_tokens(length: int, block_size: int) -> int:
    """Unused slots of a paged sequence: the tail of its last block."""
    return blocks_for(length, block_size) * block_size - int(length)


class _State:
    def __init__(self, num_blocks: int, free_order: Sequence[int]):
        self.stack: List[int] = list(reversed([int(b) for b in free_order]))  # top = end
        self.refcnt: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.cow_copies = 0
        self.forks = 0
        self.host_stack: List[int] = []  # top = end
        self.num_host = 0
        self.swapped: set = set()
        self.swap_outs = 0
        self.swap_ins = 0
        self.prefix_cache = False
        self.cached: Dict[tuple, int] = {}  # token prefix -> block
        self.key_of: Dict[int, tuple] = {}   # block -> its registered prefix
        self.lru: List[int] = []             # front = evicted next
        self.hits = 0
        self.misses = 0
        self.evictions = 0


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArgument("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.st = _State(num_blocks, order)

    # -- queries -------------------------------------------------------
    @property
    def refcnt(self) -> List[int]:
        return list(self.st.refcnt)

    @property
    def free_stack(self) -> List[int]:
        """Free block ids from the bottom of the stack to its top."""
        return list(self.st.stack)

    def table(self, seq: int) -> List[int]:
        if seq not in self.st.tables:
            raise UnknownSeq(seq)
        return list(self.st.tables[seq])

    def length(self, seq: int) -> int:
        if seq not in self.st.lens:
            raise UnknownSeq(seq)
        return self.st.lens[seq]

    def seqs(self) -> List[int]:
        return list(self.st.tables)

    @property
    def host_free_stack(self) -> List[int]:
        return list(self.st.host_stack)

    def is_swapped(self, seq: int) -> bool:
        if seq not in self.st.tables:
            raise UnknownSeq(seq)
        return seq in self.st.swapped

    def host_stats(self) -> dict:
        return dict(num_host_blocks=self.st.num_host, num_host_free=len(self.st.host_stack),
                    num_swapped=len(self.st.swapped), swap_outs=self.st.swap_outs, swap_ins=self.st.swap_ins)

    def stats(self) -> dict:
        rc = self.st.refcnt
        return dict(num_blocks=self.num_blocks, num_free=len(self.st.stack),
                    num_used=sum(1 for r in rc if r > 0), num_shared=sum(1 for r in rc if r > 1),
                    cow_copies=self.st.cow_copies, forks=self.st.forks,
                    num_seqs=len(self.st.tables))

    # -- operations ----------------------------------------------------
    @staticmethod
    def _pop(st: _State) -> int:
        if st.stack:
            return st.stack.pop()
        if not st.lru:
            raise OutOfBlocks("pool exhausted")
        blk = st.lru.pop(0)
        del st.cached[st.key_of.pop(blk)]
        st.evictions += 1
        return blk

    @staticmethod
    def _release(st: _State, dead: List[int]) -> None:
        """Blocks (logical order) whose refcount just reached 0."""
        st.stack.extend(b for b in dead if b not in st.key_of)
        st.lru.extend(b for b in reversed(dead) if b in st.key_of)

    def _grow(self, st: _State, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        bs = self.block_size
        if n < 0:
            raise InvalidArgument("negative token count")
        if seq not in st.tables:
            st.tables[seq] = []
            st.lens[seq] = 0
        if seq in st.swapped:
            raise InvalidArgument("sequence is swapped out")
        table = st.tables[seq]
        length = st.lens[seq]
        cows: List[Tuple[int, int]] = []
        if n > 0 and length % bs != 0 and st.refcnt[table[-1]] > 1:
            old = table[-1]
            new = self._pop(st)
            st.refcnt[old] -= 1
            st.refcnt[new] = 1
            table[-1] = new
            cows.append((old, new))
            st.cow_copies += 1
        while len(table) < blocks_for(length + n, bs):
            blk = self._pop(st)
            st.refcnt[blk] = 1
            table.append(blk)
        slots = [table[t // bs] * bs + t % bs for t in range(length, length + n)]
        st.lens[seq] = length + n
        return slots, cows

    def alloc(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Room for ``n`` more tokens of ``seq`` (created if unknown).
        Returns (slots of the new tokens, copy-on-write pairs)."""
        return self.alloc_batch([seq], [n])

    def alloc_batch(self, seqs: Sequence[int], ns: Sequence[int]):
        if len(seqs) != len(ns):
            raise InvalidArgument("length mismatch")
        if len(set(seqs)) != len(seqs):
            raise InvalidArgument("a sequence appears twice in one batch")
        st = copy.deepcopy(self.st)
        slots: List[int] = []
        cows: List[Tuple[int, int]] = []
        for seq, n in zip(seqs, ns):
            s_slots, s_cows = self._grow(st, seq, int(n))
            slots += s_slots
            cows += s_cows
        self.st = st
        return slots, cows

    def fork(self, parent: int, child: int) -> None:
        """``child`` starts as a copy of ``parent``'s table; every block gains
        one reference."""
        if child in self.st.tables:
            raise SeqExists(child)
        if parent not in self.st.tables:
            raise UnknownSeq(parent)
        if parent in self.st.swapped:
            raise InvalidArgument("sequence is swapped out")
        self.st.tables[child] = list(self.st.tables[parent])
        self.st.lens[child] = self.st.lens[parent]
        for blk in self.st.tables[child]:
            self.st.refcnt[blk] += 1
        self.st.forks += 1

    def free(self, seq: int) -> None:
        """Release ``seq``: each block (logical order) loses one reference and
        goes back on the free stack when none is left."""
        if seq not in self.st.tables:
            raise UnknownSeq(seq)
        if seq in self.st.swapped:
            self.st.host_stack.extend(self.st.tables.pop(seq))
            self.st.swapped.discard(seq)
        else:
            dead = []
            for blk in self.st.tables.pop(seq):
                self.st.refcnt[blk] -= 1
                if self.st.refcnt[blk] == 0:
                    dead.append(blk)
            self._release(self.st, dead)
        del self.st.lens[seq]

    def set_host_pool(self, num_host_blocks: int) -> None:
        if num_host_blocks < 0:
            raise InvalidArgument("negative host pool")
        if len(self.st.host_stack) != self.st.num_host:
            raise InvalidArgument("host blocks in use")
        self.st.num_host = int(num_host_blocks)
        self.st.host_stack = list(range(num_host_blocks - 1, -1, -1))

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """Move ``seq``'s blocks to the host pool; (device, host) pairs."""
        if seq not in self.st.tables:
            raise UnknownSeq(seq)
        if seq in self.st.swapped:
            raise InvalidArgument("already swapped out")
        table = self.st.tables[seq]
        if len(table) > len(self.st.host_stack):
            raise OutOfBlocks("host pool exhausted")
        pairs = []
        dead = []
        for i, blk in enumerate(table):
            h = self.st.host_stack.pop()
            pairs.append((blk, h))
            table[i] = h
            self.st.refcnt[blk] -= 1
            if self.st.refcnt[blk] == 0:
                dead.append(blk)
        self._release(self.st, dead)
        self.st.swapped.add(seq)
        self.st.swap_outs += 1
        return pairs

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """Bring ``seq``'s blocks back into fresh device blocks; (host,
        device) pairs."""
        if seq not in self.st.tables:
            raise UnknownSeq(seq)
        if seq not in self.st.swapped:
            raise InvalidArgument("not swapped out")
        table = self.st.tables[seq]
        if len(table) > len(self.st.stack) + len(self.st.lru):
            raise OutOfBlocks("pool exhausted")
        pairs = []
        for i, h in enumerate(table):
            blk = self._pop(self.st)
            self.st.refcnt[blk] = 1
            pairs.append((h, blk))
            table[i] = blk
            self.st.host_stack.append(h)
        self.st.swapped.discard(seq)
        self.st.swap_ins += 1
        return pairs

    # -- prefix caching -------------------------------------------------
    def set_prefix_cache(self, enable: bool) -> None:
        if not enable and self.st.prefix_cache:
            self.st.stack.extend(self.st.lru)
            self.st.lru = []
            self.st.cached = {}
            self.st.key_of = {}
        self.st.prefix_cache = bool(enable)

    def alloc_prompt(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """New sequence ``seq`` for a prompt; (slots of all tokens, tokens
        covered by reused cached blocks)."""
        if seq in self.st.tables:
            raise SeqExists(seq)
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        nfull = n // bs
        st = copy.deepcopy(self.st)
        hit = []
        if st.prefix_cache:
            for i in range(nfull):
                key = tuple(tokens[: (i + 1) * bs])
                if key not in st.cached:
                    break
                hit.append(st.cached[key])
        need = blocks_for(n, bs) - len(hit)
        if need > len(st.stack) + len(st.lru) - sum(1 for b in hit if b in st.lru):
            raise OutOfBlocks("pool exhausted")
        table = []
        for b in hit:
            if b in st.lru:
                st.lru.remove(b)
            st.refcnt[b] += 1
            table.append(b)
        for i in range(len(hit), blocks_for(n, bs)):
            blk = self._pop(st)
            st.refcnt[blk] = 1
            table.append(blk)
            key = tuple(tokens[: (i + 1) * bs])
            if st.prefix_cache and i < nfull and key not in st.cached:
                st.cached[key] = blk
                st.key_of[blk] = key
        st.tables[seq] = table
        st.lens[seq] = n
        if st.prefix_cache:
            st.hits += len(hit)
            st.misses += nfull - len(hit)
        self.st = st
        return [table[t // bs] * bs + t % bs for t in range(n)], len(hit) * bs

    def prefix_cache_stats(self) -> dict:
        return dict(num_cached_blocks=len(self.st.cached), num_evictable=len(self.st.lru), hits=self.st.hits,
                    misses=self.st.misses, evictions=self.st.evictions)

    @property
    def evictable(self) -> List[int]:
        return list(self.st.lru)

    def pack(self, seqs: Sequence[int], max_blocks: int, pad: int = -1):
        """(tables [n][max_blocks] padded with ``pad``, context lengths [n])."""
        tables, lens = [], []
        for seq in seqs:
            t = self.table(seq)
            if seq in self.st.swapped:
                raise InvalidArgument("sequence is swapped out")
            if len(t) > max_blocks:
                raise InvalidArgument("table wider than max_blocks")
            tables.append(t + [pad] * (max_blocks - len(t)))
            lens.append(self.length(seq))
        return tables, lens
