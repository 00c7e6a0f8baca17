"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 model of what the paged decode path
computes. It exists to check the HIP library; it is not part of it. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The HIP library never calls it, and it shares no
code, table or constant with the HIP sources.

Pages cited (by title and section):
  [course] "PagedAttention" — Phase 7 · Document 04 · Production Serving
           (ai-engineer-zt0.pages.dev, llm-mastery/07-production-serving)
  [note]   "PagedAttention" — an LLM study note, written in Chinese
           (lux-666-github-io.pages.dev, 2026/07/13)
  [intent] "Building Intent-Aware Configuration for LLM Serving"
           (marcusacosta.dev)

Modules:
  attention  — contiguous reconstruction through the block table and naive
               single-query softmax attention (fp64)
  cache_ops  — the slot-mapped cache write and the whole-block copy, on
               the pools' storage bits
  fp8        — OCP E4M3 (e4m3fn) decode table and round-to-nearest-even
               saturating encoder, from the format definition
  allocator  — the block manager: free stack, refcounts, on-demand growth,
               fork, copy-on-write, release

Parity pins: every function, and every storage-format branch of the
attention decoder (f16, bf16, fp8), is checked in ``tests/test_oracle_*.py``
against something other than the oracle itself: torch's
scaled_dot_product_attention and float8 cast, closed forms, values worked
out by hand, the pages' worked examples and invariants; planted mistakes
(``test_planted_mistake_is_caught``) show the pins reject plausible bugs.
"""
from . import allocator, attention, cache_ops, fp8  # noqa: F401
