"""Seeded synthetic decode workloads.

Every array here is drawn from ``numpy.random.default_rng`` (PCG64) with a
fixed seed; nothing is read from disk. Draw order inside one workload:
context lengths, then the order of free physical block ids, then q; K and V
of sequence ``s`` come from their own stream ``default_rng([seed, 1, s])``
(K first, then V, token-major) so that any subset of sequences can be
regenerated without drawing the rest.

Values are float32 standard normals rounded (round-to-nearest-even, by the
torch cast) to the storage type. For an fp8 cache the source values stay
bf16 and the per-tensor scale is ``amax / 448`` over that tensor (448 is the
largest finite OCP E4M3 value); quantising them is the cache write's job.

Workload shapes follow the decode batches the pages' serving setting implies:
  tiny      4 seqs, lengths {1,17,33,100}, 8/8 heads, D=64, bs=16, fp16
  gqa       64 seqs, lengths U[512,4096], 32/8 heads, D=128, bs=16, bf16
  long      8 seqs, lengths U[32768,131072], 32/8 heads, D=128, bs=16, bf16
  prefix    16 prompts x 8 samples over a shared 2048(+r)-token prefix
  mixed     256 seqs, lognormal lengths (median 1024, sigma 1) in [16,16384],
            64/8 heads, D=128, bs in {8,16,32}, bf16 or fp8 e4m3
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

E4M3_MAX = 448.0

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _pool_blocks(lengths, block_size: int, headroom: float) -> int:
    """Pool size: every sequence's blocks plus ``headroom`` spare (sizing only)."""
    used = int(sum(-(-int(n) // block_size) for n in lengths))
    return max(1, int(np.ceil(used * (1.0 + headroom))))


def _normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


@dataclasses.dataclass
class DecodeWorkload:
    """One decode batch: B sequences, one query token each.

    ``lengths[s]`` is the number of tokens in sequence s's cache when
    attention runs. ``free_order`` is the order in which a fresh allocator
    hands out physical block ids (first element first).
    """

    name: str
    seed: int
    lengths: np.ndarray  # int64 [B]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks], a permutation
    kv_dtype: str  # "f16" | "bf16" | "fp8"
    q_dtype: str  # "f16" | "bf16"
    src_dtype: str  # dtype of the K/V values handed to the cache write
    scale: float  # softmax scale, an fp32 value
    _q: Optional[torch.Tensor] = None
    _kv_cache: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = dataclasses.field(default_factory=dict)
    _scales: Optional[Tuple[float, float]] = None
    cache_kv: bool = True

    @property
    def batch(self) -> int:
        return int(len(self.lengths))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def q(self) -> torch.Tensor:
        """q [B][Hq][D] in ``q_dtype`` (CPU)."""
        if self._q is None:
            rng = np.random.default_rng([self.seed, 0])
            self._q = _normal(rng, (self.batch, self.num_q_heads, self.head_dim), self.q_dtype)
        return self._q

    def kv(self, s: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """(K, V) of sequence s, each [L_s][Hkv][D] in ``src_dtype`` (CPU), token order."""
        if s in self._kv_cache:
            return self._kv_cache[s]
        rng = np.random.default_rng([self.seed, 1, s])
        shape = (int(self.lengths[s]), self.num_kv_heads, self.head_dim)
        k = _normal(rng, shape, self.src_dtype)
        v = _normal(rng, shape, self.src_dtype)
        if self.cache_kv:
            self._kv_cache[s] = (k, v)
        return k, v

    def kv_scales(self) -> Tuple[float, float]:
        """Per-tensor (k_scale, v_scale): amax/448 for an fp8 cache, else (1, 1)."""
        if self.kv_dtype != "fp8":
            return 1.0, 1.0
        if self._scales is None:
            ka = va = 0.0
            for s in range(self.batch):
                k, v = self.kv(s)
                if k.numel():
                    ka = max(ka, float(k.float().abs().max()))
                    va = max(va, float(v.float().abs().max()))
            ks = float(np.float32(max(ka, 1e-30) / E4M3_MAX))
            vs = float(np.float32(max(va, 1e-30) / E4M3_MAX))
            self._scales = (ks, vs)
        return self._scales

    def total_tokens(self) -> int:
        return int(self.lengths.sum())


def _draw_common(rng, lengths, block_size, headroom):
    nb = _pool_blocks(lengths, block_size, headroom)
    order = rng.permutation(nb).astype(np.int32)
    return nb, order


def tiny_decode(seed: int = 4901) -> DecodeWorkload:
    """4 seqs, lengths {1,17,33,100}; 8 q heads = 8 KV heads; D=64; bs=16;
    a 64-block pool whose ids are handed out in a seeded random order; fp16
    N(0,1) values; scale 1/sqrt(64)."""
    rng = np.random.default_rng(seed)
    lengths = np.array([1, 17, 33, 100], dtype=np.int64)
    order = rng.permutation(64).astype(np.int32)
    return DecodeWorkload("tiny", seed, lengths, 8, 8, 64, 16, 64, order,
                          "f16", "f16", "f16", float(np.float32(1.0 / 8.0)))


def gqa_decode(seed: int = 4902, batch: int = 64, lo: int = 512, hi: int = 4096,
               block_size: int = 16, headroom: float = 0.10) -> DecodeWorkload:
    """64 seqs with lengths U[512,4096]; 32 q heads over 8 KV heads (group 4);
    D=128; bs=16; bf16; pool = all blocks plus 10% spare, ids shuffled."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    nb, order = _draw_common(rng, lengths, block_size, headroom)
    return DecodeWorkload("gqa", seed, lengths, 32, 8, 128, block_size, nb, order,
                          "bf16", "bf16", "bf16", float(np.float32(1.0 / np.sqrt(128.0))))


def long_context(seed: int = 4903, batch: int = 8, lo: int = 32768, hi: int = 131072,
                 headroom: float = 0.10) -> DecodeWorkload:
    """8 seqs with lengths U[32768,131072]; 32/8 heads; D=128; bs=16; bf16."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    nb, order = _draw_common(rng, lengths, 16, headroom)
    return DecodeWorkload("long", seed, lengths, 32, 8, 128, 16, nb, order,
                          "bf16", "bf16", "bf16", float(np.float32(1.0 / np.sqrt(128.0))))


def mixed_lengths(block_size: int = 16, kv_dtype: str = "bf16", seed: int = 4905,
                  batch: int = 256, headroom: float = 0.10) -> DecodeWorkload:
    """256 seqs, lengths clip(rint(exp(N(ln 1024, 1))), 16, 16384); 64 q heads
    over 8 KV heads (group 8); D=128; bs in {8,16,32}; KV bf16 or fp8 e4m3
    (per-tensor scale); q bf16. The logical K/V values do not depend on bs."""
    rng = np.random.default_rng(seed)
    raw = np.exp(rng.normal(np.log(1024.0), 1.0, size=batch))
    lengths = np.clip(np.rint(raw), 16, 16384).astype(np.int64)
    nb = _pool_blocks(lengths, block_size, headroom)
    order = np.random.default_rng([seed, 2, block_size]).permutation(nb).astype(np.int32)
    return DecodeWorkload(f"mixed-bs{block_size}-{kv_dtype}", seed, lengths, 64, 8, 128,
                          block_size, nb, order, kv_dtype, "bf16", "bf16",
                          float(np.float32(1.0 / np.sqrt(128.0))))


def random_case(seed: int, lengths, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, kv_dtype: str = "bf16", q_dtype: Optional[str] = None,
                headroom: float = 0.5, min_blocks: int = 0) -> DecodeWorkload:
    """A small randomised case with the given lengths (for parity sweeps)."""
    rng = np.random.default_rng([seed, 3])
    lengths = np.asarray(lengths, dtype=np.int64)
    nb = max(_pool_blocks(lengths, block_size, headroom), min_blocks, 1)
    order = rng.permutation(nb).astype(np.int32)
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    src = "bf16" if kv_dtype == "fp8" else kv_dtype
    return DecodeWorkload(f"random-{seed}", seed, lengths, num_q_heads, num_kv_heads, head_dim,
                          block_size, nb, order, kv_dtype, q_dtype, src,
                          float(np.float32(1.0 / np.sqrt(head_dim))))


@dataclasses.dataclass
class PrefixWorkload:
    """Parallel sampling over shared prompts.

    ``prompts`` prompts, each with ``samples`` samples. Prompt p has
    ``prefix_len[p]`` tokens shared by all its samples; sample (p, i) then
    appends ``tail_len[p][i]`` tokens of its own and finally one new token.
    """

    seed: int
    prompts: int
    samples: int
    prefix_len: np.ndarray  # int64 [prompts]
    tail_len: np.ndarray  # int64 [prompts][samples]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray
    kv_dtype: str = "bf16"
    scale: float = float(np.float32(1.0 / np.sqrt(128.0)))

    def prefix_kv(self, p: int):
        rng = np.random.default_rng([self.seed, 4, p])
        shape = (int(self.prefix_len[p]), self.num_kv_heads, self.head_dim)
        return _normal(rng, shape, self.kv_dtype), _normal(rng, shape, self.kv_dtype)

    def tail_kv(self, p: int, i: int):
        """K/V of sample (p, i)'s own tokens: its tail then the one new token."""
        rng = np.random.default_rng([self.seed, 5, p, i])
        shape = (int(self.tail_len[p, i]) + 1, self.num_kv_heads, self.head_dim)
        return _normal(rng, shape, self.kv_dtype), _normal(rng, shape, self.kv_dtype)

    def q(self) -> torch.Tensor:
        rng = np.random.default_rng([self.seed, 0])
        return _normal(rng, (self.prompts * self.samples, self.num_q_heads, self.head_dim),
                       self.kv_dtype)


def prefix_sharing(seed: int = 4904, prompts: int = 16, samples: int = 8, prefix: int = 2048,
                   partial_tail: bool = True, max_tail: int = 256,
                   headroom: float = 0.10) -> PrefixWorkload:
    """16 prompts x 8 samples; a 2048-token prefix shared by the 8 samples of
    a prompt; per-sample tails U[0,256]; then one new token per sample.

    2048 is a multiple of 16, so a 2048-token prefix ends on a full block and
    a write never lands in a shared block. With ``partial_tail`` the prefix
    is 2048 + r tokens, r ~ U[1,15] per prompt, so its last block is partial
    and shared by all samples (the copy-on-write case)."""
    rng = np.random.default_rng(seed)
    extra = rng.integers(1, 16, size=prompts) if partial_tail else np.zeros(prompts, np.int64)
    prefix_len = (prefix + extra).astype(np.int64)
    tail_len = rng.integers(0, max_tail + 1, size=(prompts, samples)).astype(np.int64)
    bs = 16
    used = 0
    for p in range(prompts):
        used += -(-int(prefix_len[p]) // bs)
        for i in range(samples):
            used += -(-(int(prefix_len[p] + tail_len[p, i]) + 1) // bs) + 1
    nb = int(np.ceil(used * (1.0 + headroom)))
    order = rng.permutation(nb).astype(np.int32)
    return PrefixWorkload(seed, prompts, samples, prefix_len, tail_len, 32, 8, 128, bs, nb, order)


def blocks_needed_for_pool(lengths, block_size: int) -> int:
    """Blocks a pool needs to hold ``lengths`` (used to size pools; sizing only)."""
    return _pool_blocks(lengths, block_size, 0.0)
