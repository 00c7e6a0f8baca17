// Shared definitions of the paged decode kernels (gfx950).
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
//
// What every decode kernel computes ([course] §2 "The insight": keys and
// values are fetched through the block table as attention runs; [note]
// 最小模型: blocks are visited in logical token order; [note] "why it works":
// the result is ordinary attention): for the G query heads h of KV head g
// and the tokens t of one piece of a sequence,
//     z'_t = log2(e) * scale * q_h . K_t,   m' >= max z',
//     l = sum_t 2^(z'_t - m'),   o_h = sum_t 2^(z'_t - m') V_t / l
// and the pieces of one sequence are merged by their log-sum-exp.
//
// Rules every kernel follows:
//  * the context length is clamped to [0, max_context_len]; a sequence of
//    length 0 gets a zero output;
//  * block ids: table entries past ceil(L / block_size), or outside the pool,
//    read block 0 (no access leaves the pool; those tokens are masked);
//  * the running max m' moves only when a tile exceeds it by more than 2^8
//    (then the accumulators are rescaled), which keeps every weight below
//    2^8 and makes rescales rare;
//  * masking uses selects (never multiply-by-zero), so NaN in unused cache
//    slots cannot leak into the result.
#pragma once

#include <hip/hip_runtime.h>

#include "decode_dispatch.h"
#include "device_common.h"

namespace pa {

struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  void* out;
  float* part_m;  // [B][Hq][num_partitions]   reference max (log2 domain)
  float* part_l;  // [B][Hq][num_partitions]   sum of weights
  float* part_o;  // [B][Hq][num_partitions][D] normalised partial output
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t block_stride;  // elements
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t len_cap;         // max_context_len (<= max_blocks * block_size)
  int32_t partition_size;  // tokens per partition; 0 = whole context
  int32_t num_partitions;  // grid.x
  int32_t out_dtype;       // 0 f16, 1 bf16, 2 f32
  float qk_scale_log2;     // scale * k_scale * log2(e)
  float v_scale;           // 1 for 16-bit pools
  // pa_decode_shared: tokens at the start of each sequence computed per
  // group (partitions below it are skipped here); nullptr otherwise
  const int32_t* shared_len;
};

template <typename KV, int D, int BS, int G>
struct DecodeCfg {
  static constexpr int kB = KV::kBytes;
  static constexpr int kKSteps = D / 32;                        // MFMAs per 16-token tile
  static constexpr int kKLoads = kB == 2 ? kKSteps : kKSteps / 2;  // 16-byte K loads per lane per tile
  static constexpr int kChunk = 64 * BS - (BS > 16 ? BS : 0);   // tokens whose block ids fit one VGPR
  static constexpr float kSlack = 8.0f;                         // log2 headroom before a rescale
  static_assert(D % 64 == 0, "head_dim must be a multiple of 64");
  static_assert(G >= 1 && G <= 8, "group size 1..8");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size 8, 16 or 32");
  static_assert(kChunk % 16 == 0, "chunks are whole tiles");
};

// Head-dim offset of the 8 elements lane group j feeds to QK MFMA step i.
// Any assignment works as long as q and K use the same one. 16-bit: 32i + 8j
// (each load instruction reads 64 contiguous bytes of every token row);
// fp8: one 16-byte load of 16 dims serves steps 2a and 2a+1.
template <int KVBytes>
__device__ __forceinline__ constexpr int qk_dim(int i, int j) {
  return KVBytes == 2 ? 32 * i + 8 * j : 64 * (i / 2) + 16 * j + 8 * (i % 2);
}

// LDS written by some lanes of a wave and read by others: LDS operations of
// one wave complete in order; this keeps the compiler from reordering them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
