// Cache write (reshape_and_cache) and whole-block copy (copy-on-write) for
// the paged KV pool, gfx950.
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
//
// Write: [course] §2 primer (each decode step adds one token's K/V) and §2
// "The insight" (each block holds K[BLOCK][HEADS][HEAD_DIM] and V likewise):
// token i's rows land in block slot/bs, row slot%bs.
// Copy: [course] §2 "The bonus: block sharing (copy-on-write)" and [note]
// prefix sharing section: only the block a branch writes into is copied.
//
// Both kernels are plain HBM streams: every thread moves 16-byte vectors,
// consecutive threads touch consecutive 16-byte chunks of one row / block.
#include <hip/hip_runtime.h>

#include <vector>

#include "device_common.h"
#include "internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// One work item = 8 consecutive elements of one token's K or V row.
// Items are ordered (token, K|V, chunk) so a wavefront covers contiguous
// bytes of one row.
template <typename Src, bool kToFp8>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new, const int64_t* __restrict__ slots,
    int64_t total_items, int32_t chunks_per_row, int32_t row_elems, void* __restrict__ k_pool,
    void* __restrict__ v_pool, int64_t block_stride, int32_t block_size, int64_t num_slots, float k_inv,
    float v_inv, int32_t v_dim_major) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (item >= total_items) return;
  const int64_t per_token = 2 * static_cast<int64_t>(chunks_per_row);
  const int64_t token = item / per_token;
  const int32_t rem = static_cast<int32_t>(item - token * per_token);
  const bool is_v = rem >= chunks_per_row;
  const int32_t chunk = is_v ? rem - chunks_per_row : rem;
  const int64_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t dst_elem = blk * block_stride + off * row_elems + static_cast<int64_t>(chunk) * 8;
  const int64_t src_elem = token * row_elems + static_cast<int64_t>(chunk) * 8;
  const void* src = is_v ? v_new : k_new;
  void* dst = is_v ? v_pool : k_pool;
  // dim-major V: element (h*D + d) of the row goes to block offset (h*D + d) * bs + t
  const bool scatter = is_v && v_dim_major;
  const int64_t sc_elem = blk * block_stride + static_cast<int64_t>(chunk) * 8 * block_size + off;

  if constexpr (!kToFp8) {
    // same 16-bit dtype: move the bits
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + src_elem);
    if (scatter) {
      uint16_t* d = static_cast<uint16_t*>(dst) + sc_elem;
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e * block_size] = static_cast<uint16_t>(v[e / 2] >> (16 * (e % 2)));
    } else {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + dst_elem) = v;
    }
  } else {
    float x[8];
    if constexpr (Src::kBytes == 4) {
      const float* p = static_cast<const float*>(src) + src_elem;
      const f32x4 a = *reinterpret_cast<const f32x4*>(p);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + src_elem);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (Src::kIsBf16) {
          x[2 * i] = bf16_lo(w[i]);
          x[2 * i + 1] = bf16_hi(w[i]);
        } else {
          x[2 * i] = f16_lo(w[i]);
          x[2 * i + 1] = f16_hi(w[i]);
        }
      }
    }
    const float inv = is_v ? v_inv : k_inv;
    if (scatter) {
      uint8_t* d = static_cast<uint8_t*>(dst) + sc_elem;
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i * block_size] = static_cast<uint8_t>(f32_to_e4m3(x[i] * inv));
    } else {
      u32x2 packed = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) packed[i / 4] |= f32_to_e4m3(x[i] * inv) << (8 * (i % 4));
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(dst) + dst_elem) = packed;
    }
  }
}

struct SrcF16 {
  static constexpr int kBytes = 2;
  static constexpr bool kIsBf16 = false;
};
struct SrcBF16 {
  static constexpr int kBytes = 2;
  static constexpr bool kIsBf16 = true;
};
struct SrcF32 {
  static constexpr int kBytes = 4;
  static constexpr bool kIsBf16 = false;
};

// Copy whole blocks: blockIdx.y selects K (0) or V (1), blockIdx.x the pair.
// Each thread moves kUnroll 16-byte vectors per round (loads first, then
// stores) so several loads are in flight.
constexpr int kCopyUnroll = 4;

// Source and destination pools may differ (pa_copy_blocks_between, e.g. a
// device pool and a pinned host pool, which the device reads and writes
// directly); they have the same block geometry, possibly other strides.
struct CopyPools {
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  int64_t src_stride_bytes, dst_stride_bytes;
  int32_t src_blocks, dst_blocks;
  int32_t block_vecs;  // 16-byte vectors of K (and of V) per block
};

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const int32_t* __restrict__ pairs, const CopyPools c) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= c.src_blocks || dst < 0 || dst >= c.dst_blocks) return;
  const u32x4* s = reinterpret_cast<const u32x4*>((blockIdx.y == 0 ? c.src_k : c.src_v) + src * c.src_stride_bytes);
  u32x4* d = reinterpret_cast<u32x4*>((blockIdx.y == 0 ? c.dst_k : c.dst_v) + dst * c.dst_stride_bytes);
  const int32_t block_vecs = c.block_vecs;
  for (int32_t i0 = threadIdx.x; i0 < block_vecs; i0 += kThreads * kCopyUnroll) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int32_t i = i0 + u * kThreads;
      if (i < block_vecs) v[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int32_t i = i0 + u * kThreads;
      if (i < block_vecs) d[i] = v[u];
    }
  }
}

int elem_bytes(pa_dtype t) {
  switch (t) {
    case PA_F16:
    case PA_BF16: return 2;
    case PA_F32: return 4;
    case PA_FP8_E4M3: return 1;
  }
  return 0;
}

// whole-block copies src[pairs[i][0]] -> dst[pairs[i][1]], K and V
// (descriptors validated by the caller)
pa_status launch_copy(const pa_kv_cache* dst, const pa_kv_cache* src, const int32_t* pairs, int32_t N,
                      hipStream_t stream) {
  const int eb = elem_bytes(src->dtype);
  const int64_t block_bytes = static_cast<int64_t>(src->block_size) * src->num_kv_heads * src->head_dim * eb;
  if (block_bytes / 16 > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "block too large");
  CopyPools c{};
  c.src_k = static_cast<const char*>(src->k);
  c.src_v = static_cast<const char*>(src->v);
  c.dst_k = static_cast<char*>(dst->k);
  c.dst_v = static_cast<char*>(dst->v);
  c.src_stride_bytes = src->block_stride * eb;
  c.dst_stride_bytes = dst->block_stride * eb;
  c.src_blocks = src->num_blocks;
  c.dst_blocks = dst->num_blocks;
  c.block_vecs = static_cast<int32_t>(block_bytes / 16);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(N), 2), dim3(kThreads), 0, stream, pairs, c);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "copy_blocks launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

// Shared with the decode entry point: checks that the pool descriptor is
// well formed (host-side only, nothing launched).
pa_status validate_cache(const pa_kv_cache* c) {
  if (c == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (c->k == nullptr || c->v == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "cache k or v is NULL");
  if (c->v_layout != PA_LAYOUT_TOKEN_MAJOR && c->v_layout != PA_LAYOUT_DIM_MAJOR)
    return fail(PA_ERR_INVALID_ARGUMENT, "v_layout %d is not a pa_layout", (int)c->v_layout);
  if (c->dtype != PA_F16 && c->dtype != PA_BF16 && c->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "pool dtype %d: pools hold F16, BF16 or FP8_E4M3", (int)c->dtype);
  if (c->num_blocks <= 0 || c->block_size <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pool dims must be positive (blocks %d, bs %d, heads %d, dim %d)",
                c->num_blocks, c->block_size, c->num_kv_heads, c->head_dim);
  if (c->head_dim % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 16", c->head_dim);
  const int64_t block_elems = static_cast<int64_t>(c->block_size) * c->num_kv_heads * c->head_dim;
  if (c->block_stride < block_elems)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_stride %lld < block_size*heads*head_dim = %lld",
                (long long)c->block_stride, (long long)block_elems);
  const int eb = elem_bytes(c->dtype);
  if ((c->block_stride * eb) % 16 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_stride * element size must be a multiple of 16 bytes");
  if ((reinterpret_cast<uintptr_t>(c->k) | reinterpret_cast<uintptr_t>(c->v)) % 16 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "cache k and v must be 16-byte aligned");
  if (c->dtype == PA_FP8_E4M3 && !(c->k_scale > 0.f && c->v_scale > 0.f && c->k_scale < 3.4e38f &&
                                   c->v_scale < 3.4e38f))
    return fail(PA_ERR_INVALID_ARGUMENT, "fp8 pools need finite positive k_scale and v_scale");
  return PA_OK;
}

}  // namespace pa

using pa::fail;

extern "C" {

pa_status pa_reshape_and_cache(const pa_kv_cache* cache, const void* k_new, const void* v_new, pa_dtype src_dtype,
                               const int64_t* slot_mapping, int32_t T, void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (T < 0) return fail(PA_ERR_INVALID_ARGUMENT, "T = %d is negative", T);
  if (T == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "k_new, v_new or slot_mapping is NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(slot_mapping) % 8 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "k_new / v_new must be 16-byte aligned, slot_mapping 8-byte aligned");
  const bool to_fp8 = cache->dtype == PA_FP8_E4M3;
  if (!to_fp8 && src_dtype != cache->dtype)
    return fail(PA_ERR_UNSUPPORTED, "a %s pool takes %s sources (got dtype %d)",
                cache->dtype == PA_F16 ? "F16" : "BF16", cache->dtype == PA_F16 ? "F16" : "BF16", (int)src_dtype);
  if (to_fp8 && src_dtype != PA_F16 && src_dtype != PA_BF16 && src_dtype != PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "an FP8 pool takes F16, BF16 or F32 sources (got dtype %d)", (int)src_dtype);
  const int32_t row_elems = cache->num_kv_heads * cache->head_dim;
  const int64_t num_slots = static_cast<int64_t>(cache->num_blocks) * cache->block_size;
  if (pa::debug_enabled()) {
    std::vector<int64_t> h(T);
    if (hipMemcpy(h.data(), slot_mapping, sizeof(int64_t) * T, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading slot_mapping failed");
    for (int32_t i = 0; i < T; ++i)
      if (h[i] >= num_slots)
        return fail(PA_ERR_INVALID_ARGUMENT, "slot_mapping[%d] = %lld >= num_blocks*block_size = %lld", i,
                    (long long)h[i], (long long)num_slots);
  }
  const int32_t chunks = row_elems / 8;
  const int64_t items = static_cast<int64_t>(T) * 2 * chunks;
  const int64_t grid = (items + pa::kThreads - 1) / pa::kThreads;
  if (grid > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "T = %d too large for one launch", T);
  const float kinv = to_fp8 ? 1.0f / cache->k_scale : 1.0f;
  const float vinv = to_fp8 ? 1.0f / cache->v_scale : 1.0f;
  hipStream_t s = static_cast<hipStream_t>(stream);
#define PA_LAUNCH_RC(SRC, FP8)                                                                                 \
  hipLaunchKernelGGL((pa::reshape_and_cache_kernel<SRC, FP8>), dim3(static_cast<uint32_t>(grid)),            \
                     dim3(pa::kThreads), 0, s, k_new, v_new, slot_mapping, items, chunks, row_elems, cache->k, \
                     cache->v, cache->block_stride, cache->block_size, num_slots, kinv, vinv,  \
                     cache->v_layout == PA_LAYOUT_DIM_MAJOR ? 1 : 0)
  if (!to_fp8) {
    PA_LAUNCH_RC(pa::SrcF16, false);
  } else if (src_dtype == PA_F32) {
    PA_LAUNCH_RC(pa::SrcF32, true);
  } else if (src_dtype == PA_BF16) {
    PA_LAUNCH_RC(pa::SrcBF16, true);
  } else {
    PA_LAUNCH_RC(pa::SrcF16, true);
  }
#undef PA_LAUNCH_RC
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "reshape_and_cache launch: %s", hipGetErrorString(e));
  return PA_OK;
}

pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* pairs, int32_t N, void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (N < 0) return fail(PA_ERR_INVALID_ARGUMENT, "N = %d is negative", N);
  if (N == 0) return PA_OK;
  if (pairs == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "pairs is NULL");
  if (pa::debug_enabled()) {
    std::vector<int32_t> h(2 * static_cast<size_t>(N));
    if (hipMemcpy(h.data(), pairs, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading pairs failed");
    std::vector<char> is_dst(cache->num_blocks, 0), is_src(cache->num_blocks, 0);
    for (int32_t i = 0; i < N; ++i) {
      const int32_t a = h[2 * i], b = h[2 * i + 1];
      if (a < 0 || a >= cache->num_blocks || b < 0 || b >= cache->num_blocks)
        return fail(PA_ERR_INVALID_ARGUMENT, "pair %d = (%d, %d) outside [0, %d)", i, a, b, cache->num_blocks);
      if (is_dst[b]) return fail(PA_ERR_INVALID_ARGUMENT, "block %d is the destination of two pairs", b);
      is_dst[b] = 1;
      is_src[a] = 1;
    }
    for (int32_t b = 0; b < cache->num_blocks; ++b)
      if (is_dst[b] && is_src[b]) return fail(PA_ERR_INVALID_ARGUMENT, "block %d is both a source and a destination", b);
  }
  return pa::launch_copy(cache, cache, pairs, N, static_cast<hipStream_t>(stream));
}

pa_status pa_copy_blocks_between(const pa_kv_cache* dst, const pa_kv_cache* src, const int32_t* pairs, int32_t N,
                                 void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(dst);
  if (st != PA_OK) return st;
  st = pa::validate_cache(src);
  if (st != PA_OK) return st;
  if (dst->block_size != src->block_size || dst->num_kv_heads != src->num_kv_heads ||
      dst->head_dim != src->head_dim || dst->dtype != src->dtype || dst->v_layout != src->v_layout)
    return fail(PA_ERR_INVALID_ARGUMENT, "the two pools differ in block size, heads, head_dim, dtype or V layout");
  if (N < 0) return fail(PA_ERR_INVALID_ARGUMENT, "N = %d is negative", N);
  if (N == 0) return PA_OK;
  if (pairs == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "pairs is NULL");
  if (pa::debug_enabled()) {
    std::vector<int32_t> h(2 * static_cast<size_t>(N));
    if (hipMemcpy(h.data(), pairs, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading pairs failed");
    std::vector<char> is_dst(dst->num_blocks, 0);
    for (int32_t i = 0; i < N; ++i) {
      const int32_t a = h[2 * i], b = h[2 * i + 1];
      if (a < 0 || a >= src->num_blocks || b < 0 || b >= dst->num_blocks)
        return fail(PA_ERR_INVALID_ARGUMENT, "pair %d = (%d, %d) outside the pools", i, a, b);
      if (is_dst[b]) return fail(PA_ERR_INVALID_ARGUMENT, "block %d is the destination of two pairs", b);
      is_dst[b] = 1;
    }
  }
  return pa::launch_copy(dst, src, pairs, N, static_cast<hipStream_t>(stream));
}

}  // extern "C"
