// pa_decode entry point: argument validation, kernel selection, and the
// log-sum-exp merge of context partitions.
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving.
// The pages do not describe a split of long contexts; splitting a context
// into partitions and merging them is exact because softmax attention over
// a sequence equals the weighted merge of attention over consecutive parts:
//   out = sum_p w_p o_p / sum_p w_p,   w_p = l_p * 2^(m_p - max_q m_q)
// where o_p is partition p's normalised output, l_p its sum of weights and
// m_p its running max (log2 domain). [course] §9 "Observations from Real
// Systems" notes long-context serving is gated by blocks per sequence; the
// partitions keep one long sequence from serialising on one workgroup.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "decode_kernel.h"
#include "device_common.h"
#include "internal.h"

namespace pa {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct ReduceParams {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  void* out;
  const int32_t* context_lens;
  int32_t len_cap;
  int32_t partition_size;
  int32_t num_partitions;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t out_dtype;
};

// grid = (Hq, B); one thread per head-dim element. Sums run over partitions
// in index order, so the result does not depend on scheduling.
__global__ __launch_bounds__(128) void decode_reduce_kernel(const ReduceParams p) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int L = p.context_lens[s];
  L = L < p.len_cap ? L : p.len_cap;
  L = L > 0 ? L : 0;
  const int np = (L + p.partition_size - 1) / p.partition_size;
  if (np <= 1) return;  // written directly by the partition kernel
  const int64_t row = static_cast<int64_t>(s) * p.num_q_heads + h;
  const float* m = p.part_m + row * p.num_partitions;
  const float* l = p.part_l + row * p.num_partitions;
  const float* o = p.part_o + row * p.num_partitions * p.head_dim;
  float mmax = -INFINITY;
  for (int i = 0; i < np; ++i) mmax = fmaxf(mmax, m[i]);
  for (int d = threadIdx.x; d < p.head_dim; d += blockDim.x) {
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int i = 0; i < np; ++i) {
      const float w = l[i] * __builtin_amdgcn_exp2f(m[i] - mmax);
      den += w;
      num = fmaf(w, o[static_cast<int64_t>(i) * p.head_dim + d], num);
    }
    store_out(p.out, row * p.head_dim + d, p.out_dtype, num / den);
  }
}

int out_code(pa_dtype t) { return t == PA_F32 ? 2 : (t == PA_BF16 ? 1 : 0); }

int64_t partitions_for(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || max_context_len <= partition_size) return 1;
  return (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
}

size_t workspace_bytes_for(int64_t B, int64_t Hq, int64_t D, int64_t P) {
  if (P <= 1) return 0;
  const size_t rows = static_cast<size_t>(B * Hq * P);
  return 2 * align_up(rows * sizeof(float)) + align_up(rows * D * sizeof(float));
}

}  // namespace
}  // namespace pa

using pa::fail;

extern "C" {

size_t pa_decode_workspace_size(int32_t B, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                int32_t partition_size) {
  if (B <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  return pa::workspace_bytes_for(B, num_q_heads, head_dim, pa::partitions_for(max_context_len, partition_size));
}

pa_status pa_decode(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                    int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (B < 0) return fail(PA_ERR_INVALID_ARGUMENT, "B = %d is negative", B);
  if (B == 0) return PA_OK;
  if (out == nullptr || q == nullptr || block_tables == nullptr || context_lens == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "out, q, block_tables or context_lens is NULL");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q)) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(context_lens)) % 4 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned, tables and lengths 4-byte aligned");
  const int32_t hkv = cache->num_kv_heads;
  const int32_t D = cache->head_dim;
  const int32_t bs = cache->block_size;
  if (num_q_heads <= 0 || num_q_heads % hkv != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, hkv);
  const int32_t G = num_q_heads / hkv;
  if (out_dtype != PA_F16 && out_dtype != PA_BF16 && out_dtype != PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "out_dtype %d: outputs are F16, BF16 or F32", (int)out_dtype);
  const bool dtype_ok = (cache->dtype == PA_F16 && q_dtype == PA_F16) ||
                        (cache->dtype == PA_BF16 && q_dtype == PA_BF16) ||
                        (cache->dtype == PA_FP8_E4M3 && q_dtype == PA_BF16);
  if (!dtype_ok)
    return fail(PA_ERR_UNSUPPORTED, "pool dtype %d with q dtype %d: supported are F16/F16, BF16/BF16, FP8/BF16",
                (int)cache->dtype, (int)q_dtype);
  const pa::DecodeLaunch launch = pa::find_decode(cache->dtype, cache->v_layout, D, bs, G);
  if (launch == nullptr)
    return fail(PA_ERR_UNSUPPORTED,
                "no decode kernel for head_dim %d, block_size %d, group %d (built: head_dim 64/128, block_size "
                "8/16/32, group 1/2/4/8)",
                D, bs, G);
  if (max_blocks <= 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks %d must be positive, max_context_len %d non-negative",
                max_blocks, max_context_len);
  if (static_cast<int64_t>(max_blocks) * bs > 0x7fffffff)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks * block_size exceeds INT32_MAX");
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks) * bs)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len %d > max_blocks %d * block_size %d", max_context_len,
                max_blocks, bs);
  if (partition_size < 0 || partition_size % 16 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "partition_size %d must be 0 or a positive multiple of 16", partition_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (hkv > 65535 || B > 65535) return fail(PA_ERR_INVALID_ARGUMENT, "B and num_kv_heads must be <= 65535");
  const int64_t P = pa::partitions_for(max_context_len, partition_size);
  if (P > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "too many partitions");
  const size_t need = pa::workspace_bytes_for(B, num_q_heads, D, P);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes needed (got %zu)", need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % pa::kAlign != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  if (pa::debug_enabled()) {
    std::vector<int32_t> lens(B), tab(static_cast<size_t>(B) * max_blocks);
    if (hipMemcpy(lens.data(), context_lens, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(tab.data(), block_tables, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading block_tables / context_lens failed");
    for (int32_t i = 0; i < B; ++i) {
      if (lens[i] < 0 || lens[i] > max_context_len)
        return fail(PA_ERR_INVALID_ARGUMENT, "context_lens[%d] = %d outside [0, max_context_len %d]", i, lens[i],
                    max_context_len);
      const int32_t nb = (lens[i] + bs - 1) / bs;
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t id = tab[static_cast<size_t>(i) * max_blocks + j];
        if (id < 0 || id >= cache->num_blocks)
          return fail(PA_ERR_INVALID_ARGUMENT, "block_tables[%d][%d] = %d outside [0, %d)", i, j, id,
                      cache->num_blocks);
      }
    }
  }

  pa::DecodeParams prm{};
  prm.q = q;
  prm.k_pool = cache->k;
  prm.v_pool = cache->v;
  prm.out = out;
  const size_t rows = static_cast<size_t>(B) * num_q_heads * P;
  if (need > 0) {
    char* ws = static_cast<char*>(workspace);
    prm.part_m = reinterpret_cast<float*>(ws);
    prm.part_l = reinterpret_cast<float*>(ws + pa::align_up(rows * sizeof(float)));
    prm.part_o = reinterpret_cast<float*>(ws + 2 * pa::align_up(rows * sizeof(float)));
  }
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.block_stride = cache->block_stride;
  prm.num_blocks = cache->num_blocks;
  prm.num_kv_heads = hkv;
  prm.num_q_heads = num_q_heads;
  prm.max_blocks = max_blocks;
  prm.len_cap = max_context_len;
  prm.partition_size = P > 1 ? partition_size : 0;
  prm.num_partitions = static_cast<int32_t>(P);
  prm.out_dtype = pa::out_code(out_dtype);
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  prm.qk_scale_log2 = scale * (fp8 ? cache->k_scale : 1.0f) * 1.44269504088896340736f;
  prm.v_scale = fp8 ? cache->v_scale : 1.0f;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t wgs = P * hkv * B;
  if (wgs > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "too many workgroups (%lld)", (long long)wgs);
  hipError_t e = launch(prm, dim3(static_cast<uint32_t>(wgs)), s);
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
  if (P > 1) {
    pa::ReduceParams r{};
    r.part_m = prm.part_m;
    r.part_l = prm.part_l;
    r.part_o = prm.part_o;
    r.out = out;
    r.context_lens = context_lens;
    r.len_cap = max_context_len;
    r.partition_size = partition_size;
    r.num_partitions = static_cast<int32_t>(P);
    r.num_q_heads = num_q_heads;
    r.head_dim = D;
    r.out_dtype = prm.out_dtype;
    hipLaunchKernelGGL(pa::decode_reduce_kernel, dim3(num_q_heads, B), dim3(D < 128 ? D : 128), 0, s, r);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "decode reduce launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // extern "C"
