// Selection of a compiled decode kernel by (pool dtype, head_dim, block size,
// query-head group size). Each pool dtype's kernels live in their own
// translation unit so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "libpagedattn.h"

namespace pa {

struct DecodeParams;
using DecodeLaunch = hipError_t (*)(const DecodeParams&, dim3 grid, hipStream_t stream);
// balanced split: the launcher sizes the grid from the device's CU count and
// the kernel's occupancy, at most max_wgs workgroups (partition mode:
// exactly max_wgs), and reports the grid it used in *wgs
struct SkParams;
using SkLaunch = hipError_t (*)(const SkParams&, int cus, int max_wgs, hipStream_t stream, int* wgs);

// partition kernels (QK and PV on the matrix cores): dim-major V blocks, and
// token-major V blocks (_tv: each tile's V rows transposed through LDS)
DecodeLaunch find_decode_vt_f16(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_bf16(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_fp8(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_f16_tv(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_bf16_tv(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_fp8_tv(int head_dim, int block_size, int group);

// shared-prefix group kernels (dim-major V; _tv: token-major V)
struct SharedParams;
using GroupLaunch = hipError_t (*)(const DecodeParams&, const SharedParams&, dim3 grid, hipStream_t stream);
GroupLaunch find_decode_group_f16(int head_dim, int block_size, int group);
GroupLaunch find_decode_group_bf16(int head_dim, int block_size, int group);
GroupLaunch find_decode_group_fp8(int head_dim, int block_size, int group);
GroupLaunch find_decode_group_f16_tv(int head_dim, int block_size, int group);
GroupLaunch find_decode_group_bf16_tv(int head_dim, int block_size, int group);
GroupLaunch find_decode_group_fp8_tv(int head_dim, int block_size, int group);

inline GroupLaunch find_decode_group(pa_dtype pool, pa_layout v_layout, int head_dim, int block_size, int group) {
  const bool tv = v_layout == PA_LAYOUT_TOKEN_MAJOR;
  switch (pool) {
    case PA_F16:
      return tv ? find_decode_group_f16_tv(head_dim, block_size, group)
                : find_decode_group_f16(head_dim, block_size, group);
    case PA_BF16:
      return tv ? find_decode_group_bf16_tv(head_dim, block_size, group)
                : find_decode_group_bf16(head_dim, block_size, group);
    case PA_FP8_E4M3:
      return tv ? find_decode_group_fp8_tv(head_dim, block_size, group)
                : find_decode_group_fp8(head_dim, block_size, group);
    default: return nullptr;
  }
}

SkLaunch find_decode_sk_f16(int head_dim, int block_size, int group, bool append);
SkLaunch find_decode_sk_bf16(int head_dim, int block_size, int group, bool append);
SkLaunch find_decode_sk_fp8(int head_dim, int block_size, int group, bool append);
SkLaunch find_decode_sk_f16_tv(int head_dim, int block_size, int group, bool append);
SkLaunch find_decode_sk_bf16_tv(int head_dim, int block_size, int group, bool append);
SkLaunch find_decode_sk_fp8_tv(int head_dim, int block_size, int group, bool append);

// the balanced split's kernel for the pool's dtype and V layout (nullptr:
// not built)
inline SkLaunch find_decode_sk(pa_dtype pool, pa_layout v_layout, int head_dim, int block_size, int group,
                               bool append) {
  const bool tv = v_layout == PA_LAYOUT_TOKEN_MAJOR;
  switch (pool) {
    case PA_F16:
      return tv ? find_decode_sk_f16_tv(head_dim, block_size, group, append)
                : find_decode_sk_f16(head_dim, block_size, group, append);
    case PA_BF16:
      return tv ? find_decode_sk_bf16_tv(head_dim, block_size, group, append)
                : find_decode_sk_bf16(head_dim, block_size, group, append);
    case PA_FP8_E4M3:
      return tv ? find_decode_sk_fp8_tv(head_dim, block_size, group, append)
                : find_decode_sk_fp8(head_dim, block_size, group, append);
    default: return nullptr;
  }
}

// the cascade variant of the balanced kernel (pa_decode_shared): built on
// the staged path, token-major V or fp8 pools (nullptr otherwise)
SkLaunch find_decode_cas_fp8(int head_dim, int block_size, int group);
SkLaunch find_decode_cas_f16_tv(int head_dim, int block_size, int group);
SkLaunch find_decode_cas_bf16_tv(int head_dim, int block_size, int group);
SkLaunch find_decode_cas_fp8_tv(int head_dim, int block_size, int group);

inline SkLaunch find_decode_cas(pa_dtype pool, pa_layout v_layout, int head_dim, int block_size, int group) {
  const bool tv = v_layout == PA_LAYOUT_TOKEN_MAJOR;
  switch (pool) {
    case PA_F16: return tv ? find_decode_cas_f16_tv(head_dim, block_size, group) : nullptr;
    case PA_BF16: return tv ? find_decode_cas_bf16_tv(head_dim, block_size, group) : nullptr;
    case PA_FP8_E4M3:
      return tv ? find_decode_cas_fp8_tv(head_dim, block_size, group) : find_decode_cas_fp8(head_dim, block_size, group);
    default: return nullptr;
  }
}

// the partition kernel for the pool's dtype and V layout
inline DecodeLaunch find_decode(pa_dtype pool, pa_layout v_layout, int head_dim, int block_size, int group) {
  const bool tv = v_layout == PA_LAYOUT_TOKEN_MAJOR;
  switch (pool) {
    case PA_F16:
      return tv ? find_decode_vt_f16_tv(head_dim, block_size, group) : find_decode_vt_f16(head_dim, block_size, group);
    case PA_BF16:
      return tv ? find_decode_vt_bf16_tv(head_dim, block_size, group) : find_decode_vt_bf16(head_dim, block_size, group);
    case PA_FP8_E4M3:
      return tv ? find_decode_vt_fp8_tv(head_dim, block_size, group) : find_decode_vt_fp8(head_dim, block_size, group);
    default: return nullptr;
  }
}

}  // namespace pa
