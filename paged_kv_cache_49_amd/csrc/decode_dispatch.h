// Selection of a compiled decode kernel by (pool dtype, head_dim, block size,
// query-head group size). Each pool dtype's kernels live in their own
// translation unit so they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "libpagedattn.h"

namespace pa {

struct DecodeParams;
using DecodeLaunch = hipError_t (*)(const DecodeParams&, dim3 grid, hipStream_t stream);

DecodeLaunch find_decode_f16(int head_dim, int block_size, int group);
DecodeLaunch find_decode_bf16(int head_dim, int block_size, int group);
DecodeLaunch find_decode_fp8(int head_dim, int block_size, int group);
// kernels for dim-major V blocks (PV on the matrix cores)
DecodeLaunch find_decode_vt_f16(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_bf16(int head_dim, int block_size, int group);
DecodeLaunch find_decode_vt_fp8(int head_dim, int block_size, int group);

inline DecodeLaunch find_decode(pa_dtype pool, pa_layout v_layout, int head_dim, int block_size, int group) {
  const bool vt = v_layout == PA_LAYOUT_DIM_MAJOR;
  switch (pool) {
    case PA_F16: return vt ? find_decode_vt_f16(head_dim, block_size, group) : find_decode_f16(head_dim, block_size, group);
    case PA_BF16:
      return vt ? find_decode_vt_bf16(head_dim, block_size, group) : find_decode_bf16(head_dim, block_size, group);
    case PA_FP8_E4M3:
      return vt ? find_decode_vt_fp8(head_dim, block_size, group) : find_decode_fp8(head_dim, block_size, group);
    default: return nullptr;
  }
}

}  // namespace pa
