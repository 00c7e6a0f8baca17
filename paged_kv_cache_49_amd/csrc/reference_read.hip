// The attainable read bandwidth of the device, as the reference the decode
// kernels' bytes per second are compared with: a plain contiguous read of
// one buffer, 16-byte non-temporal loads (eight per thread in flight), a
// grid-stride loop, and an XOR of everything read folded into one word per
// thread so the loads cannot be dropped. Not part of the attention method.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace pa {
namespace {

typedef uint32_t ref_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void reference_read_kernel(const ref_u32x4* __restrict__ p, int64_t n,
                                                             uint32_t* sink) {
  constexpr int kU = 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; base < n; base += kU * stride) {
    ref_u32x4 v[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int64_t idx = base + k * stride;
      v[k] = idx < n ? __builtin_nontemporal_load(p + idx) : ref_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kU; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_ref_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0 || grid <= 0 || grid > (1 << 20))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "pa_ref_stream_read: buf/sink non-null, bytes a positive multiple of 16, "
                                              "grid in [1, 2^20]");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "buf must be 16-byte aligned");
  hipLaunchKernelGGL(pa::reference_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const pa::ref_u32x4*>(buf), bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "pa_ref_stream_read launch: %s", hipGetErrorString(e));
  return PA_OK;
}
