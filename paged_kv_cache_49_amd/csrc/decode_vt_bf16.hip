// Decode kernels for BF16 pools with dim-major V blocks (q BF16): head_dim
// 64/128, block size 8/16/32, query-head group 1/2/4/8; and the
// shared-prefix group kernels of the same shapes.
#include "decode_shared_kernel.h"

namespace pa {
DecodeLaunch find_decode_vt_bf16(int head_dim, int block_size, int group) {
  return select_decode_vt<BF16, BF16, false>(head_dim, block_size, group);
}
GroupLaunch find_decode_group_bf16(int head_dim, int block_size, int group) {
  return select_decode_group<BF16, BF16, false>(head_dim, block_size, group);
}
}  // namespace pa
