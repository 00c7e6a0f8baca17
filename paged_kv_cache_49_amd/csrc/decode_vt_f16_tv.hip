// Decode kernels for F16 pools (q F16) with token-major V blocks (the page's
// KVBlock layout; each tile's V rows transposed through LDS): head_dim
// 64/128, block size 8/16/32, query-head group 1/2/4/8; and the shared-prefix
// group kernels of the same shapes.
#include "decode_shared_kernel.h"

namespace pa {
DecodeLaunch find_decode_vt_f16_tv(int head_dim, int block_size, int group) {
  return select_decode_vt<F16, F16, true>(head_dim, block_size, group);
}
GroupLaunch find_decode_group_f16_tv(int head_dim, int block_size, int group) {
  return select_decode_group<F16, F16, true>(head_dim, block_size, group);
}
}  // namespace pa
