// Balanced-split decode kernels for F16 pools (q F16) with dim-major V blocks:
// head_dim 64/128, block size 8/16/32, query-head group 1/2/4/8.
#include "decode_sk_kernel.h"

namespace pa {
SkLaunch find_decode_sk_f16(int head_dim, int block_size, int group, bool append) {
  return select_decode_sk<F16, F16, false>(head_dim, block_size, group, append);
}
}  // namespace pa
