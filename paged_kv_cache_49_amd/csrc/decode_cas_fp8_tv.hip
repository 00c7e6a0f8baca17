// Cascade (shared-prefix) variant of the balanced-split decode kernel for
// FP8 e4m3 pools (q BF16) with token-major V blocks: head_dim 64/128, block size 8/16/32,
// query-head group 1/2/4/8.
#include "decode_sk_kernel.h"

namespace pa {
SkLaunch find_decode_cas_fp8_tv(int head_dim, int block_size, int group) {
  return select_decode_cas<FP8, BF16, true>(head_dim, block_size, group);
}
}  // namespace pa
