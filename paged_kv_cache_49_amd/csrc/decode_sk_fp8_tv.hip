// Balanced-split decode kernels for FP8 E4M3 pools (q BF16) with token-major V
// blocks (the unit's V rows widened to bf16 in the LDS stage and read back
// transposed): head_dim 64/128, block size 8/16/32, query-head group 1/2/4/8.
#include "decode_sk_kernel.h"

namespace pa {
SkLaunch find_decode_sk_fp8_tv(int head_dim, int block_size, int group, bool append) {
  return select_decode_sk<FP8, BF16, true>(head_dim, block_size, group, append);
}
}  // namespace pa
