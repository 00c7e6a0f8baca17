// Paged decode attention, gfx950: one wave64 workgroup per (context
// partition, KV head, sequence).
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
//
// What is computed ([course] §2 "The insight": the kernel follows the block
// table to gather K/V during the dot product; [note] 最小模型: blocks are
// visited in logical token order; [note] "why it works": the result is
// ordinary attention): for the G query heads h of KV head g and the tokens
// t of one partition,
//     z'_t = log2(e) * scale * q_h . K_t,   m' >= max z',
//     l = sum_t 2^(z'_t - m'),   o_h = sum_t 2^(z'_t - m') V_t / l
// Partitions of one sequence are merged by decode_reduce_kernel.
//
// The wave walks the partition's 16-token tiles in order; nothing in the
// kernel waits on another wave:
//  * start: the context length, the group's q rows and the first block-table
//    entries are requested together (one memory latency before the first
//    K/V request).
//  * block ids: the wave holds the block-table entries of the current chunk
//    (up to 64 blocks) in one VGPR, lane i = entry i; a tile's id is read
//    with v_readlane (block >= 16 tokens: one id per tile) or ds_bpermute
//    (8-token blocks). Ids outside the pool or past ceil(L / bs) read
//    block 0, so no access leaves the pool.
//  * loads: a tile's K rows are loaded in MFMA B-operand layout (lane =
//    token n = lane % 16, head-dim slice j = lane / 16, 16-byte loads) and
//    its V rows in PV layout (D/8 lanes per row, 8 elements each); the next
//    tile's K and V are requested before the current tile is processed.
//  * QK: v_mfma_f32_16x16x32_{bf16,f16} with the group's q rows as rows
//    0..G-1 of the A operand; lane (n, j) then holds the logits of token n
//    for heads 4j..4j+3.
//  * online softmax per wave: tile maxima by 16-lane DPP row reductions; the
//    running max m' moves only when a tile exceeds it by more than 2^8
//    (then the accumulators are rescaled), which keeps every weight below
//    2^8 and makes rescales rare; weights go through a wave-private LDS
//    slot to the PV lanes.
//  * PV on VALU: G x 8 fp32 accumulators per lane.
//  * epilogue: the rows of the wave are combined with lane shuffles and the
//    lanes of one row store the G x D result (or the partition's partial).
// Masking uses selects (never multiply-by-zero), so NaN in unused cache
// slots cannot leak into the result.
#pragma once

#include <hip/hip_runtime.h>

#include "decode_dispatch.h"
#include "device_common.h"

namespace pa {

struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  void* out;
  float* part_m;  // [B][Hq][num_partitions]   reference max (log2 domain)
  float* part_l;  // [B][Hq][num_partitions]   sum of weights
  float* part_o;  // [B][Hq][num_partitions][D] normalised partial output
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t block_stride;  // elements
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t len_cap;         // max_context_len (<= max_blocks * block_size)
  int32_t partition_size;  // tokens per partition; 0 = whole context
  int32_t num_partitions;  // grid.x
  int32_t out_dtype;       // 0 f16, 1 bf16, 2 f32
  float qk_scale_log2;     // scale * k_scale * log2(e)
  float v_scale;           // 1 for 16-bit pools
  // pa_decode_shared: tokens at the start of each sequence computed per
  // group (partitions below it are skipped here); nullptr otherwise
  const int32_t* shared_len;
};

template <typename KV, int D, int BS, int G>
struct DecodeCfg {
  static constexpr int kB = KV::kBytes;
  static constexpr int kThreads = 64;  // one wave per workgroup
  static constexpr int kKSteps = D / 32;                        // MFMAs per 16-token tile
  static constexpr int kKLoads = kB == 2 ? kKSteps : kKSteps / 2;  // 16-byte K loads per lane per tile
  static constexpr int kLpr = D / 8;                            // lanes per V row in PV
  static constexpr int kRpi = 64 / kLpr;                        // V rows per PV step
  static constexpr int kPvi = 16 / kRpi;                        // PV steps per tile
  static constexpr int kChunk = 64 * BS - (BS > 16 ? BS : 0);   // tokens whose block ids fit one VGPR
  static constexpr int kHRows = (G + 3) / 4;                    // MFMA output rows holding real heads
  static constexpr float kSlack = 8.0f;                         // log2 headroom before a rescale
  static_assert(D % 64 == 0, "head_dim must be a multiple of 64");
  static_assert(G >= 1 && G <= 8, "group size 1..8");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size 8, 16 or 32");
  static_assert(kChunk % 16 == 0, "chunks are whole tiles");
};

// Head-dim offset of the 8 elements lane group j feeds to QK MFMA step i.
// Any assignment works as long as q and K use the same one. 16-bit: 32i + 8j
// (each load instruction reads 64 contiguous bytes of every token row);
// fp8: one 16-byte load of 16 dims serves steps 2a and 2a+1.
template <int KVBytes>
__device__ __forceinline__ constexpr int qk_dim(int i, int j) {
  return KVBytes == 2 ? 32 * i + 8 * j : 64 * (i / 2) + 16 * j + 8 * (i % 2);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// max / sum over the 16 lanes of each DPP row (row_ror 8, 4, 2, 1); every
// lane of the row ends with the row's result.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0x128>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x122>(v));
  return fmaxf(v, dpp_f<0x121>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x122>(v);
  return v + dpp_f<0x121>(v);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// LDS written by some lanes of a wave and read by others: LDS operations of
// one wave complete in order; this keeps the compiler from reordering them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-lane V pieces: `type` = 8 token-major elements (PV on VALU),
// `raw_dm` = 4 tokens of one head dim from a dim-major block.
template <typename KV>
struct VVecT {
  using type = u32x4;
  using raw_dm = u32x2;
};
template <>
struct VVecT<FP8> {
  using type = u32x2;
  using raw_dm = uint32_t;
};

template <typename KV, typename QT, int D, int BS, int G>
__global__ __launch_bounds__(64) void paged_decode_kernel(const DecodeParams p) {
  using C = DecodeCfg<KV, D, BS, G>;
  constexpr int kB = C::kB;
  using VVec = typename VVecT<KV>::type;
  __shared__ float s_p[16 * G];

  // 1-D grid in partition-major order: workgroup w -> (part, seq, kv head).
  // Consecutive workgroups are dealt round-robin to the 8 XCDs, so each XCD
  // receives the same mix of partition indices (late partitions of short
  // sequences are empty; a partition-fastest order would pile all first
  // partitions onto one XCD).
  const int pairs = static_cast<int>(gridDim.x) / p.num_partitions;  // B * Hkv
  const int part = static_cast<int>(blockIdx.x) / pairs;
  const int pr = static_cast<int>(blockIdx.x) - part * pairs;
  const int s = pr / p.num_kv_heads;
  const int g = pr - s * p.num_kv_heads;
  const int lane = threadIdx.x;
  const int32_t* bt = p.block_tables + static_cast<int64_t>(s) * p.max_blocks;
  // issued together with the length: the first chunk's block-table entries
  // (in-bounds of the table row; masked once the length is known)
  const int blk_first = p.partition_size > 0 ? part * p.partition_size / BS : 0;
  const int id_first = blk_first + lane < p.max_blocks ? bt[blk_first + lane] : 0;

  int L = p.context_lens[s];
  L = L < p.len_cap ? L : p.len_cap;
  L = L > 0 ? L : 0;
  const int ps = p.partition_size > 0 ? p.partition_size : (L > 0 ? L : 1);
  const int nparts = (L + ps - 1) / ps;
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int64_t head0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(g) * G;
  if (L == 0) {
    for (int i = lane; i < G * D; i += C::kThreads) store_out(p.out, head0 * D + i, p.out_dtype, 0.f);
    return;
  }
  const int tok_begin = part * ps;
  const int tok_end = min(L, tok_begin + ps);

  const int col = lane & 15, j = lane >> 4;         // MFMA layout: token column, head-dim slice / head row
  const int vrow = lane / C::kLpr, vcc = lane % C::kLpr;  // PV layout: row in step, 8-element piece

  // q rows of the group as MFMA A operands (rows >= G are zero)
  u32x4 qa[C::kKSteps];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (head0 + (col < G ? col : 0)) * D;
#pragma unroll
    for (int i = 0; i < C::kKSteps; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + qk_dim<kB>(i, j));
      qa[i] = col < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);
  const int64_t blk_bytes = p.block_stride * kB;
  const int64_t tok_bytes = static_cast<int64_t>(p.num_kv_heads) * D * kB;
  const int64_t head_bytes = static_cast<int64_t>(g) * D * kB;
  const int nvalid_blk = (L + BS - 1) / BS;

  float m_w[G];  // running reference max per head (uniform across the wave)
  float l_r[4];  // per-lane partial sums, MFMA output layout
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_w[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) l_r[r] = 0.f;

  for (int c0 = tok_begin; c0 < tok_end; c0 += C::kChunk) {
    const int n = min(C::kChunk, tok_end - c0);
    const int ntiles = (n + 15) >> 4;
    const int blk0 = c0 / BS;
    const int nblk = (c0 + ntiles * 16 - 1) / BS - blk0 + 1;  // <= 64
    int ids;
    {
      const int bi = blk0 + lane;
      const int id = c0 == tok_begin ? id_first : (bi < p.max_blocks ? bt[bi] : 0);
      ids = (lane < nblk && bi < nvalid_blk && static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks)) ? id : 0;
    }

    // row pointers of one token for K (lane's column) and V (lane's PV row)
    auto phys_of = [&](int t) -> int {
      if constexpr (BS >= 16) {
        return __builtin_amdgcn_readlane(ids, (t & ~15) / BS - blk0);
      } else {
        return __shfl(ids, t / BS - blk0, 64);
      }
    };
    auto load_tile = [&](int tile, u32x4 (&kr)[C::kKLoads], VVec (&vr)[C::kPvi]) {
      const int tb = c0 + tile * 16;
      {
        const int t = tb + col;
        const char* krow = kbase + phys_of(t) * blk_bytes + (t % BS) * tok_bytes + head_bytes;
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
          const int off = kB == 2 ? 2 * qk_dim<2>(i, j) : qk_dim<1>(2 * i, j);
          kr[i] = *reinterpret_cast<const u32x4*>(krow + off);
        }
      }
#pragma unroll
      for (int it = 0; it < C::kPvi; ++it) {
        const int t = tb + it * C::kRpi + vrow;
        const char* vr_ = vbase + phys_of(t) * blk_bytes + (t % BS) * tok_bytes + head_bytes + vcc * 8 * kB;
        vr[it] = *reinterpret_cast<const VVec*>(vr_);
      }
    };

    u32x4 kc[C::kKLoads], kn[C::kKLoads];
    VVec vc[C::kPvi], vn[C::kPvi];
    load_tile(0, kc, vc);
    for (int tile = 0; tile < ntiles; ++tile) {
      // request the next tile (the last tile re-requests itself: a cache hit)
      load_tile(tile + 1 < ntiles ? tile + 1 : tile, kn, vn);
      const int tb = c0 + tile * 16;

      // ---- QK on MFMA
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kB == 2) {
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) sacc = mfma_16x16x32<QT>(qa[i], kc[i], sacc);
      } else {
#pragma unroll
        for (int a = 0; a < C::kKLoads; ++a) {
          const u32x2 b0 = e4m3x4_to_bf16x4(kc[a].x), b1 = e4m3x4_to_bf16x4(kc[a].y);
          const u32x2 b2 = e4m3x4_to_bf16x4(kc[a].z), b3 = e4m3x4_to_bf16x4(kc[a].w);
          sacc = mfma_16x16x32<QT>(qa[2 * a], u32x4{b0.x, b0.y, b1.x, b1.y}, sacc);
          sacc = mfma_16x16x32<QT>(qa[2 * a + 1], u32x4{b2.x, b2.y, b3.x, b3.y}, sacc);
        }
      }
      const bool kval = tb + col < tok_end;
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = kval ? sacc[r] * p.qk_scale_log2 : -INFINITY;

      // ---- online softmax
      float mt[G];
      {
        float mx[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mx[r] = row16_max(sv[r]);
#pragma unroll
        for (int h = 0; h < G; ++h) mt[h] = readlane_f(mx[h % 4], 16 * (h / 4));
      }
      bool rescale = false;
#pragma unroll
      for (int h = 0; h < G; ++h) rescale |= mt[h] > m_w[h] + C::kSlack;
      if (rescale) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (mt[h] > m_w[h] + C::kSlack) {
            const float a = __builtin_amdgcn_exp2f(m_w[h] - mt[h]);
            m_w[h] = mt[h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= a;
            l_r[h % 4] *= (j == h / 4) ? a : 1.0f;
          }
        }
      }
      float pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mh = m_w[r < G ? r : 0];
        if constexpr (G > 4) mh = j == 1 ? m_w[4 + r] : mh;
        pw[r] = __builtin_amdgcn_exp2f(sv[r] - mh);
        l_r[r] += pw[r];
      }
      if (j < C::kHRows) {
        float* dst = &s_p[col * G + 4 * j];
        if constexpr (G >= 4) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{pw[0], pw[1], pw[2], pw[3]};
        } else {
#pragma unroll
          for (int r = 0; r < G; ++r) dst[r] = pw[r];
        }
      }
      wave_lds_sync();

      // ---- PV on VALU
      const bool tail = tb + 16 > tok_end;
#pragma unroll
      for (int it = 0; it < C::kPvi; ++it) {
        const int tr = it * C::kRpi + vrow;
        float vf[8];
        if constexpr (kB == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (__is_same(KV, BF16)) {
              vf[2 * e] = bf16_lo(vc[it][e]);
              vf[2 * e + 1] = bf16_hi(vc[it][e]);
            } else {
              vf[2 * e] = f16_lo(vc[it][e]);
              vf[2 * e + 1] = f16_hi(vc[it][e]);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; e += 4) {
            const f32x4 f = e4m3x4_to_f32x4(vc[it][e / 4]);
            vf[e] = f.x;
            vf[e + 1] = f.y;
            vf[e + 2] = f.z;
            vf[e + 3] = f.w;
          }
        }
        if (tail) {
          const bool ok = tb + tr < tok_end;
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = ok ? vf[e] : 0.f;
        }
        float w[G];
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int h4 = 0; h4 < G; h4 += 4) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&s_p[tr * G + h4]);
            w[h4] = w4.x;
            w[h4 + 1] = w4.y;
            w[h4 + 2] = w4.z;
            w[h4 + 3] = w4.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) w[h] = s_p[tr * G + h];
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w[h], vf[e], acc[h][e]);
      }
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i) kc[i] = kn[i];
#pragma unroll
      for (int i = 0; i < C::kPvi; ++i) vc[i] = vn[i];
    }
  }

  // ---- epilogue: sums over the 16 lanes of each head row, partial outputs
  // over the kRpi rows of the PV layout, then lanes 0..kLpr-1 store.
  float lw[G];
  {
    float ls[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ls[r] = row16_sum(l_r[r]);
#pragma unroll
    for (int h = 0; h < G; ++h) lw[h] = readlane_f(ls[h % 4], 16 * (h / 4));
  }
#pragma unroll
  for (int off = C::kLpr; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
  if (lane < C::kLpr) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = p.v_scale / lw[h];
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = acc[h][e] * inv;
      if (nparts == 1) {
        store_out8(p.out, (head0 + h) * D + lane * 8, p.out_dtype, o);
      } else {
        const int64_t pi = (head0 + h) * p.num_partitions + part;
        float* po = p.part_o + pi * D + lane * 8;
        *reinterpret_cast<f32x4*>(po) = f32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<f32x4*>(po + 4) = f32x4{o[4], o[5], o[6], o[7]};
        if (lane == 0) {
          p.part_m[pi] = m_w[h];
          p.part_l[pi] = lw[h];
        }
      }
    }
  }
}

}  // namespace pa

namespace pa {

template <typename KV, typename QT, int D, int BS, int G>
hipError_t launch_decode(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_kernel<KV, QT, D, BS, G>), grid, dim3(DecodeCfg<KV, D, BS, G>::kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename KV, typename QT, int D, int BS>
DecodeLaunch select_decode_g(int G) {
  switch (G) {
    case 1: return &launch_decode<KV, QT, D, BS, 1>;
    case 2: return &launch_decode<KV, QT, D, BS, 2>;
    case 4: return &launch_decode<KV, QT, D, BS, 4>;
    case 8: return &launch_decode<KV, QT, D, BS, 8>;
    default: return nullptr;
  }
}

template <typename KV, typename QT, int D>
DecodeLaunch select_decode_bs(int BS, int G) {
  switch (BS) {
    case 8: return select_decode_g<KV, QT, D, 8>(G);
    case 16: return select_decode_g<KV, QT, D, 16>(G);
    case 32: return select_decode_g<KV, QT, D, 32>(G);
    default: return nullptr;
  }
}

template <typename KV, typename QT>
DecodeLaunch select_decode(int D, int BS, int G) {
  switch (D) {
    case 64: return select_decode_bs<KV, QT, 64>(BS, G);
    case 128: return select_decode_bs<KV, QT, 128>(BS, G);
    default: return nullptr;
  }
}

}  // namespace pa
