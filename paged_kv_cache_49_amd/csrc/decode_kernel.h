// Paged decode attention, gfx950: one workgroup per (context partition,
// KV head, sequence).
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
//
// What is computed ([course] §2 "The insight": the kernel follows the block
// table to gather K/V during the dot product; [note] 最小模型: blocks are
// visited in logical token order; [note] "why it works": the result is
// ordinary attention): for the G query heads h of KV head g and the tokens
// t of one partition,
//     z_t = scale * q_h . K_t,   m = max z,   l = sum 2^(z' - m'),
//     o_h = sum_t 2^(z'_t - m') V_t / l        (z' = z * log2 e)
// Partitions of one sequence are merged by decode_reduce_kernel.
//
// Workgroup layout (256 threads = 4 wave64):
//  * the partition is walked in chunks of kChunk tokens; for each chunk the
//    slice of the block table it needs is staged in LDS once (ids outside
//    the pool or past ceil(L/bs) read block 0, so no access leaves the pool)
//  * QK: each wave takes 16-token tiles; K rows are loaded straight from
//    the pool in MFMA operand layout (lane = token column n = lane%16,
//    head-dim slice j = lane/16, 16-byte loads) and multiplied against the
//    group's q rows (rows 0..G-1 of a 16-row A operand) with
//    v_mfma_f32_16x16x32_{bf16,f16}; lane (n, j) then holds the logits of
//    token n for heads 4j..4j+3. Logits go to LDS.
//  * softmax: chunk max per head (wave reduce + LDS), weights 2^(z'-m')
//    written back in place, running max / sum rescaled once per chunk.
//  * PV: lanes split a V row into 8-element pieces (D/8 lanes per row,
//    64/(D/8) rows per instruction, 16-byte loads for 16-bit pools) and
//    accumulate G x 8 fp32 partial outputs with FMAs.
//  * epilogue: partial outputs summed across the rows of a wave (lane
//    shuffles) and across waves (LDS), divided by the sum.
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
  float* part_m;  // [B][Hq][num_partitions]   running max (log2 domain)
  float* part_l;  // [B][Hq][num_partitions]   sum of weights
  float* part_o;  // [B][Hq][num_partitions][D] normalised partial output
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t block_stride;  // elements
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t len_cap;         // min(max_context_len, max_blocks * block_size)
  int32_t partition_size;  // tokens per partition; 0 = whole context
  int32_t num_partitions;  // grid.x
  int32_t out_dtype;       // 0 f16, 1 bf16, 2 f32
  float qk_scale_log2;     // scale * k_scale * log2(e)
  float v_scale;           // 1 for 16-bit pools
};

template <typename KV, int D, int BS, int G>
struct DecodeCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kChunk = 512;
  static constexpr int kKSteps = D / 32;  // MFMAs per 16-token tile
  static constexpr int kLpr = D / 8;      // lanes per V row in PV
  static constexpr int kTpi = 64 / kLpr;  // V rows per PV instruction
  static constexpr int kTblSlots = kChunk / BS + 2;
  static constexpr int kLogits = kChunk * G;
  static constexpr int kOutPartials = kWaves * G * D;
  static constexpr int kScratch = kLogits > kOutPartials ? kLogits : kOutPartials;
  static_assert(D % 64 == 0, "head_dim must be a multiple of 64");
  static_assert(G >= 1 && G <= 8, "group size 1..8");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size 8, 16 or 32");
};

// Head-dim offset of the 8 elements lane group j feeds to QK MFMA step i.
// Any assignment works as long as q and K use the same one; this one makes
// each 16-byte load contiguous (16-bit: 32i + 8j; fp8: one 16-byte load of
// 16 dims serves steps 2a and 2a+1).
template <int KVBytes>
__device__ __forceinline__ constexpr int qk_dim(int i, int j) {
  return KVBytes == 2 ? 32 * i + 8 * j : 64 * (i / 2) + 16 * j + 8 * (i % 2);
}

template <typename KV, typename QT, int D, int BS, int G>
__global__ __launch_bounds__(256) void paged_decode_kernel(const DecodeParams p) {
  using C = DecodeCfg<KV, D, BS, G>;
  constexpr int kB = KV::kBytes;
  __shared__ float s_buf[C::kScratch];
  __shared__ int32_t s_tbl[C::kTblSlots];
  __shared__ float s_red[C::kWaves][G];
  __shared__ float s_sum[C::kWaves][G];

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int L = p.context_lens[s];
  L = L < p.len_cap ? L : p.len_cap;
  L = L > 0 ? L : 0;
  const int ps = p.partition_size > 0 ? p.partition_size : (L > 0 ? L : 1);
  const int nparts = (L + ps - 1) / ps;
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int64_t head0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(g) * G;
  if (L == 0) {
    for (int i = tid; i < G * D; i += C::kThreads) store_out(p.out, head0 * D + i, p.out_dtype, 0.f);
    return;
  }
  const int tok_begin = part * ps;
  const int tok_end = min(L, tok_begin + ps);

  // q rows of the group as MFMA A operands (rows >= G are zero)
  u32x4 qa[C::kKSteps];
  {
    const int h = lane & 15, j = lane >> 4;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (head0 + (h < G ? h : 0)) * D;
#pragma unroll
    for (int i = 0; i < C::kKSteps; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + qk_dim<kB>(i, j));
      qa[i] = h < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);
  const int64_t blk_bytes = p.block_stride * kB;
  const int64_t tok_bytes = static_cast<int64_t>(p.num_kv_heads) * D * kB;
  const int64_t head_bytes = static_cast<int64_t>(g) * D * kB;
  const int nvalid_blk = (L + BS - 1) / BS;
  const int32_t* bt = p.block_tables + static_cast<int64_t>(s) * p.max_blocks;

  float acc[G][8];
  float m_run[G], l_th[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_th[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  for (int c0 = tok_begin; c0 < tok_end; c0 += C::kChunk) {
    const int n = min(C::kChunk, tok_end - c0);
    const int ntiles = (n + 15) >> 4;
    const int first_blk = c0 / BS;
    const int nblk = (c0 + ntiles * 16 - 1) / BS - first_blk + 1;
    for (int i = tid; i < nblk; i += C::kThreads) {
      const int bi = first_blk + i;
      int32_t id = bi < nvalid_blk ? bt[bi] : 0;
      s_tbl[i] = static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks) ? id : 0;
    }
    __syncthreads();

    // ---- QK on MFMA: 16-token tiles, one per wave per step
    for (int tile = wave; tile < ntiles; tile += C::kWaves) {
      const int col = lane & 15, j = lane >> 4;
      const int t = c0 + tile * 16 + col;
      const int32_t phys = s_tbl[t / BS - first_blk];
      const char* krow = kbase + phys * blk_bytes + (t % BS) * tok_bytes + head_bytes;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kB == 2) {
        u32x4 kb[C::kKSteps];
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) kb[i] = *reinterpret_cast<const u32x4*>(krow + 2 * qk_dim<2>(i, j));
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) sacc = mfma_16x16x32<QT>(qa[i], kb[i], sacc);
      } else {
        u32x4 kb[C::kKSteps / 2];
#pragma unroll
        for (int a = 0; a < C::kKSteps / 2; ++a)
          kb[a] = *reinterpret_cast<const u32x4*>(krow + qk_dim<1>(2 * a, j));
#pragma unroll
        for (int a = 0; a < C::kKSteps / 2; ++a) {
          const u32x2 b0 = e4m3x4_to_bf16x4(kb[a].x), b1 = e4m3x4_to_bf16x4(kb[a].y);
          const u32x2 b2 = e4m3x4_to_bf16x4(kb[a].z), b3 = e4m3x4_to_bf16x4(kb[a].w);
          sacc = mfma_16x16x32<QT>(qa[2 * a], u32x4{b0.x, b0.y, b1.x, b1.y}, sacc);
          sacc = mfma_16x16x32<QT>(qa[2 * a + 1], u32x4{b2.x, b2.y, b3.x, b3.y}, sacc);
        }
      }
      const bool valid = t < tok_end;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * j + r;
        if (h < G) s_buf[(tile * 16 + col) * G + h] = valid ? sacc[r] * p.qk_scale_log2 : -INFINITY;
      }
    }
    __syncthreads();

    // ---- softmax over the chunk: max, weights, running sums
    float mloc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
    for (int t = tid; t < ntiles * 16; t += C::kThreads) {
#pragma unroll
      for (int h = 0; h < G; ++h) mloc[h] = fmaxf(mloc[h], s_buf[t * G + h]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mloc[h] = wave_max(mloc[h]);
      if (lane == 0) s_red[wave][h] = mloc[h];
    }
    __syncthreads();
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mc = s_red[0][h];
#pragma unroll
      for (int w = 1; w < C::kWaves; ++w) mc = fmaxf(mc, s_red[w][h]);
      const float mn = fmaxf(m_run[h], mc);
      alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - mn);
      m_run[h] = mn;
    }
    float lsum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lsum[h] = 0.f;
    for (int t = tid; t < ntiles * 16; t += C::kThreads) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float e = __builtin_amdgcn_exp2f(s_buf[t * G + h] - m_run[h]);
        s_buf[t * G + h] = e;
        lsum[h] += e;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l_th[h] = l_th[h] * alpha[h] + lsum[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
    }
    __syncthreads();

    // ---- PV on VALU: each lane owns 8 head-dim elements of one row
    {
      const int row = lane / C::kLpr;
      const int cc = lane % C::kLpr;
      for (int tile = wave; tile < ntiles; tile += C::kWaves) {
#pragma unroll
        for (int it = 0; it < 16 / C::kTpi; ++it) {
          const int tr = tile * 16 + it * C::kTpi + row;
          const int t = c0 + tr;
          const int32_t phys = s_tbl[t / BS - first_blk];
          const char* vrow = vbase + phys * blk_bytes + (t % BS) * tok_bytes + head_bytes + cc * 8 * kB;
          float vf[8];
          if constexpr (kB == 2) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(vrow);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (__is_same(KV, BF16)) {
                vf[2 * e] = bf16_lo(w[e]);
                vf[2 * e + 1] = bf16_hi(w[e]);
              } else {
                vf[2 * e] = f16_lo(w[e]);
                vf[2 * e + 1] = f16_hi(w[e]);
              }
            }
          } else {
            const u32x2 w = *reinterpret_cast<const u32x2*>(vrow);
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = e4m3_to_f32((w[e / 4] >> (8 * (e % 4))) & 0xffu);
          }
          const bool valid = t < tok_end;
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[e] = valid ? vf[e] : 0.f;
          float wt[G];
#pragma unroll
          for (int h = 0; h < G; ++h) wt[h] = s_buf[tr * G + h];
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(wt[h], vf[e], acc[h][e]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: combine rows within a wave, then waves through LDS
#pragma unroll
  for (int off = C::kLpr; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = wave_sum(l_th[h]);
    if (lane == 0) s_sum[wave][h] = v;
  }
  if (lane < C::kLpr) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_buf[(wave * G + h) * D + lane * 8 + e] = acc[h][e];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += C::kThreads) {
    const int h = i / D, d = i % D;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < C::kWaves; ++w) {
      o += s_buf[(w * G + h) * D + d];
      l += s_sum[w][h];
    }
    const float val = o / l * p.v_scale;
    if (nparts == 1) {
      store_out(p.out, (head0 + h) * D + d, p.out_dtype, val);
    } else {
      const int64_t pi = (head0 + h) * p.num_partitions + part;
      p.part_o[pi * D + d] = val;
      if (d == 0) {
        p.part_m[pi] = m_run[h];
        p.part_l[pi] = l;
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
