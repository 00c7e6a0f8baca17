// Decode over shared prefixes: the blocks a group of sequences shares are
// read once for all of the group's query rows.
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
// [course] §2 "The bonus" and §3: forked sequences (parallel sampling, beam
// search) share the prompt's physical blocks through their block tables;
// [note] prefix-sharing section: sequences with a common prefix point at the
// same blocks. The attention of each sequence is unchanged (it is still
// softmax attention over its own tokens in logical order); what changes is
// how often the shared blocks are read: with the prefix split into
// partitions, one pass over a shared partition serves every member of the
// group, because its K/V rows are the same for all of them.
//
// pa_decode_shared runs two kernels on the caller's stream:
//  1. paged_decode_shared_kernel, one wave per workgroup, two kinds of
//     workgroups in one grid (the short second kind fills the CUs the first
//     leaves idle):
//     * group units, one per (shared partition, group, KV head, set of CT
//       row tiles). A row tile's 16 q rows are (member, query head) pairs of
//       the group: row r of tile rt = member rt * (16 / G) + r / G, head
//       r % G. The wave attends all CT tiles of its set to each K/V tile it
//       loads (CT = 2 when a group has more than 16 rows, e.g. 8 samples x
//       4 heads: every shared K/V tile is then fetched once per KV head).
//       The partition's K/V tiles come through the first member's table
//       (the shared entries are identical in every member's table). Per-row
//       results are written as partition partials (m, l, o) of each member.
//     * tail units: the partitions past each sequence's shared prefix, per
//       (sequence, KV head) as in the partition kernel (vt_unit).
//  2. decode_reduce_kernel: the log-sum-exp merge of all partitions.
// When a group needs several row-tile sets (more than 32 rows), the sets of
// one (partition, group, KV head) are placed on the same XCD, next to each
// other in dispatch order (workgroups are dealt to the 8 XCDs round-robin),
// so the K/V they all read is fetched from HBM once and served from that
// XCD's L2 to the others.
#pragma once

#include "decode_vt_kernel.h"

namespace pa {

struct SharedParams {
  const int32_t* group_offsets;  // [num_groups + 1] into group_members
  const int32_t* group_members;  // batch rows of each group's sequences
  const int32_t* shared_len;     // [B] tokens of the sequence's shared prefix (a multiple of partition_size)
  int32_t num_groups;
  int32_t row_tiles;     // ceil(max_group_size * G / 16)
  int32_t tiles_per_wg;  // CT: row tiles one group unit attends together (1 or 2)
  int32_t row_sets;      // ceil(row_tiles / CT): group units per (partition, group, KV head)
  int32_t shared_parts;  // max shared_len / partition_size
  int32_t group_wgs;     // workgroups [0, group_wgs) are group units, the rest tail units
  int32_t pairs;         // B * num_kv_heads
};

// One group unit; wg < sp.group_wgs; s_out = the wave's 16 x D floats.
template <typename KV, typename QT, int D, int BS, int G, bool TV, int CT>
__device__ __forceinline__ void group_unit(const DecodeParams& p, const SharedParams& sp, int wg, float* s_out) {
  using C = DecodeCfg<KV, D, BS, G>;
  constexpr int kB = C::kB;
  constexpr int kNT = D / 16;
  constexpr int kMembersPerTile = 16 / G;

  // workgroup -> (unit, row-tile set): unit u's sets are workgroups
  // ((u / 8) * RS + rs) * 8 + u % 8, all on XCD u % 8
  const int RS = sp.row_sets;
  const int k = wg >> 3;
  const int rs = k % RS;
  const int64_t u = static_cast<int64_t>(k / RS) * 8 + (wg & 7);
  const int Hkv = p.num_kv_heads;
  if (u >= static_cast<int64_t>(sp.shared_parts) * sp.num_groups * Hkv) return;
  const int g = static_cast<int>(u % Hkv);
  const int rest = static_cast<int>(u / Hkv);
  const int gi = rest % sp.num_groups;
  const int part = rest / sp.num_groups;
  const int m0 = sp.group_offsets[gi];
  const int gsize = sp.group_offsets[gi + 1] - m0;
  const int rt0 = rs * CT;  // first row tile of the set
  if (gsize <= 0 || rt0 * kMembersPerTile >= gsize) return;
  const int first = sp.group_members[m0];
  const int ps = p.partition_size;
  const int tok_begin = part * ps;
  if (tok_begin + ps > sp.shared_len[first]) return;  // past this group's shared prefix

  const int lane = threadIdx.x & 63;
  const int col = lane & 15, j = lane >> 4;
  const int32_t* bt = p.block_tables + static_cast<int64_t>(first) * p.max_blocks;
  const int blk_first = tok_begin / BS;
  const int id_first = blk_first + lane < p.max_blocks ? bt[blk_first + lane] : 0;
  int L = p.context_lens[first];
  L = L < p.len_cap ? L : p.len_cap;

  // this lane's q row in tile ct: member (rt0 + ct) * kMembersPerTile + col / G, head col % G
  u32x4 qb[CT][C::kKSteps];
  bool row_ok[CT];
  int seq_r[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int mi = (rt0 + ct) * kMembersPerTile + col / G;
    row_ok[ct] = mi < gsize;
    seq_r[ct] = row_ok[ct] ? sp.group_members[m0 + mi] : first;
    const int64_t head = static_cast<int64_t>(seq_r[ct]) * p.num_q_heads + static_cast<int64_t>(g) * G + col % G;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + head * D;
#pragma unroll
    for (int i = 0; i < C::kKSteps; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + qk_dim<kB>(i, j));
      qb[ct][i] = row_ok[ct] ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m_w[CT], l_w[CT];
  f32x4 acc[CT][kNT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_w[ct] = -INFINITY;
    l_w[ct] = 0.f;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  vt_attend<KV, QT, D, BS, G, TV, CT>(p, bt, g, L, tok_begin, tok_begin + ps, id_first, qb, row_ok, m_w, l_w, acc,
                                      s_out);

#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int rt = rt0 + ct;
    if (rt * kMembersPerTile >= gsize) break;  // (uniform) no member in this tile
    // rows of this tile that belong to members: a prefix of the 16
    const int nrows = min(16, (gsize - rt * kMembersPerTile) * G);
    const float l_head = vt_normalise<D>(acc[ct], l_w[ct], p.v_scale, nrows, s_out);
    // the member (batch row) of each of the lane's output rows
    for (int i = lane * 8; i < nrows * D; i += 64 * 8) {
      const int r = i / D, d = i % D;
      const int seq = sp.group_members[m0 + rt * kMembersPerTile + r / G];
      const int64_t pi = ((static_cast<int64_t>(seq) * p.num_q_heads + static_cast<int64_t>(g) * G + r % G) *
                          p.num_partitions) + part;
      float* po = p.part_o + pi * D + d;
      *reinterpret_cast<f32x4*>(po) = f32x4{s_out[i], s_out[i + 1], s_out[i + 2], s_out[i + 3]};
      *reinterpret_cast<f32x4*>(po + 4) = f32x4{s_out[i + 4], s_out[i + 5], s_out[i + 6], s_out[i + 7]};
    }
    if (lane < nrows) {
      const int64_t pi = ((static_cast<int64_t>(seq_r[ct]) * p.num_q_heads + static_cast<int64_t>(g) * G + lane % G) *
                          p.num_partitions) + part;
      p.part_m[pi] = m_w[ct];
      p.part_l[pi] = l_head;
    }
    wave_lds_sync();  // the next tile's rows reuse s_out
  }
}

template <typename KV, typename QT, int D, int BS, int G, bool TV, int CT>
__global__ __launch_bounds__(64) void paged_decode_shared_kernel(const DecodeParams p, const SharedParams sp) {
  // 16 output rows of D floats; also the V tile's room (token-major V)
  static_assert(vt_tile_floats(D) <= 16 * D, "the V tile fits the output tile");
  __shared__ float s_out[16 * D];
  const int wg = static_cast<int>(blockIdx.x);
  if (wg < sp.group_wgs) {
    group_unit<KV, QT, D, BS, G, TV, CT>(p, sp, wg, s_out);
  } else {
    vt_unit<KV, QT, D, BS, G, TV>(p, wg - sp.group_wgs, sp.pairs, s_out);
  }
}

using GroupLaunch = hipError_t (*)(const DecodeParams&, const SharedParams&, dim3 grid, hipStream_t stream);

// sp.tiles_per_wg picks the build: 2 row tiles per group unit, or 1
template <typename KV, typename QT, int D, int BS, int G, bool TV>
hipError_t launch_decode_group(const DecodeParams& p, const SharedParams& sp, dim3 grid, hipStream_t stream) {
  if (sp.tiles_per_wg == 2) {
    hipLaunchKernelGGL((paged_decode_shared_kernel<KV, QT, D, BS, G, TV, 2>), grid, dim3(64), 0, stream, p, sp);
  } else {
    hipLaunchKernelGGL((paged_decode_shared_kernel<KV, QT, D, BS, G, TV, 1>), grid, dim3(64), 0, stream, p, sp);
  }
  return hipGetLastError();
}

template <typename KV, typename QT, int D, int BS, bool TV>
GroupLaunch select_decode_group_g(int G) {
  switch (G) {
    case 1: return &launch_decode_group<KV, QT, D, BS, 1, TV>;
    case 2: return &launch_decode_group<KV, QT, D, BS, 2, TV>;
    case 4: return &launch_decode_group<KV, QT, D, BS, 4, TV>;
    case 8: return &launch_decode_group<KV, QT, D, BS, 8, TV>;
    default: return nullptr;
  }
}

template <typename KV, typename QT, int D, bool TV>
GroupLaunch select_decode_group_bs(int BS, int G) {
  switch (BS) {
    case 8: return select_decode_group_g<KV, QT, D, 8, TV>(G);
    case 16: return select_decode_group_g<KV, QT, D, 16, TV>(G);
    case 32: return select_decode_group_g<KV, QT, D, 32, TV>(G);
    default: return nullptr;
  }
}

// TV = token-major V blocks
template <typename KV, typename QT, bool TV>
GroupLaunch select_decode_group(int D, int BS, int G) {
  switch (D) {
    case 64: return select_decode_group_bs<KV, QT, 64, TV>(BS, G);
    case 128: return select_decode_group_bs<KV, QT, 128, TV>(BS, G);
    default: return nullptr;
  }
}

}  // namespace pa
