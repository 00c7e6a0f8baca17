// Paged decode attention with both products on the matrix cores, for pools
// whose V blocks are dim-major (V[heads][head_dim][block]) or token-major
// (the page's V[block][heads][head_dim], TV).
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
// decode_common.h states what is computed and the block-table and masking
// rules. One wave64 workgroup per (partition, sequence, KV head).
//
// Per 16-token tile:
//  * S^T = K q^T with v_mfma_f32_16x16x32 (A = the tile's K rows, one token
//    per lane row, 8 head dims per lane; B = the group's q rows, padded to 16
//    heads with zeros). Lane (h = lane % 16, j = lane / 16) ends up holding
//    the logits of head h for tokens 4j..4j+3 of the tile.
//  * online softmax per head: the tile max is a 4-register max and two
//    cross-row lane exchanges; the running max moves only past a 2^8 slack.
//  * the weights are already in the A-operand layout of v_mfma_f32_16x16x16
//    (row = head, k = 4 tokens per lane), so PV needs no data movement: each
//    weight is split into a high and a low 16-bit part (hi + lo carries ~16
//    mantissa bits) and both are multiplied against V.
//  * V: dim-major blocks give each lane the 4 consecutive tokens of one head
//    dimension as one 8-byte load (a 16-dim tile of a 16-token block is 512
//    contiguous bytes), which is exactly the B operand (k = tokens, n = dim).
//    Token-major blocks (TV): the tile's V rows load like its K rows, go to
//    the wave's LDS tile (fp8 widened to bf16 on the way) and come back
//    transposed, one ds_read_b64_tr_b16 per 16-dim n-tile giving the same
//    operand.
//  * acc: one 16x16 fp32 tile per 16 head dims, rows = heads.
// Unused weight rows (heads >= G) are zero; V elements of tokens past the
// end are zeroed with masks (never multiplied by a zero weight), so NaN in
// unused cache slots cannot reach the result.
#pragma once

#include "decode_common.h"

namespace pa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four 16-bit elements of a transposing LDS read (ds_read_b64_tr_b16): in
// each 16-lane group, lane i gets element i % 4 of the 8 bytes that lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group point at, in
// that order.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Eight 8-bit elements of a transposing LDS read (ds_read_b64_tr_b8): in
// each 16-lane group, lane i gets element i % 8 of the 8 bytes that lanes
// i / 8, 2 + i / 8, 4 + i / 8, ..., 14 + i / 8 of the group point at, in
// that order (element k in byte k of the result).
__device__ __forceinline__ u32x2 lds_read_tr8(const char* p) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// A 16-token V tile in LDS for the transposing reads: 16 rows of D 16-bit
// elements, padded by 16 elements (the reads of a 16-lane group then hit
// distinct banks). kVTileRow elements per row; vt_tile_floats(D) = its size
// in floats.
template <int D>
struct VTile {
  static constexpr int kRow = D + 16;
};
__host__ __device__ constexpr int vt_tile_floats(int D) { return 16 * (D + 16) / 2; }

// V registers per lane and tile: dim-major runs (4 tokens of one head dim:
// u32x2 for 16-bit pools, one dword for fp8), or token-major row pieces
// (u32x4, as K)
template <typename KV, bool TV>
struct VtVRegs {
  using type = u32x2;
};
template <>
struct VtVRegs<FP8, false> {
  using type = uint32_t;
};
template <typename KV>
struct VtVRegs<KV, true> {
  using type = u32x4;
};

template <typename T>
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_16x16x16<BF16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                    0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x16<F16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                0);
}

// Two fp32 values -> one dword of two 16-bit values (round to nearest even),
// and the exact fp32 value of each half.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
template <typename T>
__device__ __forceinline__ float half_lo(uint32_t w) {
  if constexpr (__is_same(T, BF16)) return bf16_lo(w);
  return f16_lo(w);
}
template <typename T>
__device__ __forceinline__ float half_hi(uint32_t w) {
  if constexpr (__is_same(T, BF16)) return bf16_hi(w);
  return f16_hi(w);
}

// Attention of one wave's 16 q rows over tokens [tok_begin, tok_end) of a
// sequence with block table row `bt` and clamped length L (table entries
// past ceil(L / BS) are never read), KV head g. qb holds the q rows as the
// B operand of S^T = K q^T; lane row `col` takes part iff row_ok. id_first
// = table entry (tok_begin / BS + lane), loaded by the caller ahead of time.
// Leaves, per lane: m_w = running reference max of row `col` (log2 domain),
// l_w = this lane's share of that row's weight sum, acc = the unnormalised
// output tile (rows = q rows).
//
// Per 16-token tile:
//  * S^T = K q^T with v_mfma_f32_16x16x32 (A = the tile's K rows, one token
//    per lane row, 8 head dims per lane). Lane (r = lane % 16, j = lane / 16)
//    ends up holding the logits of row r for tokens 4j..4j+3 of the tile.
//  * online softmax per row: the tile max is a 4-register max and two
//    cross-row lane exchanges; the running max moves only past a 2^8 slack.
//  * the weights are already in the A-operand layout of v_mfma_f32_16x16x16
//    (row = q row, k = 4 tokens per lane), so PV needs no data movement:
//    each weight is split into a high and a low 16-bit part (hi + lo carries
//    ~16 mantissa bits) and both are multiplied against V.
//  * V: dim-major blocks give each lane the 4 consecutive tokens of one head
//    dimension as one 8-byte load (a 16-dim tile of a 16-token block is 512
//    contiguous bytes), which is exactly the B operand (k = tokens, n = dim).
//  * loads are staggered over single buffers: K(t+1) is requested right
//    after QK(t) has consumed K(t), and V(t+1) right after PV(t) has
//    consumed V(t); loads complete in order, so QK(t+1) waits only for
//    K(t+1) while V(t+1) is still in flight, and vice versa.
// s_lds: the wave's LDS region (token-major V only; vt_tile_floats(D)
// floats), free again when the call returns.
// CT column tiles: the wave attends CT sets of 16 q rows to the same
// tokens (qb[ct], row_ok[ct], m_w[ct], l_w[ct], acc[ct]); each tile's K and
// V are loaded, staged and converted once and used for every set (the
// shared-prefix group units, whose rows outnumber 16).
template <typename KV, typename QT, int D, int BS, int G, bool TV, int CT = 1>
__device__ __forceinline__ void vt_attend(const DecodeParams& p, const int32_t* bt, int g, int L, int tok_begin,
                                          int tok_end, int id_first, const u32x4 (&qb)[CT][D / 32],
                                          const bool (&row_ok)[CT], float (&m_w)[CT], float (&l_w)[CT],
                                          f32x4 (&acc)[CT][D / 16], float* s_lds) {
  using C = DecodeCfg<KV, D, BS, G>;
  constexpr int kB = C::kB;
  constexpr int kNT = D / 16;
  using VRaw = typename VtVRegs<KV, TV>::type;
  constexpr int kVL = TV ? C::kKLoads : kNT;  // V loads per lane and tile
  constexpr int kVRow = VTile<D>::kRow;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, j = lane >> 4;
  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);
  const int64_t blk_bytes = p.block_stride * kB;
  const int64_t tok_bytes = static_cast<int64_t>(p.num_kv_heads) * D * kB;
  const int64_t khead_bytes = static_cast<int64_t>(g) * D * kB;
  // lane's V run inside a block: head dim (g*D + col) of the first n-tile, token 4j
  const int64_t vlane_bytes = (static_cast<int64_t>(g) * D + col) * BS * kB;
  const uint32_t voff_lane = static_cast<uint32_t>(vlane_bytes + 4 * j * kB);
  // lane's K row inside a 16-token tile: token col, head g, first head-dim slice
  const uint32_t koff_lane = static_cast<uint32_t>(col * tok_bytes + khead_bytes + qk_dim<kB>(0, j) * kB);
  constexpr int kVTileBytes = 16 * BS * kB;  // one 16-dim n-tile of a block
  const int nvalid_blk = (L + BS - 1) / BS;

  for (int c0 = tok_begin; c0 < tok_end; c0 += C::kChunk) {
    const int n = min(C::kChunk, tok_end - c0);
    const int ntiles = (n + 15) >> 4;
    const int blk0 = c0 / BS;
    const int nblk = (c0 + ntiles * 16 - 1) / BS - blk0 + 1;  // <= 64
    int ids;
    {
      const int bi = blk0 + lane;
      const int id = c0 == tok_begin ? id_first : (bi < p.max_blocks ? bt[bi] : 0);
      ids = (lane < nblk && bi < nvalid_blk && static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks)) ? id
                                                                                                                 : 0;
    }
    auto phys_of = [&](int t) -> int {
      if constexpr (BS >= 16) {
        return __builtin_amdgcn_readlane(ids, (t & ~15) / BS - blk0);
      } else {
        return __shfl(ids, t / BS - blk0, 64);
      }
    };
    // K rows: block base (uniform for blocks >= 16 tokens) + per-lane offset
    auto load_k = [&](int tile, u32x4 (&kr)[C::kKLoads]) {
      const int tb = c0 + tile * 16;
      const int t = tb + col;
      const char* krow;
      if constexpr (BS >= 16) {
        const char* base = kbase + static_cast<int64_t>(phys_of(tb)) * blk_bytes + (tb % BS) * tok_bytes;
        krow = base + koff_lane;
      } else {
        krow = kbase + static_cast<int64_t>(phys_of(t)) * blk_bytes + (t % BS) * tok_bytes + khead_bytes;
      }
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i) {
        const int off = kB == 2 ? 2 * qk_dim<2>(i, j) : qk_dim<1>(2 * i, j);
        kr[i] = *reinterpret_cast<const u32x4*>(krow + (BS >= 16 ? off - qk_dim<kB>(0, j) * kB : off));
      }
    };
    // V: dim-major, runs of 4 tokens of one head dim per lane and n-tile;
    // token-major, the lane's pieces of its token row, exactly as K
    auto load_v = [&](int tile, VRaw (&vr)[kVL]) {
      const int tb = c0 + tile * 16;
      if constexpr (TV) {
        const int t = tb + col;
        const char* vrow;
        if constexpr (BS >= 16) {
          vrow = vbase + static_cast<int64_t>(phys_of(tb)) * blk_bytes + (tb % BS) * tok_bytes + koff_lane;
        } else {
          vrow = vbase + static_cast<int64_t>(phys_of(t)) * blk_bytes + (t % BS) * tok_bytes + khead_bytes;
        }
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
          const int off = kB == 2 ? 2 * qk_dim<2>(i, j) : qk_dim<1>(2 * i, j);
          vr[i] = *reinterpret_cast<const u32x4*>(vrow + (BS >= 16 ? off - qk_dim<kB>(0, j) * kB : off));
        }
      } else {
        const int t = tb + 4 * j;
        const char* vrun;
        if constexpr (BS >= 16) {
          vrun = vbase + static_cast<int64_t>(phys_of(tb)) * blk_bytes + (tb % BS) * kB + voff_lane;
        } else {
          vrun = vbase + static_cast<int64_t>(phys_of(t)) * blk_bytes + vlane_bytes + (t % BS) * kB;
        }
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) vr[nt] = *reinterpret_cast<const VRaw*>(vrun + nt * kVTileBytes);
      }
    };

    // Loads are staggered over single buffers: K(t+1) is requested right
    // after QK(t) has consumed K(t), and V(t+1) right after PV(t) has
    // consumed V(t). Loads complete in order, so QK(t+1) waits only for
    // K(t+1) while V(t+1) is still in flight, and vice versa.
    // The requests stay where they are written (K before V, tile by tile):
    // with token-major V its registers are free as soon as the rows are in
    // LDS, and the scheduler would otherwise hoist V(t+1) above K(t+1), so
    // that QK(t+1) waited for both.
    u32x4 kr[C::kKLoads];
    VRaw vr[kVL];
    __builtin_amdgcn_sched_barrier(0);
    load_k(0, kr);
    __builtin_amdgcn_sched_barrier(0);
    load_v(0, vr);
    __builtin_amdgcn_sched_barrier(0);
    for (int tile = 0; tile < ntiles; ++tile) {
      const int tb = c0 + tile * 16;
      const int next = tile + 1 < ntiles ? tile + 1 : tile;  // a missing next tile re-requests this one
      // ---- S^T = K q^T (per column tile; fp8 K widened once)
      f32x4 sacc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) sacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kB == 2) {
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) sacc[ct] = mfma_16x16x32<QT>(kr[i], qb[ct][i], sacc[ct]);
      } else {
#pragma unroll
        for (int a = 0; a < C::kKLoads; ++a) {
          const u32x2 b0 = e4m3x4_to_bf16x4(kr[a].x), b1 = e4m3x4_to_bf16x4(kr[a].y);
          const u32x2 b2 = e4m3x4_to_bf16x4(kr[a].z), b3 = e4m3x4_to_bf16x4(kr[a].w);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            sacc[ct] = mfma_16x16x32<QT>(u32x4{b0.x, b0.y, b1.x, b1.y}, qb[ct][2 * a], sacc[ct]);
            sacc[ct] = mfma_16x16x32<QT>(u32x4{b2.x, b2.y, b3.x, b3.y}, qb[ct][2 * a + 1], sacc[ct]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_k(next, kr);
      __builtin_amdgcn_sched_barrier(0);
      u32x2 phi[CT], plo[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = tb + 4 * j + r < tok_end ? sacc[ct][r] * p.qk_scale_log2 : -INFINITY;

        // ---- online softmax (row = col of this column tile)
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, mx), 0x401F)));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool need = row_ok[ct] && mx > m_w[ct] + C::kSlack;
        if (__builtin_amdgcn_ballot_w64(need)) {
          const float a = need ? __builtin_amdgcn_exp2f(m_w[ct] - mx) : 1.0f;
          m_w[ct] = need ? mx : m_w[ct];
          l_w[ct] *= a;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(a, 4 * j + r, 64);  // factor of row 4j + r (held by lane 4j + r)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) acc[ct][nt][r] *= ar;
          }
        }
        float pw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pw[r] = row_ok[ct] ? __builtin_amdgcn_exp2f(sv[r] - m_w[ct]) : 0.f;
          l_w[ct] += pw[r];
        }
        const uint32_t h0 = pack2<QT>(pw[0], pw[1]), h1 = pack2<QT>(pw[2], pw[3]);
        const uint32_t l0 = pack2<QT>(pw[0] - half_lo<QT>(h0), pw[1] - half_hi<QT>(h0));
        const uint32_t l1 = pack2<QT>(pw[2] - half_lo<QT>(h1), pw[3] - half_hi<QT>(h1));
        phi[ct] = u32x2{h0, h1};
        plo[ct] = u32x2{l0, l1};
      }

      // ---- PV: acc[h][d] += sum_t w[h][t] V[t][d]
      u32x2 vmask = {0xffffffffu, 0xffffffffu};
      if (tb + 16 > tok_end) {
        const int t = tb + 4 * j;
        vmask.x = (t < tok_end ? 0xffffu : 0u) | (t + 1 < tok_end ? 0xffff0000u : 0u);
        vmask.y = (t + 2 < tok_end ? 0xffffu : 0u) | (t + 3 < tok_end ? 0xffff0000u : 0u);
      }
      // token-major V: the tile's rows into the wave's LDS tile (fp8 widened
      // to bf16), then lane (d, j) reads tokens 4j .. 4j + 3 of head dim
      // 16 nt + d with one transposing read per n-tile, its group's lanes
      // pointing at rows 4j + lane / 4, dims 4 (lane % 4) ..
      const uint16_t* vt_src = nullptr;
      if constexpr (TV) {
        uint16_t* vt = reinterpret_cast<uint16_t*>(s_lds);
        if constexpr (kB == 2) {
#pragma unroll
          for (int i = 0; i < C::kKLoads; ++i)
            *reinterpret_cast<u32x4*>(vt + col * kVRow + qk_dim<2>(i, j)) = vr[i];
        } else {
#pragma unroll
          for (int a = 0; a < C::kKLoads; ++a) {
            const u32x2 b0 = e4m3x4_to_bf16x4(vr[a].x), b1 = e4m3x4_to_bf16x4(vr[a].y);
            const u32x2 b2 = e4m3x4_to_bf16x4(vr[a].z), b3 = e4m3x4_to_bf16x4(vr[a].w);
            uint16_t* dst = vt + col * kVRow + qk_dim<1>(2 * a, j);
            *reinterpret_cast<u32x4*>(dst) = u32x4{b0.x, b0.y, b1.x, b1.y};
            *reinterpret_cast<u32x4*>(dst + 8) = u32x4{b2.x, b2.y, b3.x, b3.y};
          }
        }
        wave_lds_sync();
        vt_src = vt + (4 * j + (col >> 2)) * kVRow + 4 * (col & 3);
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        u32x2 vop;
        if constexpr (TV) {
          vop = lds_read_tr16(vt_src + 16 * nt);
        } else if constexpr (kB == 2) {
          vop = vr[nt];
        } else {
          vop = e4m3x4_to_bf16x4(vr[nt]);
        }
        vop.x &= vmask.x;
        vop.y &= vmask.y;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[ct][nt] = mfma_16x16x16<QT>(phi[ct], vop, acc[ct][nt]);
          acc[ct][nt] = mfma_16x16x16<QT>(plo[ct], vop, acc[ct][nt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_v(next, vr);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

}

// Row sums and normalised rows of a finished vt_attend, in LDS: s_out[r][D]
// for every row r < nrows (rows = q rows of the wave, LDS owned by the
// wave). Returns in lane r (r < 16) the weight sum of row r.
template <int D>
__device__ __forceinline__ float vt_normalise(const f32x4 (&acc)[D / 16], float l_w, float v_scale, int nrows,
                                              float* s_out) {
  constexpr int kNT = D / 16;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, j = lane >> 4;
  float l_head = l_w + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, l_w), 0x401F));
  l_head += __shfl_xor(l_head, 32, 64);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * j + r;
    const float lr = __shfl(l_head, h, 64);  // lane h (row 0) holds row h's sum
    if (h < nrows) {
      const float inv = v_scale / lr;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) s_out[h * D + nt * 16 + col] = acc[nt][r] * inv;
    }
  }
  wave_lds_sync();
  return l_head;
}

// One (partition, sequence, KV head) unit of the partition kernel. wg =
// the unit's index in partition-major order over `pairs` = B * Hkv
// (sequence, head) pairs; s_out = the wave's G x D floats of LDS. With
// p.shared_len (pa_decode_shared) partition indices count from the
// sequence's first partition past its shared prefix (the shared ones are
// computed once per group).
template <typename KV, typename QT, int D, int BS, int G, bool TV>
__device__ __forceinline__ void vt_unit(const DecodeParams& p, int wg, int pairs, float* s_out) {
  using C = DecodeCfg<KV, D, BS, G>;
  constexpr int kB = C::kB;
  constexpr int kNT = D / 16;  // 16-dim output tiles
  static_assert(G <= 16, "at most 16 query heads per KV head");

  const int part0 = wg / pairs;
  const int pr = wg - part0 * pairs;
  const int s = pr / p.num_kv_heads;
  const int g = pr - s * p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int32_t* bt = p.block_tables + static_cast<int64_t>(s) * p.max_blocks;
  int id_first = 0;
  if (p.shared_len == nullptr) {
    // the table entries of the partition, requested together with the length
    const int blk_first = p.partition_size > 0 ? part0 * p.partition_size / BS : 0;
    id_first = blk_first + lane < p.max_blocks ? bt[blk_first + lane] : 0;
  }

  int L = p.context_lens[s];
  L = L < p.len_cap ? L : p.len_cap;
  L = L > 0 ? L : 0;
  const int ps = p.partition_size > 0 ? p.partition_size : (L > 0 ? L : 1);
  const int nparts = (L + ps - 1) / ps;
  const int part = p.shared_len == nullptr ? part0 : part0 + p.shared_len[s] / ps;
  if (part >= (nparts > 0 ? nparts : 1)) return;
  if (p.shared_len != nullptr) {
    const int blk_first = part * ps / BS;
    id_first = blk_first + lane < p.max_blocks ? bt[blk_first + lane] : 0;
  }
  const int64_t head0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(g) * G;
  if (L == 0) {
    for (int i = lane; i < G * D; i += 64) store_out(p.out, head0 * D + i, p.out_dtype, 0.f);
    return;
  }
  const int tok_begin = part * ps;
  const int tok_end = min(L, tok_begin + ps);
  const int col = lane & 15, j = lane >> 4;

  // q rows as the B operand of S^T = K q^T (columns >= G are zero)
  u32x4 qb[1][C::kKSteps];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (head0 + (col < G ? col : 0)) * D;
#pragma unroll
    for (int i = 0; i < C::kKSteps; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + qk_dim<kB>(i, j));
      qb[0][i] = col < G ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m_w[1] = {-INFINITY};
  float l_w[1] = {0.f};
  const bool row_ok[1] = {col < G};
  f32x4 acc[1][kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) acc[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  vt_attend<KV, QT, D, BS, G, TV>(p, bt, g, L, tok_begin, tok_end, id_first, qb, row_ok, m_w, l_w, acc, s_out);

  // ---- epilogue: normalised rows through LDS for wide stores
  const float l_head = vt_normalise<D>(acc[0], l_w[0], p.v_scale, G, s_out);
  for (int i = lane * 8; i < G * D; i += 64 * 8) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = s_out[i + e];
    const int h = i / D, d = i % D;
    if (nparts == 1) {
      store_out8(p.out, (head0 + h) * D + d, p.out_dtype, o);
    } else {
      const int64_t pi = (head0 + h) * p.num_partitions + part;
      float* po = p.part_o + pi * D + d;
      *reinterpret_cast<f32x4*>(po) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(po + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
  }
  if (nparts > 1 && lane < G) {
    const int64_t pi = (head0 + lane) * p.num_partitions + part;
    p.part_m[pi] = m_w[0];
    p.part_l[pi] = l_head;
  }
}

template <typename KV, typename QT, int D, int BS, int G, bool TV>
__global__ __launch_bounds__(64) void paged_decode_vt_kernel(const DecodeParams p) {
  // the output tile (G x D floats), which holds the V tile while the unit
  // runs (token-major V)
  __shared__ float s_out[TV && vt_tile_floats(D) > G * D ? vt_tile_floats(D) : G * D];
  vt_unit<KV, QT, D, BS, G, TV>(p, static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x) / p.num_partitions,
                                s_out);
}

template <typename KV, typename QT, int D, int BS, int G, bool TV>
hipError_t launch_decode_vt(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_vt_kernel<KV, QT, D, BS, G, TV>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <typename KV, typename QT, int D, int BS, bool TV>
DecodeLaunch select_decode_vt_g(int G) {
  switch (G) {
    case 1: return &launch_decode_vt<KV, QT, D, BS, 1, TV>;
    case 2: return &launch_decode_vt<KV, QT, D, BS, 2, TV>;
    case 4: return &launch_decode_vt<KV, QT, D, BS, 4, TV>;
    case 8: return &launch_decode_vt<KV, QT, D, BS, 8, TV>;
    default: return nullptr;
  }
}

template <typename KV, typename QT, int D, bool TV>
DecodeLaunch select_decode_vt_bs(int BS, int G) {
  switch (BS) {
    case 8: return select_decode_vt_g<KV, QT, D, 8, TV>(G);
    case 16: return select_decode_vt_g<KV, QT, D, 16, TV>(G);
    case 32: return select_decode_vt_g<KV, QT, D, 32, TV>(G);
    default: return nullptr;
  }
}

// TV = token-major V blocks
template <typename KV, typename QT, bool TV>
DecodeLaunch select_decode_vt(int D, int BS, int G) {
  switch (D) {
    case 64: return select_decode_vt_bs<KV, QT, 64, TV>(BS, G);
    case 128: return select_decode_vt_bs<KV, QT, 128, TV>(BS, G);
    default: return nullptr;
  }
}

}  // namespace pa
