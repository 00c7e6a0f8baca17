// pa_decode entry point: argument validation, kernel selection, and the
// log-sum-exp merge of context partitions.
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving.
// The pages do not describe a split of long contexts; splitting a context
// into partitions and merging them is exact because softmax attention over
// a sequence equals the weighted merge of attention over consecutive parts:
//   out = sum_p w_p o_p / sum_p w_p,   w_p = l_p * 2^(m_p - max_q m_q)
// where o_p is partition p's normalised output, l_p its sum of weights and
// m_p its running max (log2 domain). [course] §9 "Observations from Real
// Systems" notes long-context serving is gated by blocks per sequence; the
// partitions keep one long sequence from serialising on one workgroup.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "decode_common.h"
#include "decode_shared_kernel.h"
#include "decode_sk_kernel.h"
#include "device_common.h"
#include "internal.h"

namespace pa {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct ReduceParams {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  void* out;
  const int32_t* context_lens;
  int32_t len_cap;
  int32_t partition_size;
  int32_t num_partitions;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t out_dtype;
};

// grid = (Hq, B); one thread per head-dim element. Sums run over partitions
// in index order, so the result does not depend on scheduling.
__global__ __launch_bounds__(128) void decode_reduce_kernel(const ReduceParams p) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int L = p.context_lens[s];
  L = L < p.len_cap ? L : p.len_cap;
  L = L > 0 ? L : 0;
  const int np = (L + p.partition_size - 1) / p.partition_size;
  if (np <= 1) return;  // written directly by the partition kernel
  const int64_t row = static_cast<int64_t>(s) * p.num_q_heads + h;
  const float* m = p.part_m + row * p.num_partitions;
  const float* l = p.part_l + row * p.num_partitions;
  const float* o = p.part_o + row * p.num_partitions * p.head_dim;
  float mmax = -INFINITY;
  for (int i = 0; i < np; ++i) mmax = fmaxf(mmax, m[i]);
  for (int d = threadIdx.x; d < p.head_dim; d += blockDim.x) {
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int i = 0; i < np; ++i) {
      const float w = l[i] * __builtin_amdgcn_exp2f(m[i] - mmax);
      den += w;
      num = fmaf(w, o[static_cast<int64_t>(i) * p.head_dim + d], num);
    }
    store_out(p.out, row * p.head_dim + d, p.out_dtype, num / den);
  }
}

// Merge the partial pieces of segments whose units span several
// workgroups, and write zeros for sequences without tokens.
struct SkMergeParams {
  const float* piece_m;
  const float* piece_l;
  const float* piece_o;
  const int32_t* seg_desc;  // [head groups][B][2]
  const int32_t* context_lens;
  void* out;
  int32_t len_cap;
  int32_t batch;
  int32_t num_q_heads;
  int32_t heads_per_wg;
  int32_t group;  // G
  int32_t head_dim;
  int32_t out_dtype;
  int32_t piece_slots;  // piece slots per workgroup (2 balanced, 1 partition mode)
};

// piece groups of a split merge workgroup: group g takes pieces g, g + 16, ...
constexpr int kMergeGroups = 16;

// Running log-sum-exp merge of the pieces wf + k_first, wf + k_first +
// k_step, ... (up to wl) of one segment, query head hq, head dims 8c..8c+7.
// The segment's descriptor (written by the balanced kernel, see
// decode_sk_kernel.h) names the workgroups wf..wl that hold its pieces:
// wf's in slot first_slot, the others' in slot 0. Up to kChunk pieces are
// read per round of loads.
template <int kChunk = 8>
__device__ __forceinline__ void merge_pieces(const SkMergeParams& p, int HWG, int hq, int c, int wf, int wl,
                                             int first_slot, int k_first, int k_step, float& run_m, float& den,
                                             float (&num)[8]) {
  const int D = p.head_dim;
  for (int k0 = k_first; wf + k0 <= wl; k0 += k_step * kChunk) {
    float pm[kChunk], pl[kChunk];
    f32x4 pa[kChunk], pb[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const int wv = wf + k0 + k * k_step;
      const bool valid = wv <= wl;
      const int wr = valid ? wv : wf;  // past wl: read wf's piece, weight 0
      const int slot = wr == wf ? first_slot : 0;
      const int64_t pi = (static_cast<int64_t>(wr) * p.piece_slots + slot) * HWG + hq;
      pm[k] = valid ? p.piece_m[pi] : -INFINITY;
      pl[k] = p.piece_l[pi];
      const f32x4* po = reinterpret_cast<const f32x4*>(p.piece_o + pi * D + 8 * c);
      pa[k] = po[0];
      pb[k] = po[1];
    }
    float cm = run_m;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) cm = fmaxf(cm, pm[k]);
    // pieces with m = -inf (past wl, or a workgroup without units) weigh 0
    const float r = run_m > -INFINITY ? __builtin_amdgcn_exp2f(run_m - cm) : 0.f;
    den *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] *= r;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float wt = pm[k] > -INFINITY ? pl[k] * __builtin_amdgcn_exp2f(pm[k] - cm) : 0.f;
      den += wt;
      num[0] = fmaf(wt, pa[k].x, num[0]);
      num[1] = fmaf(wt, pa[k].y, num[1]);
      num[2] = fmaf(wt, pa[k].z, num[2]);
      num[3] = fmaf(wt, pa[k].w, num[3]);
      num[4] = fmaf(wt, pb[k].x, num[4]);
      num[5] = fmaf(wt, pb[k].y, num[5]);
      num[6] = fmaf(wt, pb[k].z, num[6]);
      num[7] = fmaf(wt, pb[k].w, num[7]);
    }
    run_m = cm;
  }
}

// Two layouts of the merge grid:
//  * SPLIT = false: one workgroup per (head group, sequence) segment, one
//    thread per 8 head dims of each query head of the group; a thread walks
//    all of the segment's pieces (one round of loads per 8). Few
//    workgroups: right when segments span few workgroups.
//  * SPLIT = true: one workgroup per (segment, query head), D / 8 threads
//    per piece group; kMergeGroups piece groups read up to 128 pieces in one
//    round, and their partial merges are combined through LDS. Right when
//    segments span many workgroups (few long sequences).
template <bool SPLIT>
__global__ __launch_bounds__(1024) void decode_sk_merge_kernel(const SkMergeParams p) {
  const int HWG = p.heads_per_wg * p.group;  // query heads per head group
  const int D = p.head_dim;
  const int tpr = D / 8;
  const int bx = static_cast<int>(blockIdx.x);
  const int seg = SPLIT ? bx / HWG : bx;
  const int s = seg % p.batch;
  const int hg = seg / p.batch;
  const int t = static_cast<int>(threadIdx.x);
  const int hq = SPLIT ? bx % HWG : t / tpr;
  const int c = t % tpr;
  const int pg = SPLIT ? t / tpr : 0;
  if (!SPLIT && hq >= HWG) return;
  const int64_t orow = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(hg) * HWG + hq;
  const int L = min(p.context_lens[s], p.len_cap);
  const int32_t* desc = p.seg_desc + (static_cast<int64_t>(hg) * p.batch + s) * 2;
  const int32_t d0 = desc[0], d1 = desc[1];
  if (L <= 0) {
    if (pg == 0) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      store_out8(p.out, orow * D + 8 * c, p.out_dtype, z);
    }
    return;
  }
  if (d0 == -1) return;  // stored by the workgroup that completed it
  const int wf = d0 & 0x7fffffff, wl = d1;
  const int first_slot = static_cast<int>(static_cast<uint32_t>(d0) >> 31);
  float run_m = -INFINITY, den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  merge_pieces(p, HWG, hq, c, wf, wl, first_slot, pg, SPLIT ? kMergeGroups : 1, run_m, den, num);
  if constexpr (SPLIT) {
    __shared__ float s_m[kMergeGroups], s_den[kMergeGroups];
    __shared__ float s_num[kMergeGroups * 128];
    if (c == 0) {
      s_m[pg] = run_m;
      s_den[pg] = den;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_num[pg * D + 8 * c + e] = num[e];
    __syncthreads();
    if (pg != 0) return;
    float mx = s_m[0];
    for (int g = 1; g < kMergeGroups; ++g) mx = fmaxf(mx, s_m[g]);
    den = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = 0.f;
    for (int g = 0; g < kMergeGroups; ++g) {
      const float w = s_m[g] > -INFINITY ? __builtin_amdgcn_exp2f(s_m[g] - mx) : 0.f;
      den = fmaf(w, s_den[g], den);
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] = fmaf(w, s_num[g * D + 8 * c + e], num[e]);
    }
  }
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = num[e] / den;
  store_out8(p.out, orow * D + 8 * c, p.out_dtype, o);
}

// ---- the cascade's merge (pa_decode_shared on the balanced kernel): each
// row's output is the log-sum-exp merge of its prefix part (its group's
// shared tokens) and its tail part (its own tokens), each part either a
// state row (one workgroup completed it) or pieces (cut between
// workgroups; piece rows RW = 32 per wave: the prefix's member-major rows,
// or a tail's G heads).
struct CasMergeParams {
  SkMergeParams pieces;  // piece arrays, slots, shape, lengths, out
  const float* state_m;  // [2][B][num_q_heads]: prefix part, then tail part
  const float* state_l;
  const float* state_o;  // [2][B][num_q_heads][D]
  const int32_t* row_map;  // [B][4]: group (or -1), place in the group, has a tail
  int32_t num_groups;
};

constexpr int kCasPieceRows = 32;  // piece rows per wave (two 16-row tiles)
constexpr int kCasMergeGroups = 4;  // piece groups of a cascade merge workgroup

// grid = B x num_kv_heads (row-major); kCasMergeGroups groups of G x D / 8
// threads (one per 8 head dims of each query head of the KV head): group g
// merges pieces g, g + 4, ... of each part (a state row counts as group 0's
// one piece), then group 0 combines the four partial merges through LDS.
__global__ __launch_bounds__(512) void decode_cascade_merge_kernel(const CasMergeParams p) {
  const SkMergeParams& m = p.pieces;
  const int G = m.group;
  const int HW = m.heads_per_wg;
  const int HWG = HW * G;
  const int D = m.head_dim;
  const int tpr = D / 8;
  const int B = m.batch;
  const int hkv = m.num_q_heads / G;
  const int s = static_cast<int>(blockIdx.x) / hkv;
  const int g = static_cast<int>(blockIdx.x) % hkv;
  const int hg = g / HW, wave = g % HW;
  const int t = static_cast<int>(threadIdx.x);
  const int per = G * tpr;  // threads per piece group
  const int pg = t / per;
  const int h = (t % per) / tpr;
  const int c = t % tpr;
  const bool active = pg < kCasMergeGroups;
  const int hq = wave * G + h;
  const int64_t head = static_cast<int64_t>(hg) * HWG + hq;
  const int64_t orow = static_cast<int64_t>(s) * m.num_q_heads + head;
  const int L = min(m.context_lens[s], m.len_cap);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (L <= 0) {
    if (active && pg == 0) store_out8(m.out, orow * D + 8 * c, m.out_dtype, o);
    return;
  }
  const int NG = p.num_groups;
  const int NV = NG + B;
  // the row map and both descriptors (the prefix's at a valid place even
  // for rows without a prefix: the cascade runs with groups)
  const int32_t* rm = p.row_map + 4 * static_cast<int64_t>(s);
  const int32_t* tdesc = m.seg_desc + (static_cast<int64_t>(hg) * NV + NG + s) * 2;
  const int gi = rm[0], mi = rm[1], has_tail = rm[2];
  const int32_t t0 = tdesc[0], t1 = tdesc[1];
  const int32_t* pdesc = m.seg_desc + (static_cast<int64_t>(hg) * NV + (gi >= 0 ? gi : 0)) * 2;
  const int32_t p0 = pdesc[0], p1 = pdesc[1];
  float run_m = -INFINITY, den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // part `part` with descriptor {d0, d1}; r = the row among the wave's
  // piece rows
  auto add_part = [&](int part, int32_t d0, int32_t d1, int r) {
    if (d0 != -1) {
      merge_pieces<4>(m, HW * kCasPieceRows, wave * kCasPieceRows + r, c, d0 & 0x7fffffff, d1,
                      static_cast<int>(static_cast<uint32_t>(d0) >> 31), pg, kCasMergeGroups, run_m, den, num);
      return;
    }
    if (pg != 0) return;
    const int64_t row = (static_cast<int64_t>(part) * B + s) * m.num_q_heads + head;
    const float pm = p.state_m[row];
    const float pl = p.state_l[row];
    const f32x4* po = reinterpret_cast<const f32x4*>(p.state_o + row * D + 8 * c);
    const f32x4 pa = po[0], pb = po[1];
    const float cm = fmaxf(run_m, pm);
    const float r0 = run_m > -INFINITY ? __builtin_amdgcn_exp2f(run_m - cm) : 0.f;
    const float wt = pm > -INFINITY ? pl * __builtin_amdgcn_exp2f(pm - cm) : 0.f;
    den = den * r0 + wt;
    const float v8[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = fmaf(wt, v8[e], num[e] * r0);
    run_m = cm;
  };
  if (active) {
    if (has_tail) add_part(1, t0, t1, h);
    if (gi >= 0) add_part(0, p0, p1, mi * G + h);
  }
  // combine the groups' partial merges (G x D floats each)
  __shared__ float s_m[kCasMergeGroups][8], s_den[kCasMergeGroups][8];
  __shared__ float s_num[kCasMergeGroups][8 * 128];
  if (active) {
    if (c == 0) {
      s_m[pg][h] = run_m;
      s_den[pg][h] = den;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_num[pg][h * D + 8 * c + e] = num[e];
  }
  __syncthreads();
  if (!active || pg != 0) return;
  float mx = s_m[0][h];
  for (int k = 1; k < kCasMergeGroups; ++k) mx = fmaxf(mx, s_m[k][h]);
  float dsum = 0.f, acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kCasMergeGroups; ++k) {
    const float w = s_m[k][h] > -INFINITY ? __builtin_amdgcn_exp2f(s_m[k][h] - mx) : 0.f;
    dsum = fmaf(w, s_den[k][h], dsum);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = fmaf(w, s_num[k][h * D + 8 * c + e], acc8[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = dsum > 0.f ? acc8[e] / dsum : 0.f;
  store_out8(m.out, orow * D + 8 * c, m.out_dtype, o);
}

int out_code(pa_dtype t) { return t == PA_F32 ? 2 : (t == PA_BF16 ? 1 : 0); }

int64_t partitions_for(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || max_context_len <= partition_size) return 1;
  return (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size;
}

// workspace of a partitioned call: per (sequence, query head, partition)
// m, l, o[D], then (partition mode of the staged kernel) the merge
// descriptors [num_kv_heads][B][2]
size_t workspace_bytes_for(int64_t B, int64_t Hq, int64_t hkv, int64_t D, int64_t P) {
  if (P <= 1) return 0;
  const size_t rows = static_cast<size_t>(B * Hq * P);
  return 2 * align_up(rows * sizeof(float)) + align_up(rows * D * sizeof(float)) +
         align_up(static_cast<size_t>(B * hkv) * 2 * sizeof(int32_t));
}

// ---- balanced split
// At most kSkWavesPerCu waves of the balanced kernel per CU: it bounds the
// grid, so the piece buffers can be sized before the launch.
constexpr int kSkWavesPerCu = 32;

// LDS one workgroup of the balanced kernel may use: 64 KiB, or with the
// stage (token-major V, fp8 pools) up to gfx950's 160 KiB, as far as the
// device allows per workgroup (sk_device_lds)
constexpr size_t kSkMaxLds = 64 * 1024;
constexpr size_t kSkMaxLdsStage = 160 * 1024;

// LDS the current device allows one workgroup (cached per device; 0 if it
// cannot be read)
size_t sk_device_lds() {
  static DeviceIntCache cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int n = cache.get(dev, [dev]() {
    int v = 0, optin = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) == hipSuccess && optin > v)
      v = optin;
    return v;
  });
  return n > 0 ? static_cast<size_t>(n) : 0;
}

// KV heads per workgroup: the largest divisor of num_kv_heads up to 8 (a
// power of two when staged: the stage splits a row slice by shifts)
int sk_heads_per_wg(int hkv, bool staged) {
  for (int hw = 8; hw > 1; --hw)
    if (hkv % hw == 0 && (!staged || (hw & (hw - 1)) == 0)) return hw;
  return 1;
}

// CUs of the current device (cached per device)
int device_cus() {
  static DeviceIntCache cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int n = cache.get(dev, [dev]() {
    int v = 0;
    return hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? v : 0;
  });
  return n > 0 ? n : 0;
}

struct SkLayout {
  size_t desc, m, l, o, total;  // byte offsets and total size
};

// workspace of the balanced split: merge descriptors [head groups][B][2],
// then per piece row (workgroup, slot, query head of the group) m, l, o[D],
// for `rows` piece rows
SkLayout sk_layout_rows(int64_t B, int64_t hkv, int64_t D, size_t rows) {
  SkLayout L{};
  L.desc = 0;
  L.m = align_up(static_cast<size_t>(B) * hkv * 2 * sizeof(int32_t));
  L.l = L.m + align_up(rows * sizeof(float));
  L.o = L.l + align_up(rows * sizeof(float));
  L.total = L.o + align_up(rows * D * sizeof(float));
  return L;
}

// the layout pa_decode_workspace_size promises: W * HW <= cus *
// kSkWavesPerCu, and a workgroup holds 2 * HW * G rows
SkLayout sk_layout(int64_t B, int64_t Hq, int64_t hkv, int64_t D, int cus) {
  const int64_t G = Hq / hkv;
  return sk_layout_rows(B, hkv, D, static_cast<size_t>(cus) * kSkWavesPerCu * 2 * G);
}

// workspace of the cascade (pa_decode_shared on the balanced kernel):
// merge descriptors [head groups][num_groups + B][2], the row map [B][4],
// the state rows m, l [2][B][Hq] and o [2][B][Hq][D], then the pieces: per
// piece row (workgroup, slot, wave, 32 rows) m, l, o[D], for `wgs`
// workgroups of hw waves
struct CasLayout {
  size_t desc, map, sm, sl, so, pm, pl, po, total;
};
CasLayout cas_layout(int64_t B, int64_t Hq, int64_t hkv, int64_t hw, int64_t D, int64_t groups, int64_t wgs) {
  CasLayout L{};
  const size_t srows = static_cast<size_t>(2 * B * Hq);
  const size_t prows = static_cast<size_t>(wgs * 2 * hw * kCasPieceRows);
  L.desc = 0;
  L.map = align_up(static_cast<size_t>((hkv / hw) * (groups + B) * 2) * sizeof(int32_t));
  L.sm = L.map + align_up(static_cast<size_t>(B) * 4 * sizeof(int32_t));
  L.sl = L.sm + align_up(srows * sizeof(float));
  L.so = L.sl + align_up(srows * sizeof(float));
  L.pm = L.so + align_up(srows * D * sizeof(float));
  L.pl = L.pm + align_up(prows * sizeof(float));
  L.po = L.pl + align_up(prows * sizeof(float));
  L.total = L.po + align_up(prows * D * sizeof(float));
  return L;
}

// the cascade workspace pa_decode_workspace_size promises for partitioned
// calls: any grouping of the batch (at most B groups), one workgroup of 8
// waves per CU (the cascade's 8-wave workgroups use more than half of a
// SIMD's registers, so at most that many are resident)
size_t cas_workspace_bound(int64_t B, int64_t Hq, int64_t hkv, int64_t D, int cus) {
  const int64_t hw = sk_heads_per_wg(static_cast<int>(hkv), true);
  return cas_layout(B, Hq, hkv, hw, D, B, static_cast<int64_t>(cus) * std::max<int64_t>(1, 8 / hw)).total;
}

}  // namespace

// The balanced split: one launch of the persistent kernel over the device's
// resident workgroups, then the merge of sequences cut between them. The
// arguments are validated by pa_decode.
// With k_new != nullptr it is the append variant (pa_decode_append).
// With partition_size >= 0 (num_parts partitions; 0: one per sequence) the
// same kernel runs in partition mode: one workgroup per (head group,
// sequence, partition), merged by the same merge kernel (the partitioned
// path for token-major V and fp8 pools).
pa_status decode_balanced(const pa_kv_cache* cache, void* out, int out_code, const void* q,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                          int32_t num_q_heads, int32_t max_context_len, float qk_scale_log2, float v_scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream, int32_t partition_size = -1,
                          int64_t num_parts = 0, const void* k_new = nullptr, const void* v_new = nullptr,
                          const int64_t* slot_mapping = nullptr, bool fit_workspace = false) {
  const bool part_mode = partition_size >= 0;
  const int32_t hkv = cache->num_kv_heads;
  const int32_t D = cache->head_dim;
  const int32_t G = num_q_heads / hkv;
  const bool append = k_new != nullptr;
  const bool tv = cache->v_layout == PA_LAYOUT_TOKEN_MAJOR;
  const SkLaunch launch = find_decode_sk(cache->dtype, cache->v_layout, D, cache->block_size, G, append);
  if (launch == nullptr)
    return fail(PA_ERR_UNSUPPORTED,
                "no balanced decode%s kernel for pool dtype %d, %s V, head_dim %d, block_size %d, group %d%s",
                append ? " + append" : "", (int)cache->dtype, tv ? "token-major" : "dim-major", D, cache->block_size, G,
                append ? " (append: F16 and BF16 pools)" : "");
  // the kernel stages whole rows through LDS for token-major V and fp8 pools
  const bool staged = tv || cache->dtype == PA_FP8_E4M3;
  // partition mode: at most 4 KV heads per workgroup, so that two
  // workgroups share a CU and overlap their starts
  const int HW = part_mode ? std::min(sk_heads_per_wg(hkv, staged), 4) : sk_heads_per_wg(hkv, staged);
  const int n_hg = hkv / HW;
  const size_t lds = sk_lds_bytes(B, HW, G, D, staged, cache->dtype == PA_FP8_E4M3 ? 1 : 2, tv, 1, append);
  if (lds > (staged ? kSkMaxLdsStage : kSkMaxLds))
    return fail(PA_ERR_UNSUPPORTED, "B = %d is too large for the balanced split (use partition_size > 0)", B);
  // units (tiles x head groups) must stay below 2^31; counted in 16-token
  // tiles, an upper bound for the 32-token tiles of fp8 pools
  if (static_cast<int64_t>(B) * ((static_cast<int64_t>(max_context_len) + 15) / 16) * n_hg > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "B x max_context_len is too large for the balanced split");
  // the merge grid, at most one workgroup of D / 8 * kMergeGroups threads
  // per (sequence, query head) (its split layout)
  if (static_cast<int64_t>(B) * num_q_heads * (D / 8 * kMergeGroups) > 0xffffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "B x num_q_heads is too large for the balanced split");
  if (!part_mode && workspace == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "the balanced split needs a workspace");
  const int cus = device_cus();
  if (cus <= 0) return fail(PA_ERR_DEVICE, "cannot read the device's CU count");
  if (lds > kSkMaxLds) {
    const size_t dev_lds = sk_device_lds();
    if (dev_lds == 0) return fail(PA_ERR_DEVICE, "cannot read the device's LDS size");
    if (lds > dev_lds)
      return fail(PA_ERR_UNSUPPORTED, "the balanced split needs %zu bytes of LDS per workgroup (device: %zu)", lds,
                  dev_lds);
  }
  // staged: two stages (one barrier per unit instead of two) when the
  // workgroups that hold 8 waves per CU still fit a CU's LDS with them
  int stage_bufs = 1;
  if (staged) {
    const size_t lds2 = sk_lds_bytes(B, HW, G, D, true, cache->dtype == PA_FP8_E4M3 ? 1 : 2, tv, 2, append);
    const size_t dev_lds = sk_device_lds();
    const size_t per_cu = static_cast<size_t>(std::max(1, 8 / HW));
    if (dev_lds > 0 && lds2 <= dev_lds && lds2 * per_cu <= kSkMaxLdsStage) stage_bufs = 2;
    if (const char* v = std::getenv("PA_SK_STAGES")) {  // measurement aid
      if (std::atoi(v) == 1) stage_bufs = 1;
    }
  }
  SkLayout lay{};
  // grid bound of the balanced split (the launch takes at most the resident
  // workgroups, fewer if max_wgs is lower)
  int max_wgs = cus * kSkWavesPerCu / HW;
  if (part_mode) {
    // [m][l][o] per (sequence, query head, partition) = per piece row of
    // workgroup ((hg * B + s) * P + part), then the descriptors (the caller
    // checked the size; none is needed for one partition)
    const size_t rows = static_cast<size_t>(B) * num_q_heads * num_parts;
    lay.m = 0;
    lay.l = align_up(rows * sizeof(float));
    lay.o = 2 * align_up(rows * sizeof(float));
    lay.desc = lay.o + align_up(rows * D * sizeof(float));
  } else {
    lay = sk_layout(B, num_q_heads, hkv, D, cus);
    if (fit_workspace && workspace != nullptr && workspace_bytes < lay.total) {
      // a fixed buffer (pa_decode_noalloc): size the pieces for as many
      // workgroups as it holds, which bounds the grid; the launch takes
      // fewer only when that is below the resident workgroups
      const size_t per_wg = static_cast<size_t>(2) * HW * G;  // piece rows of a workgroup
      const size_t fixed = align_up(static_cast<size_t>(B) * hkv * 2 * sizeof(int32_t)) + 3 * kAlign;
      const size_t wg_bytes = per_wg * (2 + static_cast<size_t>(D)) * sizeof(float);
      int64_t fit = workspace_bytes > fixed ? static_cast<int64_t>((workspace_bytes - fixed) / wg_bytes) : 0;
      fit = std::min<int64_t>(fit, max_wgs);
      while (fit > 0 && sk_layout_rows(B, hkv, D, static_cast<size_t>(fit) * per_wg).total > workspace_bytes) --fit;
      if (fit <= 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "the balanced split of B = %d needs more than %zu bytes of scratch", B,
                    workspace_bytes);
      max_wgs = static_cast<int>(fit);
      lay = sk_layout_rows(B, hkv, D, static_cast<size_t>(fit) * per_wg);
    }
    if (workspace == nullptr || workspace_bytes < lay.total)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes needed (got %zu)", lay.total,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  const bool merge = !part_mode || num_parts > 1;
  char* ws = static_cast<char*>(workspace);
  SkParams p{};
  p.q = q;
  p.k_pool = cache->k;
  p.v_pool = cache->v;
  p.out = out;
  if (merge) {
    p.piece_m = reinterpret_cast<float*>(ws + lay.m);
    p.piece_l = reinterpret_cast<float*>(ws + lay.l);
    p.piece_o = reinterpret_cast<float*>(ws + lay.o);
    p.seg_desc = reinterpret_cast<int32_t*>(ws + lay.desc);
  }
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.block_stride = cache->block_stride;
  p.num_blocks = cache->num_blocks;
  p.num_kv_heads = hkv;
  p.num_q_heads = num_q_heads;
  p.max_blocks = max_blocks;
  p.len_cap = max_context_len;
  p.batch = B;
  p.heads_per_wg = HW;
  p.num_head_groups = n_hg;
  p.piece_slots = part_mode ? 1 : 2;
  p.stage_bufs = stage_bufs;
  if (part_mode) {
    // tiles per partition: 16 tokens (32 for fp8 pools; the caller keeps
    // partition_size a multiple of it, or uses one partition)
    const int tt = cache->dtype == PA_FP8_E4M3 ? 32 : 16;
    p.part_tiles = num_parts > 1 ? partition_size / tt : std::max(1, (max_context_len + tt - 1) / tt);
    p.num_parts = static_cast<int32_t>(num_parts);
  }
  p.out_dtype = out_code;
  p.qk_scale_log2 = qk_scale_log2;
  p.v_scale = v_scale;
  p.k_new = k_new;
  p.v_new = v_new;
  p.slot_mapping = slot_mapping;
  if (part_mode) {
    const int64_t grid = num_parts * B * n_hg;
    if (grid > 0x7fffffffLL) return fail(PA_ERR_INVALID_ARGUMENT, "too many workgroups (%lld)", (long long)grid);
    max_wgs = static_cast<int>(grid);
  } else if (const char* cap = std::getenv("PA_SK_WGS")) {
    const int v = std::atoi(cap);
    if (v > 0 && v < max_wgs) max_wgs = v;
  }
  int wgs = 0;
  hipError_t e = launch(p, cus, max_wgs, stream, &wgs);
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "balanced decode launch: %s", hipGetErrorString(e));
  if (!merge) return PA_OK;
  SkMergeParams m{};
  m.piece_m = p.piece_m;
  m.piece_l = p.piece_l;
  m.piece_o = p.piece_o;
  m.seg_desc = p.seg_desc;
  m.context_lens = context_lens;
  m.out = out;
  m.len_cap = max_context_len;
  m.batch = B;
  m.num_q_heads = num_q_heads;
  m.heads_per_wg = HW;
  m.group = G;
  m.head_dim = D;
  m.out_dtype = out_code;
  m.piece_slots = p.piece_slots;
  // segments that span many workgroups on average (fewer segments than a
  // quarter of the workgroups) take the split merge; so does partition mode
  // always, whose result must not depend on the rest of the batch (the
  // merge layout sets the rounding order)
  if (part_mode || static_cast<int64_t>(B) * n_hg * 4 < wgs) {
    const int64_t merge_wgs = static_cast<int64_t>(B) * n_hg * HW * G;
    hipLaunchKernelGGL(decode_sk_merge_kernel<true>, dim3(static_cast<uint32_t>(merge_wgs)), dim3(D / 8 * kMergeGroups),
                       0, stream, m);
  } else {
    const int merge_threads = (HW * G * D / 8 + 63) / 64 * 64;
    hipLaunchKernelGGL(decode_sk_merge_kernel<false>, dim3(B * n_hg), dim3(merge_threads), 0, stream, m);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "balanced decode merge launch: %s", hipGetErrorString(e));
  return PA_OK;
}

// pa_decode_shared on the balanced kernel's cascade variant (see
// decode_sk_kernel.h): one launch over the prefixes of the groups and the
// tails of the rows, then decode_cascade_merge_kernel. Returns
// PA_ERR_UNSUPPORTED without launching anything when this shape has no
// cascade build or does not fit it (the caller then takes the
// shared-prefix partition kernels). Arguments are validated by the caller.
pa_status decode_cascade(const pa_kv_cache* cache, void* out, int out_code, const void* q,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                         int32_t num_q_heads, int32_t max_context_len, float qk_scale_log2, float v_scale,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         const int32_t* group_offsets, const int32_t* group_members, const int32_t* shared_len,
                         int32_t num_groups, int32_t max_group_size) {
  const int32_t hkv = cache->num_kv_heads;
  const int32_t D = cache->head_dim;
  const int32_t G = num_q_heads / hkv;
  const bool tv = cache->v_layout == PA_LAYOUT_TOKEN_MAJOR;
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  const SkLaunch launch = find_decode_cas(cache->dtype, cache->v_layout, D, cache->block_size, G);
  // a prefix unit holds a group's rows in two 16-row tiles
  if (launch == nullptr || static_cast<int64_t>(max_group_size) * G > kCasPieceRows)
    return PA_ERR_UNSUPPORTED;
  const int HW = sk_heads_per_wg(hkv, true);
  const int n_hg = hkv / HW;
  const int kb = fp8 ? 1 : 2;
  const size_t lds = sk_lds_bytes(B, HW, G, D, true, kb, tv, 1, false, num_groups);
  const size_t dev_lds = sk_device_lds();
  const int cus = device_cus();
  if (dev_lds == 0 || lds > dev_lds || lds > kSkMaxLdsStage || cus <= 0) return PA_ERR_UNSUPPORTED;
  // units: tiles of the tails (at most the rows' tiles plus one each) and
  // of the prefixes (at most max_context_len each), per head group
  const int64_t tiles = (static_cast<int64_t>(B) + num_groups) * ((static_cast<int64_t>(max_context_len) + 15) / 16 + 1);
  if (tiles * n_hg > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  int stage_bufs = 1;
  {
    const size_t lds2 = sk_lds_bytes(B, HW, G, D, true, kb, tv, 2, false, num_groups);
    if (lds2 <= dev_lds && lds2 * static_cast<size_t>(std::max(1, 8 / HW)) <= kSkMaxLdsStage) stage_bufs = 2;
  }
  // pieces for as many workgroups as the workspace holds (at most the
  // resident ones)
  int64_t wgs = static_cast<int64_t>(cus) * kSkWavesPerCu / HW;
  if (const char* cap = std::getenv("PA_SK_WGS")) {  // measurement aid
    const int v = std::atoi(cap);
    if (v > 0 && v < wgs) wgs = v;
  }
  while (wgs > 0 && cas_layout(B, num_q_heads, hkv, HW, D, num_groups, wgs).total > workspace_bytes) {
    const size_t fixed = cas_layout(B, num_q_heads, hkv, HW, D, num_groups, 0).total;
    const size_t per_wg = static_cast<size_t>(2) * HW * kCasPieceRows * (2 + static_cast<size_t>(D)) * sizeof(float);
    const int64_t fit = workspace_bytes > fixed ? static_cast<int64_t>((workspace_bytes - fixed) / per_wg) : 0;
    wgs = std::min(wgs - 1, fit);
  }
  // fewer than one workgroup per CU: the partition kernels serve better
  if (wgs < cus) return PA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const CasLayout lay = cas_layout(B, num_q_heads, hkv, HW, D, num_groups, wgs);
  char* ws = static_cast<char*>(workspace);
  SkParams p{};
  p.q = q;
  p.k_pool = cache->k;
  p.v_pool = cache->v;
  p.out = out;
  p.piece_m = reinterpret_cast<float*>(ws + lay.pm);
  p.piece_l = reinterpret_cast<float*>(ws + lay.pl);
  p.piece_o = reinterpret_cast<float*>(ws + lay.po);
  p.seg_desc = reinterpret_cast<int32_t*>(ws + lay.desc);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.block_stride = cache->block_stride;
  p.num_blocks = cache->num_blocks;
  p.num_kv_heads = hkv;
  p.num_q_heads = num_q_heads;
  p.max_blocks = max_blocks;
  p.len_cap = max_context_len;
  p.batch = B;
  p.heads_per_wg = HW;
  p.num_head_groups = n_hg;
  p.piece_slots = 2;
  p.stage_bufs = stage_bufs;
  p.out_dtype = out_code;
  p.qk_scale_log2 = qk_scale_log2;
  p.v_scale = v_scale;
  p.group_offsets = group_offsets;
  p.group_members = group_members;
  p.shared_len = shared_len;
  p.state_m = reinterpret_cast<float*>(ws + lay.sm);
  p.state_l = reinterpret_cast<float*>(ws + lay.sl);
  p.state_o = reinterpret_cast<float*>(ws + lay.so);
  p.row_map = reinterpret_cast<int32_t*>(ws + lay.map);
  p.num_groups = num_groups;
  int used = 0;
  hipError_t e = launch(p, cus, static_cast<int>(wgs), stream, &used);
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "cascade decode launch: %s", hipGetErrorString(e));
  CasMergeParams m{};
  m.pieces.piece_m = p.piece_m;
  m.pieces.piece_l = p.piece_l;
  m.pieces.piece_o = p.piece_o;
  m.pieces.seg_desc = p.seg_desc;
  m.pieces.context_lens = context_lens;
  m.pieces.out = out;
  m.pieces.len_cap = max_context_len;
  m.pieces.batch = B;
  m.pieces.num_q_heads = num_q_heads;
  m.pieces.heads_per_wg = HW;
  m.pieces.group = G;
  m.pieces.head_dim = D;
  m.pieces.out_dtype = out_code;
  m.pieces.piece_slots = 2;
  m.state_m = p.state_m;
  m.state_l = p.state_l;
  m.state_o = p.state_o;
  m.row_map = p.row_map;
  m.num_groups = num_groups;
  const int merge_threads = (kCasMergeGroups * G * D / 8 + 63) / 64 * 64;
  hipLaunchKernelGGL(decode_cascade_merge_kernel, dim3(static_cast<uint32_t>(B) * hkv), dim3(merge_threads), 0, stream,
                     m);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "cascade merge launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

using pa::fail;

extern "C" {

size_t pa_decode_workspace_size(int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size) {
  if (B <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  if (partition_size == PA_PARTITION_BALANCED) {
    if (num_q_heads % num_kv_heads != 0) return 0;
    const int cus = pa::device_cus();
    if (cus <= 0) return 0;
    return pa::sk_layout(B, num_q_heads, num_kv_heads, head_dim, cus).total;
  }
  if (max_context_len == 0) return 0;
  return pa::workspace_bytes_for(B, num_q_heads, num_kv_heads, head_dim,
                                 pa::partitions_for(max_context_len, partition_size));
}

size_t pa_decode_shared_workspace_size(int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0) return 0;
  const size_t part =
      pa_decode_workspace_size(B, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size);
  if (part == 0 || num_q_heads % num_kv_heads != 0) return part;
  const int cus = pa::device_cus();
  if (cus <= 0) return 0;
  return std::max(part, pa::cas_workspace_bound(B, num_q_heads, num_kv_heads, head_dim, cus));
}

}  // extern "C"

namespace pa {
namespace {

// whether the staged kernel can run a partitioned call of this shape (its
// LDS holds the batch's tile prefix; a larger batch takes the partition
// kernels)
bool sk_partition_fits(const pa_kv_cache* cache, int32_t B, int32_t G) {
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  const int HW = std::min(sk_heads_per_wg(cache->num_kv_heads, true), 4);
  return sk_lds_bytes(B, HW, G, cache->head_dim, true, fp8 ? 1 : 2, cache->v_layout == PA_LAYOUT_TOKEN_MAJOR) <=
         kSkMaxLdsStage;
}

// the group structure of pa_decode_shared
struct SharedArgs {
  const int32_t* group_offsets;
  const int32_t* group_members;
  const int32_t* shared_len;
  int32_t num_groups, max_group_size, max_shared_len, min_shared_len;
};

// ---- the scratch of pa_decode_noalloc: device memory the library owns,
// kScratchBytes on every GPU whose code object is loaded (held until the
// process ends). Host code never passes the array's name to a kernel or a
// copy: it is a host-side stand-in, not the device address. Each device's
// address comes from hipGetSymbolAddress with that device current, once,
// and is kept per device.
constexpr size_t kScratchBytes = 64ull << 20;
__device__ __align__(256) char scratch[kScratchBytes];

std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

pa_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_DEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(PA_ERR_DEVICE, "device %d: hipGetSymbolAddress(scratch): %s", dev, hipGetErrorString(e));
      if (reinterpret_cast<uintptr_t>(p) % kAlign != 0)
        return fail(PA_ERR_DEVICE, "device %d: the scratch is not %zu-byte aligned", dev, kAlign);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

// pa_decode; pa_decode_append when k_new != nullptr and pa_decode_shared
// when sh != nullptr (their own arguments are validated by them).
// fit_workspace (pa_decode_noalloc): the balanced split sizes its pieces for
// the workgroups the given buffer holds instead of requiring the bound
// pa_decode_workspace_size promises.
pa_status decode_impl(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                      int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, void* stream, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, const SharedArgs* sh = nullptr, bool fit_workspace = false) {
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (B < 0) return fail(PA_ERR_INVALID_ARGUMENT, "B = %d is negative", B);
  if (B == 0) return PA_OK;
  if (out == nullptr || q == nullptr || block_tables == nullptr || context_lens == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "out, q, block_tables or context_lens is NULL");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q)) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(context_lens)) % 4 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned, tables and lengths 4-byte aligned");
  const int32_t hkv = cache->num_kv_heads;
  const int32_t D = cache->head_dim;
  const int32_t bs = cache->block_size;
  if (num_q_heads <= 0 || num_q_heads % hkv != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, hkv);
  const int32_t G = num_q_heads / hkv;
  if (out_dtype != PA_F16 && out_dtype != PA_BF16 && out_dtype != PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "out_dtype %d: outputs are F16, BF16 or F32", (int)out_dtype);
  const bool dtype_ok = (cache->dtype == PA_F16 && q_dtype == PA_F16) ||
                        (cache->dtype == PA_BF16 && q_dtype == PA_BF16) ||
                        (cache->dtype == PA_FP8_E4M3 && q_dtype == PA_BF16);
  if (!dtype_ok)
    return fail(PA_ERR_UNSUPPORTED, "pool dtype %d with q dtype %d: supported are F16/F16, BF16/BF16, FP8/BF16",
                (int)cache->dtype, (int)q_dtype);
  const pa::DecodeLaunch launch = pa::find_decode(cache->dtype, cache->v_layout, D, bs, G);
  if (launch == nullptr)
    return fail(PA_ERR_UNSUPPORTED,
                "no decode kernel for head_dim %d, block_size %d, group %d (built: head_dim 64/128, block_size "
                "8/16/32, group 1/2/4/8)",
                D, bs, G);
  if (max_blocks <= 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks %d must be positive, max_context_len %d non-negative",
                max_blocks, max_context_len);
  if (static_cast<int64_t>(max_blocks) * bs > 0x7fffffff)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks * block_size exceeds INT32_MAX");
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks) * bs)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len %d > max_blocks %d * block_size %d", max_context_len,
                max_blocks, bs);
  const bool balanced = partition_size == PA_PARTITION_BALANCED;
  if (!balanced && (partition_size < 0 || partition_size % 16 != 0))
    return fail(PA_ERR_INVALID_ARGUMENT,
                "partition_size %d must be 0, a positive multiple of 16 or PA_PARTITION_BALANCED", partition_size);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (hkv > 65535 || B > 65535) return fail(PA_ERR_INVALID_ARGUMENT, "B and num_kv_heads must be <= 65535");
  const int64_t P = pa::partitions_for(max_context_len, partition_size);
  if (P > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "too many partitions");
  const size_t need = pa::workspace_bytes_for(B, num_q_heads, hkv, D, P);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace of %zu bytes needed (got %zu)", need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % pa::kAlign != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  if (pa::debug_enabled()) {
    std::vector<int32_t> lens(B), tab(static_cast<size_t>(B) * max_blocks);
    if (hipMemcpy(lens.data(), context_lens, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(tab.data(), block_tables, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading block_tables / context_lens failed");
    for (int32_t i = 0; i < B; ++i) {
      if (lens[i] < 0 || lens[i] > max_context_len)
        return fail(PA_ERR_INVALID_ARGUMENT, "context_lens[%d] = %d outside [0, max_context_len %d]", i, lens[i],
                    max_context_len);
      const int32_t nb = (lens[i] + bs - 1) / bs;
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t id = tab[static_cast<size_t>(i) * max_blocks + j];
        if (id < 0 || id >= cache->num_blocks)
          return fail(PA_ERR_INVALID_ARGUMENT, "block_tables[%d][%d] = %d outside [0, %d)", i, j, id,
                      cache->num_blocks);
      }
    }
  }

  const int out_c = pa::out_code(out_dtype);
  const bool fp8 = cache->dtype == PA_FP8_E4M3;
  const float qk_scale_log2 = scale * (fp8 ? cache->k_scale : 1.0f) * 1.44269504088896340736f;
  const float v_scale = fp8 ? cache->v_scale : 1.0f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pa::debug_enabled() && k_new != nullptr) {
    std::vector<int32_t> lens(B), tab(static_cast<size_t>(B) * max_blocks);
    std::vector<int64_t> slots(B);
    if (hipMemcpy(lens.data(), context_lens, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(tab.data(), block_tables, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(slots.data(), slot_mapping, sizeof(int64_t) * B, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading block_tables / context_lens / slot_mapping failed");
    for (int32_t i = 0; i < B; ++i) {
      if (slots[i] < 0 || lens[i] <= 0) continue;
      const int32_t t = lens[i] - 1;
      const int64_t want = static_cast<int64_t>(tab[static_cast<size_t>(i) * max_blocks + t / bs]) * bs + t % bs;
      if (slots[i] != want)
        return fail(PA_ERR_INVALID_ARGUMENT, "slot_mapping[%d] = %lld is not the slot of token %d (%lld)", i,
                    (long long)slots[i], t, (long long)want);
    }
  }
  if (balanced)
    return pa::decode_balanced(cache, out, out_c, q, block_tables, max_blocks, context_lens, B, num_q_heads,
                               max_context_len, qk_scale_log2, v_scale, workspace, workspace_bytes, s, -1, 0, k_new,
                               v_new, slot_mapping, fit_workspace);
  // Partitions with token-major V (16-bit pools) or fp8 pools (either V
  // layout; partition_size a multiple of their 32-token units, or one
  // partition) can run on the
  // staged kernel in partition mode: one workgroup of up to 4 KV heads per
  // partition, whole-row loads. It streams faster but its workgroups are
  // coarse (a partition of 512 tokens is 1 MiB for 4 heads): it wins when
  // few long sequences fill the device with many partitions each (long
  // context: 663 -> 484 us), and loses to the one-wave partition kernels on
  // batches of many shorter sequences (GQA, mixed, prefix batches). So: few
  // segments per CU and at least 8 partitions. PA_PARTITION_PATH=staged /
  // wave forces one path where both exist (a measurement aid).
  const bool tv = cache->v_layout == PA_LAYOUT_TOKEN_MAJOR;
  const bool staged_ok = sh == nullptr && ((tv && !fp8) || (fp8 && (P == 1 || partition_size % 32 == 0))) &&
                         pa::sk_partition_fits(cache, B, G);
  bool staged_part = false;
  if (staged_ok) {
    const int cus = pa::device_cus();
    const int64_t n_hg = hkv / std::min(pa::sk_heads_per_wg(hkv, true), 4);
    staged_part = cus > 0 && static_cast<int64_t>(B) * n_hg * 8 <= cus && P >= 8;
    if (const char* path = std::getenv("PA_PARTITION_PATH")) {
      if (std::strcmp(path, "staged") == 0) staged_part = true;
      if (std::strcmp(path, "wave") == 0) staged_part = false;
    }
  }
  if (staged_part)
    return pa::decode_balanced(cache, out, out_c, q, block_tables, max_blocks, context_lens, B, num_q_heads,
                               max_context_len, qk_scale_log2, v_scale, workspace, workspace_bytes, s,
                               partition_size, P);
  // shared prefixes: the cascade on the balanced kernel where it is built
  // and fits, else the shared-prefix partition kernels below
  // (PA_SHARED_PATH=partition / cascade forces one; cascade fails with
  // PA_ERR_UNSUPPORTED where it cannot run: measurement and test aids)
  if (sh != nullptr && sh->num_groups > 0 && sh->max_shared_len > 0) {
    const char* path = std::getenv("PA_SHARED_PATH");
    if (path == nullptr || std::strcmp(path, "partition") != 0) {
      const pa_status cs = pa::decode_cascade(cache, out, out_c, q, block_tables, max_blocks, context_lens, B,
                                              num_q_heads, max_context_len, qk_scale_log2, v_scale, workspace,
                                              workspace_bytes, s, sh->group_offsets, sh->group_members,
                                              sh->shared_len, sh->num_groups, sh->max_group_size);
      if (cs != PA_ERR_UNSUPPORTED) return cs;
      if (path != nullptr && std::strcmp(path, "cascade") == 0)
        return fail(PA_ERR_UNSUPPORTED,
                    "PA_SHARED_PATH=cascade: no cascade for this call (token-major V or fp8 pools, at most 32 "
                    "rows per group, the batch's plan in LDS, a workspace of pa_decode_shared_workspace_size)");
    }
  }

  pa::DecodeParams prm{};
  prm.q = q;
  prm.k_pool = cache->k;
  prm.v_pool = cache->v;
  prm.out = out;
  const size_t rows = static_cast<size_t>(B) * num_q_heads * P;
  if (need > 0) {
    char* ws = static_cast<char*>(workspace);
    prm.part_m = reinterpret_cast<float*>(ws);
    prm.part_l = reinterpret_cast<float*>(ws + pa::align_up(rows * sizeof(float)));
    prm.part_o = reinterpret_cast<float*>(ws + 2 * pa::align_up(rows * sizeof(float)));
  }
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.block_stride = cache->block_stride;
  prm.num_blocks = cache->num_blocks;
  prm.num_kv_heads = hkv;
  prm.num_q_heads = num_q_heads;
  prm.max_blocks = max_blocks;
  prm.len_cap = max_context_len;
  prm.partition_size = P > 1 ? partition_size : 0;
  prm.num_partitions = static_cast<int32_t>(P);
  prm.out_dtype = out_c;
  prm.qk_scale_log2 = qk_scale_log2;
  prm.v_scale = v_scale;
  const int64_t wgs = P * hkv * B;
  if (wgs > 0x7fffffff) return fail(PA_ERR_INVALID_ARGUMENT, "too many workgroups (%lld)", (long long)wgs);
  hipError_t e = hipSuccess;
  if (sh != nullptr && sh->num_groups > 0 && sh->max_shared_len > 0) {
    // group units for the shared partitions, then the rest per sequence
    // (see decode_shared_kernel.h)
    const pa::GroupLaunch glaunch = pa::find_decode_group(cache->dtype, cache->v_layout, D, bs, G);
    if (glaunch == nullptr) return fail(PA_ERR_UNSUPPORTED, "no shared-prefix kernel for these shapes");
    pa::SharedParams sp{};
    sp.group_offsets = sh->group_offsets;
    sp.group_members = sh->group_members;
    sp.shared_len = sh->shared_len;
    sp.num_groups = sh->num_groups;
    sp.row_tiles = (sh->max_group_size * G + 15) / 16;
    // two row tiles per group unit when a group has more than 16 rows: every
    // shared K/V tile is loaded once per KV head (PA_SHARED_TILES=1 forces
    // one, a measurement aid)
    sp.tiles_per_wg = sp.row_tiles > 1 ? 2 : 1;
    if (const char* t = std::getenv("PA_SHARED_TILES")) {
      if (std::atoi(t) == 1) sp.tiles_per_wg = 1;
    }
    sp.row_sets = (sp.row_tiles + sp.tiles_per_wg - 1) / sp.tiles_per_wg;
    sp.shared_parts = sh->max_shared_len / partition_size;
    sp.pairs = B * hkv;
    const int64_t units = static_cast<int64_t>(sp.shared_parts) * sh->num_groups * hkv;
    const int64_t gwgs = (units + 7) / 8 * 8 * sp.row_sets;
    // partitions past the shared prefix: at most P - min_shared_len / ps per sequence
    const int64_t twgs = (P - sh->min_shared_len / partition_size) * static_cast<int64_t>(B) * hkv;
    if (gwgs + twgs > 0x7fffffff)
      return fail(PA_ERR_INVALID_ARGUMENT, "too many shared-prefix workgroups (%lld)", (long long)(gwgs + twgs));
    sp.group_wgs = static_cast<int32_t>(gwgs);
    prm.shared_len = sh->shared_len;
    e = glaunch(prm, sp, dim3(static_cast<uint32_t>(gwgs + twgs)), s);
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "shared-prefix launch: %s", hipGetErrorString(e));
  } else {
    e = launch(prm, dim3(static_cast<uint32_t>(wgs)), s);
  }
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "decode launch: %s", hipGetErrorString(e));
  if (P > 1) {
    pa::ReduceParams r{};
    r.part_m = prm.part_m;
    r.part_l = prm.part_l;
    r.part_o = prm.part_o;
    r.out = out;
    r.context_lens = context_lens;
    r.len_cap = max_context_len;
    r.partition_size = partition_size;
    r.num_partitions = static_cast<int32_t>(P);
    r.num_q_heads = num_q_heads;
    r.head_dim = D;
    r.out_dtype = prm.out_dtype;
    hipLaunchKernelGGL(pa::decode_reduce_kernel, dim3(num_q_heads, B), dim3(D < 128 ? D : 128), 0, s, r);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "decode reduce launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_decode(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                    int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  return pa::decode_impl(cache, out, out_dtype, q, q_dtype, block_tables, max_blocks, context_lens, B, num_q_heads,
                         max_context_len, scale, partition_size, workspace, workspace_bytes, stream, nullptr, nullptr,
                         nullptr);
}

pa_status pa_decode_append(const pa_kv_cache* cache, const void* k_new, const void* v_new, pa_dtype src_dtype,
                           const int64_t* slot_mapping, void* out, pa_dtype out_dtype, const void* q,
                           pa_dtype q_dtype, const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, int32_t B, int32_t num_q_heads, int32_t max_context_len,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (B > 0 && (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "k_new, v_new or slot_mapping is NULL");
  if (cache->dtype != PA_F16 && cache->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_append takes F16 or BF16 pools (pool dtype %d)", (int)cache->dtype);
  if (src_dtype != cache->dtype)
    return fail(PA_ERR_UNSUPPORTED, "k_new / v_new dtype %d differs from the pool dtype %d", (int)src_dtype,
                (int)cache->dtype);
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(slot_mapping) % 8 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "k_new / v_new must be 16-byte aligned, slot_mapping 8-byte aligned");
  if (B == 0) return PA_OK;
  return pa::decode_impl(cache, out, out_dtype, q, q_dtype, block_tables, max_blocks, context_lens, B, num_q_heads,
                         max_context_len, scale, PA_PARTITION_BALANCED, workspace, workspace_bytes, stream, k_new,
                         v_new, slot_mapping);
}

pa_status pa_decode_noalloc(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                            int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                            void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (B <= 0) return B < 0 ? fail(PA_ERR_INVALID_ARGUMENT, "B = %d is negative", B) : PA_OK;
  if (partition_size != PA_PARTITION_BALANCED && num_q_heads > 0 && max_context_len >= 0 && partition_size >= 0) {
    const size_t need = pa::workspace_bytes_for(B, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                                pa::partitions_for(max_context_len, partition_size));
    if (need > pa::kScratchBytes)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "pa_decode_noalloc: this partitioned call needs %zu bytes of scratch; the library's static scratch "
                  "holds %zu (use pa_decode with a workspace, or a larger partition_size)",
                  need, pa::kScratchBytes);
  }
  void* ws = nullptr;
  st = pa::scratch_of_current_device(&ws);
  if (st != PA_OK) return st;
  return pa::decode_impl(cache, out, out_dtype, q, q_dtype, block_tables, max_blocks, context_lens, B, num_q_heads,
                         max_context_len, scale, partition_size, ws, pa::kScratchBytes, stream, nullptr, nullptr,
                         nullptr, nullptr, /*fit_workspace=*/true);
}

pa_status pa_decode_shared(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                           const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                           int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                           const int32_t* group_offsets, const int32_t* group_members, const int32_t* shared_len,
                           int32_t num_groups, int32_t max_group_size, int32_t max_shared_len,
                           int32_t min_shared_len, void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  pa_status st = pa::validate_cache(cache);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % 16 != 0 || partition_size % cache->block_size != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "partition_size %d must be a positive multiple of 16 and of block_size %d",
                partition_size, cache->block_size);
  if (num_groups < 0 || max_group_size < 0 || max_shared_len < 0 || min_shared_len < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative num_groups, max_group_size, max_shared_len or min_shared_len");
  if (max_shared_len % partition_size != 0 || min_shared_len % partition_size != 0 || min_shared_len > max_shared_len)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "min_shared_len %d / max_shared_len %d must be multiples of partition_size %d, min <= max",
                min_shared_len, max_shared_len, partition_size);
  if (max_shared_len >= max_context_len && max_shared_len > 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_shared_len %d must be below max_context_len %d", max_shared_len,
                max_context_len);
  if (num_groups > 0 && (group_offsets == nullptr || group_members == nullptr || shared_len == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "group_offsets, group_members or shared_len is NULL");
  if (num_groups > B || max_group_size > B)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_groups %d / max_group_size %d exceed B = %d", num_groups,
                max_group_size, B);
  if (B > 0 && num_groups > 0 && pa::debug_enabled()) {
    std::vector<int32_t> off(num_groups + 1), lens(B), shl(B), tab(static_cast<size_t>(B) * max_blocks);
    if (hipMemcpy(off.data(), group_offsets, sizeof(int32_t) * off.size(), hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(lens.data(), context_lens, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(shl.data(), shared_len, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(tab.data(), block_tables, sizeof(int32_t) * tab.size(), hipMemcpyDeviceToHost) != hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading the group arrays failed");
    if (off[0] != 0 || off[num_groups] > B) return fail(PA_ERR_INVALID_ARGUMENT, "group_offsets out of range");
    std::vector<int32_t> mem(off[num_groups]);
    if (!mem.empty() && hipMemcpy(mem.data(), group_members, sizeof(int32_t) * mem.size(), hipMemcpyDeviceToHost) !=
                            hipSuccess)
      return fail(PA_ERR_DEVICE, "PA_DEBUG: reading group_members failed");
    std::vector<int> in_group(B, 0);
    const int32_t bs = cache->block_size;
    for (int32_t gi = 0; gi < num_groups; ++gi) {
      if (off[gi + 1] < off[gi] || off[gi + 1] - off[gi] > max_group_size)
        return fail(PA_ERR_INVALID_ARGUMENT, "group %d: bad offsets or larger than max_group_size", gi);
      if (off[gi + 1] == off[gi]) continue;
      const int32_t first = mem[off[gi]];
      for (int32_t m = off[gi]; m < off[gi + 1]; ++m) {
        const int32_t sq = mem[m];
        if (sq < 0 || sq >= B || in_group[sq]++)
          return fail(PA_ERR_INVALID_ARGUMENT, "group %d: member %d out of range or in two groups", gi, sq);
        if (shl[sq] != shl[first] || shl[sq] % partition_size != 0 || shl[sq] > max_shared_len ||
            shl[sq] < min_shared_len ||
            shl[sq] >= std::min(lens[sq], max_context_len))
          return fail(PA_ERR_INVALID_ARGUMENT, "group %d: shared_len of row %d is inconsistent", gi, sq);
        for (int32_t b = 0; b < shl[sq] / bs; ++b)
          if (tab[static_cast<size_t>(sq) * max_blocks + b] != tab[static_cast<size_t>(first) * max_blocks + b])
            return fail(PA_ERR_INVALID_ARGUMENT, "group %d: rows %d and %d differ at table entry %d", gi, sq, first, b);
      }
    }
    for (int32_t i = 0; i < B; ++i) {
      if (!in_group[i] && shl[i] != 0)
        return fail(PA_ERR_INVALID_ARGUMENT, "row %d is in no group but has shared_len %d", i, shl[i]);
      if (shl[i] < min_shared_len)
        return fail(PA_ERR_INVALID_ARGUMENT, "shared_len[%d] = %d is below min_shared_len %d", i, shl[i],
                    min_shared_len);
    }
  }
  pa::SharedArgs sh{group_offsets, group_members, shared_len, num_groups, max_group_size, max_shared_len,
                    min_shared_len};
  return pa::decode_impl(cache, out, out_dtype, q, q_dtype, block_tables, max_blocks, context_lens, B, num_q_heads,
                         max_context_len, scale, partition_size, workspace, workspace_bytes, stream, nullptr, nullptr,
                         nullptr, num_groups > 0 ? &sh : nullptr);
}

}  // extern "C"
