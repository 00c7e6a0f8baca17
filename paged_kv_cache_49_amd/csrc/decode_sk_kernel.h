// Paged decode attention with the whole batch's work divided evenly over
// persistent workgroups (balanced split; also, in partition mode, one
// workgroup per context partition); V blocks dim-major, or token-major for
// 16-bit pools (TV, each tile's V rows transposed through LDS).
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
// Same result as the partition kernels (decode_common.h states what is
// computed: softmax attention of each query head over its sequence's tokens
// in logical order, gathered through the block table); the per-tile data
// flow (QK and PV on the matrix cores, online softmax) is that of
// decode_vt_kernel.h.
//
// Work units are tiles of TT tokens (16 for 16-bit pools, 32 for fp8 pools,
// so a unit's K/V is 8 KiB per KV head either way and a ring slot keeps the
// same bytes in flight), numbered head group-major, then sequence, then
// tile: unit = hg * T + prefix[s] + tile, T = total tiles of the batch.
// A head group is HW consecutive KV heads; a workgroup has HW waves and wave
// i serves KV head hg * HW + i, so one unit reads all HW heads of a tile's
// block rows at once (a whole block when HW = num_kv_heads). The grid holds
// W workgroups, about as many as are resident at once; workgroup w takes the
// units [w U / W, (w + 1) U / W), so all of them stream the same number of
// tiles, and a wave walks from one sequence into the next without ending.
//
// Per workgroup:
//  * plan: tiles per sequence (lengths clamped to the launch bound) and
//    their exclusive prefix go to LDS.
//  * append variant (AP): the newest token of each sequence (position
//    L - 1) is not read from the cache but from k_new / v_new, as one extra
//    unit per sequence holding a single valid row (the "virtual tile"); the
//    workgroup that computes it also writes that row into the cache at
//    slot_mapping[s]. The cache tiles then cover positions 0 .. L - 2. This
//    is pa_reshape_and_cache followed by pa_decode in one launch.
//  * loads, two forms. Staged (token-major V, and fp8 pools): the HW waves
//    read the unit's K rows and V (token-major rows, or the dim-major
//    region of each block) of the whole head group as contiguous 1 KiB
//    spans with non-temporal loads; at compute time they go to an LDS
//    stage and, after a workgroup barrier, each wave reads its head's
//    operands from it (K in the QK layout, V through the transposing read
//    or as 8-byte runs). Otherwise each wave loads its own head's K rows
//    and dim-major V runs directly in the operand layouts.
//  * unit batches: lane i of a batch resolves unit ub + i to its sequence,
//    tile, length, head group and block id(s); the batch after it is
//    requested one batch ahead, so block-table reads never stall the loads.
//  * a 2-slot register ring keeps the q, K and V loads of the next unit in
//    flight while one unit is computed (q rides in the ring too, so a new
//    segment never waits on a load issued behind the ring's; staged, as the
//    wave's G x D rows, rebuilt through its LDS region). The waves of a
//    workgroup pass a barrier after each unit: without it the oldest wave
//    of each SIMD takes most issue slots and finishes far ahead, and the
//    others end alone with few loads in flight.
//  * a (head group, sequence) segment that ends inside the range is
//    normalised and stored directly; a segment cut by the range's start or
//    end leaves a partial (m, l, o) piece in slot 0 (it reaches back to the
//    range start) or slot 1 (it starts inside the range), which
//    decode_sk_merge_kernel combines with the pieces of the neighbouring
//    workgroups (the log-sum-exp merge described in decode.hip).
//  * merge descriptor of a segment: {-1, -} when one workgroup completed it;
//    else {wf | slot << 31, wl}, written by the workgroups where it starts
//    (wf, its piece in `slot`) and ends (wl, slot 0). Every workgroup in
//    between holds a slot-0 piece; a workgroup with no units writes neutral
//    slot-0 pieces (m = -inf, l = 0, o = 0), so a merge may include it.
//    In partition mode a workgroup holds exactly one piece (one slot).
//
// Cascade variant (CAS, for pa_decode_shared;
// [course] §2 "The bonus": forked sequences share the prompt's blocks;
// [note] prefix-sharing section). The same persistent ranges run over
// "virtual sequences" instead of sequences: first one per group, the
// group's shared prefix (tokens [0, S) in whole units, read through the
// first member's table), then one per batch row, the row's own tokens
// [S, L). A prefix unit computes two 16-row q tiles per wave: row r of the
// pair is member r / G of the group, query head r % G of the wave's KV head,
// so each shared K/V tile is read once for every member. Softmax attention
// over the row's tokens is the log-sum-exp merge of its two parts, so each
// part leaves its partial (m, l, o): a segment one workgroup completed as a
// state row of its batch row, a cut segment as pieces; decode_cascade_merge_
// kernel (decode.hip) merges prefix and tail of every row. A prefix
// segment's q rows (two tiles) sit in the wave's LDS region from the
// segment's first unit in the range on; the two tiles are computed one
// after the other on the unit's K and V operands.
#pragma once

#include <type_traits>

#include "decode_vt_kernel.h"
#include "host_cache.h"

namespace pa {

struct SkParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  void* out;
  float* piece_m;       // [W][2][HW * G]
  float* piece_l;       // [W][2][HW * G]
  float* piece_o;       // [W][2][HW * G][D]
  int32_t* seg_desc;    // [head groups][B][2] merge descriptors, see below
  const void* k_new;              // append: [B][num_kv_heads][D] (pool dtype)
  const void* v_new;              // append: [B][num_kv_heads][D]
  const int64_t* slot_mapping;    // append: [B] cache slot of token L - 1 (< 0: no write)
  const int32_t* block_tables;
  const int32_t* context_lens;
  int64_t block_stride;  // elements
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t len_cap;
  int32_t batch;
  int32_t heads_per_wg;     // HW
  int32_t num_head_groups;  // num_kv_heads / HW
  // partition mode (part_tiles > 0): workgroup w takes the units of one
  // (head group, sequence, partition) = ((hg * B + s) * num_parts + part),
  // part_tiles units each; otherwise the balanced ranges
  int32_t part_tiles;
  int32_t num_parts;
  int32_t piece_slots;      // piece slots per workgroup: 2 (balanced), 1 (partition mode)
  int32_t stage_bufs;       // LDS stages (staged path): 2 = alternate per unit, one barrier per unit
  int32_t out_dtype;
  float qk_scale_log2;
  float v_scale;
  // cascade only: the groups (group gi's rows are group_members[
  // group_offsets[gi] .. group_offsets[gi + 1]), each row's shared length,
  // the state rows of completed segments ([part][B][num_q_heads], part 0 =
  // prefix, 1 = tail) and the merge's row map ([B][4]: group of the row's
  // prefix part or -1, the row's place in that group, whether the row has
  // a tail part)
  const int32_t* group_offsets;
  const int32_t* group_members;
  const int32_t* shared_len;
  float* state_m;
  float* state_l;
  float* state_o;
  int32_t* row_map;
  int32_t num_groups;
};

// first unit of workgroup w's range; the range of w is [start(w), start(w + 1))
__device__ __forceinline__ int sk_range_start(int w, int U, int W) {
  return static_cast<int>(static_cast<int64_t>(w) * U / W);
}
// the workgroup whose (non-empty) range holds unit u
__device__ __forceinline__ int sk_owner(int u, int U, int W) {
  return static_cast<int>((static_cast<int64_t>(u + 1) * W - 1) / U);
}

// first sequence s with pref[s + 1] > r: the sequence holding tile r of a
// head group (sequences without tiles are skipped)
__device__ __forceinline__ int sk_find_seq(const int32_t* pref, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pref[mid + 1] > r) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// LDS of one wave, in floats: its G q rows (D 16-bit elements each, rows
// padded by 16 bytes), through which the staged path rebuilds q; with
// lds_flush also its G x D fp32 output tile (the same memory), through which
// a finished segment is stored with 16-byte stores (the append variant: a
// flush straight from the accumulators keeps more addresses live, and its
// build then spilled); cascade: 32 q rows (the two row tiles of a prefix
// unit, written when its segment starts)
__host__ __device__ inline constexpr size_t sk_wave_lds_floats(int G, int D, bool lds_flush = false,
                                                                bool cas = false) {
  return cas ? static_cast<size_t>(32) * (2 * D + 16) / 4
             : (lds_flush ? static_cast<size_t>(G) * D : static_cast<size_t>(G) * (2 * D + 16) / 4);
}

// The stage: the unit's K and V as loaded (whole rows), in LDS. S = HW * D
// * b bytes is the head group's slice of a token row. (Measured with the
// LDS counters: the LDS serves 16-byte reads of 16 rows at 128 bytes per
// cycle whatever the row offsets, as long as no two rows share their banks
// outright; the transposing 8-byte read of 4 rows x 32 bytes per 16 lanes
// runs at 256 bytes per cycle when those rows sit 8 banks apart.)
//  * 16-bit pools with token-major V: K and V as two [16][S] tiles. Row
//    pitches: K rows S + 16 bytes (a pitch of S would put all 16 rows of an
//    operand read on the same banks), V rows S + 32 bytes (the 4 rows of a
//    transposing read then sit 8 banks apart).
//  * fp8 pools: K as a [32][S] tile at pitch S + 16 (rows 16..31 64 bytes
//    further; measured to make no difference). V dim-major: the head group's [HW][D][BS] region of each
//    of the unit's blocks, stored chunk-major ([HW][BS / 8][D][8 bytes]: an
//    operand read of 16 head dims is then 128 contiguous bytes; 32 S bytes);
//    token-major: the 32 rows as loaded, laid out like K, read back with
//    the 8-bit transposing read (ds_read_b64_tr_b8: a 16-lane group reads
//    8 rows x 16 bytes, rows 4 banks apart) and widened to bf16 in
//    registers.
__host__ __device__ inline constexpr int sk_stage_kpitch(int S) { return S + 16; }
__host__ __device__ inline constexpr int sk_stage_vpitch(int S) { return S + 32; }
__host__ __device__ inline constexpr size_t sk_stage_bytes(int HW, int D, int kb, bool tv) {
  return kb == 2 ? 16 * static_cast<size_t>(sk_stage_kpitch(HW * D * 2) + sk_stage_vpitch(HW * D * 2))
                 : 32 * static_cast<size_t>(sk_stage_kpitch(HW * D)) + 64 +
                       (tv ? 32 * static_cast<size_t>(sk_stage_kpitch(HW * D)) + 64 : 32 * static_cast<size_t>(HW * D));
}

// ints of the plan in LDS (a multiple of 4): the tile prefix over the
// sequences [B + 1]; the cascade (cas_groups = its number of groups NG,
// NV = NG + B virtual sequences) holds the prefix [NV + 1], per virtual
// sequence its table row or first tail unit [NV], the group offsets
// [NG + 1], the members [B], each row's shared length [B] and its place in
// a group [B]
__host__ __device__ inline constexpr int sk_plan_ints(int B, int cas_groups) {
  return ((cas_groups >= 0 ? 3 * cas_groups + 5 * B + 2 : B + 1) + 3) / 4 * 4;
}

// bytes of dynamic LDS: the plan, the stage(s) (token-major V or fp8
// pools: `staged`), then one region per wave
inline size_t sk_lds_bytes(int B, int HW, int G, int D, bool staged, int kb, bool tv, int bufs = 1,
                           bool append = false, int cas_groups = -1) {
  const size_t pref = static_cast<size_t>(sk_plan_ints(B, cas_groups)) * sizeof(int32_t);
  return pref + (staged ? bufs * sk_stage_bytes(HW, D, kb, tv) : 0) +
         static_cast<size_t>(HW) * sk_wave_lds_floats(G, D, append, cas_groups >= 0) * sizeof(float);
}

// Barrier for LDS written by some waves of the workgroup and read by others
// (orders LDS accesses only: loads in flight stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// the lane's V registers for one unit: dim-major runs (u32x2 per n-tile) or
// pieces of the unit's V as loaded for the stage (u32x4, as K)
template <bool STG>
struct SkVSlot {
  using type = u32x2;
};
template <>
struct SkVSlot<true> {
  using type = u32x4;
};

// A unit as the wave sees it (uniform values). len = valid tokens counted
// from the unit's first position; virt = the append variant's virtual tile,
// whose slot block / offset are sblk / soff.
// Cascade: pre = a prefix unit; first = the first unit of its virtual
// sequence; qsrc = where a prefix unit that needs new q rows finds them
// (0: none needed, 1: the spare set, 2: loaded at compute time).
struct SkUnit {
  int seq, tile, len, hg;
  int virt, sblk, soff;
  int pre, first, qsrc;
  int qld;  // staged: the unit carries its segment's q rows (loaded, to be stored)
};

// NBUF: LDS stages of the staged path (2: units alternate between them);
// CAS: the cascade variant (no append)
template <typename KV, typename QT, int D, int BS, int G, bool AP, bool TV, int NBUF, bool CAS>
__global__ __launch_bounds__(512) void paged_decode_sk_kernel(const SkParams p) {
  using C = DecodeCfg<KV, D, BS, G>;
  constexpr int kB = C::kB;
  constexpr int kNT = D / 16;
  static_assert(G <= 16, "at most 16 query heads per KV head");
  static_assert(!(CAS && AP), "the cascade has no append variant");
  // q row tiles per wave (two for prefix units), piece rows per wave
  constexpr int CT = CAS ? 2 : 1;
  constexpr int RW = CAS ? 16 * CT : G;
  // tokens per unit, 16-row QK tiles per unit, scores per lane (lane group
  // j holds tokens kE * j .. kE * j + kE - 1), blocks one unit spans
  constexpr int TT = kB == 1 ? 32 : 16;
  constexpr int kSub = TT / 16;
  constexpr int kE = TT / 4;
  constexpr int kTB = BS < TT ? TT / BS : 1;
  static_assert(!AP || TT == 16, "the append variant is for 16-bit pools");
  // STG: the unit's K and V are loaded as whole rows / regions and go
  // through the LDS stage (token-major V, and fp8 pools); otherwise each
  // wave loads its head's K rows and V runs in the operand layouts
  constexpr bool STG = TV || kB == 1;
  constexpr int kKP = kSub * C::kKLoads;  // 16-byte K pieces per lane and unit
  // V per lane and unit: dim-major, one run of one head dim over the lane's
  // kE tokens per n-tile (4 x 16-bit or 8 x fp8); staged, the lane's share of
  // the unit's V as loaded, as K (see the stage below)
  using VSlot = typename SkVSlot<STG>::type;
  constexpr int kVL = STG ? kKP : kNT;
  // q per lane and unit: the QK operand (kKSteps pieces), or when staged
  // the wave's G x D q rows as 16-byte pieces (lane l, piece i: byte
  // 16 (64 i + l) of the rows), rebuilt through the wave's LDS region
  constexpr int kQBytes = G * D * 2;
  constexpr int kQL = STG ? (kQBytes > 1024 ? kQBytes / 1024 : 1) : C::kKSteps;
  constexpr int kQPitch = D * 2 + 16;  // bytes per q row in LDS (rows 4 banks apart)
  // rows of a segment's output per pass through the wave's LDS region (the
  // append variant's holds G x D floats, the others' G q rows: half the
  // output rows); 0: stored from the registers
  constexpr int kTileRows = CAS ? 0 : AP ? G : G >= 4 ? G / 2 : 0;
  static_assert(kTileRows * D * 4 <= static_cast<int>(sk_wave_lds_floats(G, D, AP, CAS) * sizeof(float)),
                "an output pass fits the wave's LDS region");
  static_assert(!STG || (CAS ? 16 * CT : G) * kQPitch <= static_cast<int>(sk_wave_lds_floats(G, D, AP, CAS) * sizeof(float)),
                "the q rows fit the wave's LDS region");
  static_assert(!CAS || STG, "the cascade is built on the staged path");
  extern __shared__ int32_t sk_smem[];
  const int B = p.batch;
  // virtual sequences: the batch rows, or (cascade) NG group prefixes and
  // then the B rows' tails
  const int NG = CAS ? p.num_groups : 0;
  const int NV = NG + B;
  int32_t* s_pref = sk_smem;            // [NV + 1]
  int32_t* s_aux = s_pref + NV + 1;     // cascade: [NV] table row (prefix) / first tail unit
  int32_t* s_goff = s_aux + NV;         // cascade: [NG + 1]
  int32_t* s_mem = s_goff + NG + 1;     // cascade: [B]
  int32_t* s_shl = s_mem + B;           // cascade: [B] shared tokens of each row, whole units
  int32_t* s_in = s_shl + B;            // cascade: [B] group * 32 + place of each member row, or -1
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int HW = p.heads_per_wg;
  char* stage = reinterpret_cast<char*>(sk_smem + sk_plan_ints(B, CAS ? NG : -1));  // STG only
  // with two stages, unit x uses stage x % 2: the barrier after the stage
  // write of unit x + 1 already orders unit x's reads before the next
  // write into its stage, so no barrier is needed after a unit
  static_assert(NBUF == 1 || (NBUF == 2 && (TV || kB == 1)), "two stages on the staged path only");
  const int sbytes = STG ? static_cast<int>(sk_stage_bytes(HW, D, kB, TV)) : 0;
  float* s_out_all = reinterpret_cast<float*>(stage + NBUF * sbytes);

  // ---- plan: tiles per (virtual) sequence, then their exclusive prefix (in place)
  if constexpr (CAS) {
    // a row's shared tokens in whole units (at most the launch bound, so the
    // prefix reads stay inside the first member's table); its tail is the
    // rest. Group offsets and member ids are clamped or checked before use:
    // inconsistent groups give wrong rows, never an access out of bounds.
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
      int L = p.context_lens[i];
      L = L < p.len_cap ? L : p.len_cap;
      int sh = p.shared_len[i];
      sh = sh < 0 ? 0 : (sh < p.len_cap ? sh : p.len_cap);
      sh = sh / TT * TT;
      s_shl[i] = sh;
      s_pref[NG + i] = L > sh ? (L - sh + TT - 1) / TT : 0;
      s_aux[NG + i] = sh / TT;
      s_in[i] = -1;
    }
    for (int i = threadIdx.x; i <= NG; i += blockDim.x) {
      const int o = p.group_offsets[i];
      s_goff[i] = o < 0 ? 0 : (o < B ? o : B);
    }
    __syncthreads();
    const int nmem = s_goff[NG];
    for (int k = threadIdx.x; k < nmem; k += blockDim.x) s_mem[k] = p.group_members[k];
    __syncthreads();
    for (int v = threadIdx.x; v < NG; v += blockDim.x) {
      const int m0 = s_goff[v];
      const int first = s_goff[v + 1] > m0 && m0 < nmem ? s_mem[m0] : -1;
      const bool ok = static_cast<unsigned>(first) < static_cast<unsigned>(B);
      s_pref[v] = ok ? s_shl[first] / TT : 0;
      s_aux[v] = ok ? first : 0;
    }
    __syncthreads();
    // member slot k -> its row's place: the group holding slot k (the last
    // offset at or below k), if that group has a prefix part and the row
    // fits the prefix units' RW / G members
    for (int k = threadIdx.x; k < nmem; k += blockDim.x) {
      const int s = s_mem[k];
      if (static_cast<unsigned>(s) >= static_cast<unsigned>(B) || NG == 0) continue;
      int lo = 0, hi = NG - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_goff[mid] <= k) lo = mid; else hi = mid - 1;
      }
      const int mi = k - s_goff[lo];
      if (mi >= 0 && k < s_goff[lo + 1] && mi * G < RW && s_pref[lo] > 0) s_in[s] = lo * 32 + mi;
    }
  } else {
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
      int L = p.context_lens[i];
      L = L < p.len_cap ? L : p.len_cap;
      // append: the cache holds L - 1 tokens, plus the virtual tile
      s_pref[i] = L > 0 ? (AP ? ((L + 14) >> 4) + 1 : (L + TT - 1) / TT) : 0;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int per = (NV + 63) / 64;
    const int i0 = lane * per, i1 = min(NV, i0 + per);
    int run = 0;
    for (int i = i0; i < i1; ++i) run += s_pref[i];
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    int acc_t = incl - run;
    for (int i = i0; i < i1; ++i) {
      const int c = s_pref[i];
      s_pref[i] = acc_t;
      acc_t += c;
    }
    if (lane == 63) s_pref[NV] = incl;
  }
  __syncthreads();
  const int T = s_pref[NV];
  const int U = T * p.num_head_groups;  // the launch guarantees U < 2^31
  const int W = static_cast<int>(gridDim.x);
  const int w = static_cast<int>(blockIdx.x);
  if constexpr (CAS) {
    // the merge's row map; this workgroup writes rows w, w + W, ...
    for (int s = w + W * static_cast<int>(threadIdx.x); s < B; s += W * static_cast<int>(blockDim.x)) {
      const int e = s_in[s];
      int32_t* rm = p.row_map + 4 * static_cast<int64_t>(s);
      rm[0] = e >= 0 ? e / 32 : -1;
      rm[1] = e >= 0 ? e % 32 : 0;
      rm[2] = s_pref[NG + s + 1] > s_pref[NG + s] ? 1 : 0;
      rm[3] = 0;
    }
  }
  int u0, u1;
  if (p.part_tiles > 0) {
    // partition mode: the range is one partition of one segment; a partition
    // past the sequence's end does nothing (no merge range reaches it)
    const int part = w % p.num_parts;
    const int rest = w / p.num_parts;
    const int s = rest % B;
    const int hg = rest / B;
    const int nt = s_pref[s + 1] - s_pref[s];
    const int t0 = part * p.part_tiles;
    if (t0 >= nt) {
      // a sequence without tokens: its head group's rows are zero (written
      // here too, since one partition has no merge after it)
      if (nt == 0 && part == 0) {
        const int64_t row0 = static_cast<int64_t>(s) * p.num_q_heads + static_cast<int64_t>(hg) * HW * G;
        for (int i = threadIdx.x; i < HW * G * D; i += blockDim.x) store_out(p.out, row0 * D + i, p.out_dtype, 0.f);
      }
      return;
    }
    u0 = hg * T + s_pref[s] + t0;
    u1 = u0 + min(p.part_tiles, nt - t0);
  } else {
    u0 = sk_range_start(w, U, W);
    u1 = sk_range_start(w + 1, U, W);
  }
  if (u0 >= u1) {
    // no units: neutral slot-0 pieces (only when there are fewer units than workgroups)
    const int rows = HW * RW;
    const int64_t base = static_cast<int64_t>(w) * p.piece_slots * rows;
    for (int i = threadIdx.x; i < rows; i += blockDim.x) {
      p.piece_m[base + i] = -INFINITY;
      p.piece_l[base + i] = 0.f;
    }
    for (int i = threadIdx.x; i < rows * D; i += blockDim.x) p.piece_o[base * D + i] = 0.f;
    return;
  }

  float* s_out = s_out_all + wave * sk_wave_lds_floats(G, D, AP, CAS);
  const int col = lane & 15, j = lane >> 4;
  const int Hkv = p.num_kv_heads;
  const char* kbase = static_cast<const char*>(p.k_pool);
  const char* vbase = static_cast<const char*>(p.v_pool);
  const int64_t blk_bytes = p.block_stride * kB;
  const int64_t tok_bytes = static_cast<int64_t>(Hkv) * D * kB;
  constexpr int kVTileBytes = 16 * BS * kB;  // one 16-dim n-tile of a block
  // lane parts of the addresses: K row `col` (first head-dim slice), V run
  // of head dim `col` from token 4j
  const uint32_t koff_lane = static_cast<uint32_t>(col * tok_bytes + qk_dim<kB>(0, j) * kB);
  const uint32_t voff_lane = static_cast<uint32_t>((col * BS + 4 * j) * kB);
  // Staged (STG): the unit's K rows of the head group are read as whole
  // rows, not in the MFMA layout (a wave reading its own head's slice of 16
  // rows per instruction streams measurably slower than reading 1 KiB
  // contiguous), and so is its V (token-major: rows as K; fp8 dim-major:
  // the head group's [HW][D][BS] region of each block). The [TT][S] slice
  // is split evenly over the HW waves (kKP KiB each): lane piece i is byte
  // f % S of row f / S, f = (wave * kKP + i) KiB + 16 lane (dim-major V: byte
  // f of the unit's regions). Each unit then goes through the LDS stage:
  // written as loaded, read back per wave in the operand layouts. S is a
  // power of two (HW is, when staged).
  const int S = HW * D * kB;
  const int s_log2 = __builtin_ctz(static_cast<unsigned>(S));
  const int kpitch = sk_stage_kpitch(S), vpitch = sk_stage_vpitch(S);  // (vpitch: 16-bit V rows)
  char* stage_v = stage + TT * kpitch + (TT == 32 ? 64 : 0);
  const int SV = HW * D * BS * kB;  // dim-major V: the head group's region of one block
  const int sv_log2 = __builtin_ctz(static_cast<unsigned>(SV));
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto st_f = [&](int i) { return (wave_u * kKP + i) * 1024 + lane * 16; };
  auto st_r = [&](int i) { return st_f(i) >> s_log2; };
  auto st_cb = [&](int i) { return st_f(i) & (S - 1); };
  // LDS byte of K row r, byte b (fp8: rows 16..31 64 bytes further)
  auto st_k = [&](int r, int b) { return r * kpitch + (TT == 32 ? (r >> 4) << 6 : 0) + b; };

  // ---- unit batches: lane i resolves unit ub + i (ub is uniform). The
  // length and block ids are kept as loaded (clamped when a unit is read
  // out), so nothing waits for these loads until the batch is used.
  struct Batch {
    int ub;
    int seq, tile, len, hg;  // append: tile = ~t for the virtual tile
    int first;               // cascade: the first unit of its virtual sequence
    int id0, id1, id2, id3;  // the tile's blocks (the first kTB)
    int64_t slot;            // append only: slot_mapping[seq] as loaded
  };
  // Lanes past the range resolve the range's last unit: every lane loads,
  // so the loads land in the batch registers with no merge that would wait.
  auto resolve = [&](int ub) -> Batch {
    Batch b;
    b.ub = ub;
    const int u = min(ub + lane, u1 - 1);
    const int hg = u / T;
    const int r = u - hg * T;
    const int s = sk_find_seq(s_pref, NV, r);
    const int t = r - s_pref[s];
    // cascade: a prefix reads its first member's table from token 0 on
    // (its length: its units' tokens), a tail its own row's table from its
    // first unit on (tile = the unit's position in the row)
    const bool pre = CAS && s < NG;
    const int trow = CAS ? (pre ? s_aux[s] : s - NG) : s;
    const int ta = CAS && !pre ? t + s_aux[s] : t;
    const int32_t* row = p.block_tables + static_cast<int64_t>(trow) * p.max_blocks;
    const bool virt = AP && t == s_pref[s + 1] - s_pref[s] - 1;
    // (a virtual tile reads no cache block; its table index could lie past
    // the table's end)
    const int blk_a = virt ? 0 : (ta * TT) / BS;
    b.len = pre ? (s_pref[s + 1] - s_pref[s]) * TT : p.context_lens[trow];
    b.id0 = row[blk_a];
    b.slot = AP ? p.slot_mapping[s] : -1;
    // the tile's further blocks; past the sequence's last block their
    // values are never used (those tokens are masked)
    b.id1 = kTB > 1 ? row[min(blk_a + 1, p.max_blocks - 1)] : 0;
    b.id2 = kTB > 2 ? row[min(blk_a + 2, p.max_blocks - 1)] : 0;
    b.id3 = kTB > 3 ? row[min(blk_a + 3, p.max_blocks - 1)] : 0;
    b.seq = s;
    b.tile = virt ? ~t : ta;
    b.first = t == 0;
    b.hg = hg;
    return b;
  };
  auto block_id = [&](int id) { return static_cast<uint32_t>(id) < static_cast<uint32_t>(p.num_blocks) ? id : 0; };
  // ---- loads of one unit into a ring slot; returns the unit
  // x may lie past the range: the last unit is read out and loaded again
  // (nothing computes it; when staged every lane loads one 16-byte
  // location instead, since the non-temporal loads would fetch the unit
  // from memory again)
  auto load_unit = [&](const Batch& b, int x, u32x4 (&qr)[kQL], u32x4 (&kr)[kKP],
                       VSlot (&vr)[kVL]) -> SkUnit {
    const bool past = x >= u1;
    x = past ? u1 - 1 : x;
    const int o = x - b.ub;
    SkUnit un;
    un.seq = __builtin_amdgcn_readlane(b.seq, o);
    un.tile = __builtin_amdgcn_readlane(b.tile, o);
    un.len = min(__builtin_amdgcn_readlane(b.len, o), p.len_cap);
    un.hg = __builtin_amdgcn_readlane(b.hg, o);
    un.virt = 0;
    un.sblk = -1;
    un.soff = 0;
    un.pre = 0;
    un.first = 0;
    un.qsrc = 0;
    if constexpr (CAS) {
      // a prefix unit needs its segment's q rows when it is the segment's
      // first unit, or the range's (loaded at compute time, or for the
      // range's first unit before the ring starts)
      un.pre = un.seq < NG;
      un.first = __builtin_amdgcn_readlane(b.first, o);
      un.qsrc = un.pre && !past && un.first && x != u0 ? 2 : 0;
    }
    if constexpr (AP) {
      un.virt = un.tile < 0;
      un.tile = un.virt ? ~un.tile : un.tile;
      un.len = un.virt ? 1 : un.len - 1;  // the virtual tile holds token L - 1 alone
      // the slot as loaded, split here (uniform) so the batch never waits
      // for it; a slot outside the pool writes nothing
      const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b.slot), o));
      const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b.slot >> 32), o));
      const int64_t sl = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
      if (sl >= 0 && sl / BS < p.num_blocks) {
        un.sblk = static_cast<int>(sl / BS);
        un.soff = static_cast<int>(sl % BS);
      }
    }
    // the tile's blocks (scalars, not an array: a select over an array
    // would become a per-lane indexed load from scratch)
    const int id0 = block_id(__builtin_amdgcn_readlane(b.id0, o));
    const int id1 = kTB > 1 ? block_id(__builtin_amdgcn_readlane(b.id1, o)) : 0;
    const int id2 = kTB > 2 ? block_id(__builtin_amdgcn_readlane(b.id2, o)) : 0;
    const int id3 = kTB > 3 ? block_id(__builtin_amdgcn_readlane(b.id3, o)) : 0;
    // block i (< kTB) of the tile. The empty asm statements keep the two
    // halves of the choice apart: the compiler would otherwise turn the
    // whole select tree into a per-lane indexed load from scratch.
    auto pick = [&](int i) {
      if constexpr (kTB == 1) {
        return id0;
      } else if constexpr (kTB == 2) {
        return i ? id1 : id0;
      } else {
        int lo = (i & 1) ? id1 : id0;
        int hi = (i & 1) ? id3 : id2;
        asm volatile("" : "+v"(lo));
        asm volatile("" : "+v"(hi));
        return (i & 2) ? hi : lo;
      }
    };
    const int g = un.hg * HW + wave;
    // the unit's q rows (B operand of S^T = K q^T); columns >= G repeat head
    // 0 (finite logits whose weights are forced to zero). Staged, they go
    // to the wave's LDS rows, where they stay for the rest of the segment:
    // only a segment's first unit (or the range's) needs them (measured:
    // reloading them with every unit cost 2-4.5% on every workload). The
    // other units still issue the loads, all lanes at one address (a single
    // cache line), so every unit issues the same loads and the waits the
    // compiler counts for a slot never cover the next slot's loads.
    // Cascade prefix units take their rows from their own path.
    un.qld = !past && (CAS ? (!un.pre && (x == u0 || un.first != 0)) : (x == u0 || un.tile == 0));
    {
      // (cascade: a tail's batch row)
      const int qseq = CAS ? (un.pre ? 0 : un.seq - NG) : un.seq;
      const int64_t head0 = static_cast<int64_t>(qseq) * p.num_q_heads + static_cast<int64_t>(g) * G;
      if constexpr (STG) {
        // lanes past the rows' end repeat a piece (not used)
        const char* qblk = static_cast<const char*>(p.q) + head0 * D * 2;
#pragma unroll
        for (int i = 0; i < kQL; ++i) {
          const int f = (64 * i + lane) * 16;
          const char* qp = un.qld ? qblk + (f < kQBytes ? f : f % kQBytes) : qblk;
          qr[i] = *reinterpret_cast<const u32x4*>(qp);
        }
      } else {
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (head0 + (col < G ? col : 0)) * D;
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) qr[i] = *reinterpret_cast<const u32x4*>(qrow + qk_dim<kB>(i, j));
      }
    }
    // K and V addresses of the unit's rows: from the cache, or (append
    // variant) from the newest token's k_new / v_new row. Both cases issue
    // the same load instructions, so the loads in flight per ring slot stay
    // fixed and the compiler's waits stay tight.
    if constexpr (TV && kB == 2) {
      // the head group's slice of the 16 rows (virtual tile: every row reads
      // the new token's row; rows past the first are masked)
      // uniform bases (the first block's row `tin`, or the new token's row)
      // and 32-bit lane offsets; with 8-token blocks rows 8..15 lie in the
      // tile's second block
      const bool nv = AP && un.virt;
      const int64_t hoff = static_cast<int64_t>(un.hg) * S;
      const int tin = kTB == 1 ? (un.tile * 16) % BS : 0;
      const int64_t base = nv ? (static_cast<int64_t>(un.seq) * Hkv * D) * kB + hoff
                              : static_cast<int64_t>(id0) * blk_bytes + tin * tok_bytes + hoff;
      const char* kb = (nv ? static_cast<const char*>(p.k_new) : kbase) + base;
      const char* vb = (nv ? static_cast<const char*>(p.v_new) : vbase) + base;
      const int64_t blk2 = kTB > 1 ? (static_cast<int64_t>(id1) - id0) * blk_bytes - BS * tok_bytes : 0;
#pragma unroll
      for (int i = 0; i < C::kKLoads; ++i) {
        const int r = st_r(i);
        const uint32_t o = nv ? static_cast<uint32_t>(st_cb(i)) : static_cast<uint32_t>(r * tok_bytes + st_cb(i));
        const int64_t o2 = kTB > 1 && !nv && r >= BS ? blk2 : 0;
        const char* kp = past ? kbase : kb + o2 + o;
        const char* vp = past ? vbase : vb + o2 + o;
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp));
      }
      return un;
    } else if constexpr (STG) {
      // fp8 pools: the head group's slice of the 32 K rows (kTB blocks of BS
      // rows), and of the 32 V rows (token-major) or its dim-major V region
      // of each of those blocks
      const int64_t hoff = static_cast<int64_t>(un.hg) * S;
      const int64_t voff = static_cast<int64_t>(un.hg) * SV;
#pragma unroll
      for (int i = 0; i < kKP; ++i) {
        const int f = st_f(i);
        const int r = f >> s_log2;
        const int64_t ko = static_cast<int64_t>(pick(r / BS)) * blk_bytes + (r % BS) * tok_bytes + hoff + (f & (S - 1));
        const int64_t vo = TV ? ko : static_cast<int64_t>(pick(f >> sv_log2)) * blk_bytes + voff + (f & (SV - 1));
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(past ? kbase : kbase + ko));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(past ? vbase : vbase + vo));
      }
      return un;
    } else {
      const char* krow;  // lane's K row (QK tile 0) minus its first head-dim offset (see below)
      const char* vrun;  // lane's V run for n-tile 0
      if constexpr (TT == 32) {
        // QK tile 0 row `col` is token 8 (col / 4) + col % 4 of the unit and
        // tile 1 row `col` the token 4 past it (same block), so score lane
        // group j holds tokens 8j .. 8j + 7 and the PV operand of lane (d, j)
        // is the run of head dim d over those 8 tokens
        const int tk = 8 * (col >> 2) + (col & 3);
        const int tv = 8 * j;
        const int tin = kTB == 1 ? (un.tile * TT) % BS : 0;
        const int idk = pick(tk / BS);
        const int idv = pick(tv / BS);
        krow = kbase + static_cast<int64_t>(idk) * blk_bytes + (tin + tk % BS) * tok_bytes +
               static_cast<int64_t>(g) * D * kB;
        vrun = vbase + static_cast<int64_t>(idv) * blk_bytes + ((static_cast<int64_t>(g) * D + col) * BS + tin + tv % BS) * kB;
      } else if constexpr (BS >= 16) {
        const int tin = (un.tile * 16) % BS;
        krow = kbase + static_cast<int64_t>(id0) * blk_bytes + tin * tok_bytes + static_cast<int64_t>(g) * D * kB +
               koff_lane - qk_dim<kB>(0, j) * kB;
        vrun = vbase + static_cast<int64_t>(id0) * blk_bytes + (static_cast<int64_t>(g) * D * BS + tin) * kB + voff_lane;
      } else {
        // a tile spans two blocks: tokens 0..BS-1 in the first, the rest in the second
        const int idk = pick(col / BS);
        krow = kbase + static_cast<int64_t>(idk) * blk_bytes + (col % BS) * tok_bytes + static_cast<int64_t>(g) * D * kB;
        const int t4 = 4 * j;
        const int idv = pick(t4 / BS);
        vrun = vbase + static_cast<int64_t>(idv) * blk_bytes + ((static_cast<int64_t>(g) * D + col) * BS + t4 % BS) * kB;
      }
      int vstep = kVTileBytes;
      if constexpr (AP) {
        if (un.virt) {
          // every K row reads the new token's row (rows past the first are
          // masked); lane (d, j) reads the 4-dim group holding v_new[d] (the
          // compute step moves element d % 4 into the first token's place)
          krow = static_cast<const char*>(p.k_new) + (static_cast<int64_t>(un.seq) * Hkv + g) * D * kB;
          vrun = static_cast<const char*>(p.v_new) + ((static_cast<int64_t>(un.seq) * Hkv + g) * D + (col & ~3)) * kB;
          vstep = 16 * kB;
        }
      }
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
#pragma unroll
        for (int i = 0; i < C::kKLoads; ++i) {
          const int off = kB == 2 ? 2 * qk_dim<2>(i, j) : qk_dim<1>(2 * i, j);
          kr[s * C::kKLoads + i] = *reinterpret_cast<const u32x4*>(krow + s * 4 * tok_bytes + off);
        }
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) vr[nt] = *reinterpret_cast<const VSlot*>(vrun + nt * vstep);
      return un;
    }
  };

  // ---- segment state. A segment is the run of units of one (head group,
  // sequence) inside this workgroup's range; its identity comes with each
  // unit, so nothing is looked up when one ends and the next begins.
  bool seg_first = true;  // reaches back to u0
  bool seg_begun = true;  // starts inside the range (set from the first unit below)

  // per q row tile ct (one, or two for cascade prefix units): running
  // reference max of row `col` (log2 domain), this lane's share of its
  // weight sum, the output accumulators
  float m_w[CT], l_w[CT];
  f32x4 acc[CT][kNT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_w[ct] = -INFINITY;
    l_w[ct] = 0.f;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int pre_rows = 0;  // cascade: q rows of the current prefix segment
  // the segment state back to empty, for the segment starting at the next unit
  auto reset_segment = [&]() {
    seg_first = false;
    seg_begun = true;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      m_w[ct] = -INFINITY;
      l_w[ct] = 0.f;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // Staged path: the stores of a segment end (and the append's cache write)
  // wait for the next unit and are issued once its rows have been written
  // to the stage. A store issued while the next unit's loads are in flight
  // holds up the wait for those loads until the store completes (the waits
  // count loads and stores alike, in order); measured, 1-3 us per segment
  // end, 7-8% of the call on the mixed-length batches.
  // (pending when pf_seq / ap_blk >= 0; pf_bits: complete, ends here,
  // begun, slot; ap_oh: token offset | head group << 8)
  int pf_seq = -1, pf_hg = 0, pf_bits = 0, pf_rows = 0;
  int ap_blk = -1, ap_oh = 0;

  // cascade: the q rows of prefix segment v for this wave's KV head in
  // head group hg, as the QK B operands of the two row tiles; row r =
  // 16 ct + col is member r / G of the group, query head r % G. Rows past
  // the group (or a member id outside the batch) read row 0's q: their
  // weights are forced to zero. Returns the valid rows.
  using PreQ = u32x4[CT][C::kKSteps];
  auto fetch_prefix_q = [&](int v, int hg, PreQ& dst) -> int {
    const int m0 = s_goff[v];
    const int gsz = max(0, s_goff[v + 1] - m0);
    const int64_t gq = static_cast<int64_t>(hg * HW + wave) * G;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int r = ct * 16 + col;
      int mem = r / G < gsz ? s_mem[m0 + r / G] : 0;
      mem = static_cast<unsigned>(mem) < static_cast<unsigned>(B) ? mem : 0;
      const uint16_t* qrow =
          static_cast<const uint16_t*>(p.q) + (mem * static_cast<int64_t>(p.num_q_heads) + gq + r % G) * D;
#pragma unroll
      for (int i = 0; i < C::kKSteps; ++i) dst[ct][i] = *reinterpret_cast<const u32x4*>(qrow + qk_dim<kB>(i, j));
    }
    return min(gsz, RW / G) * G;
  };
  // ... into the wave's q rows in LDS (read back per unit like a tail's)
  auto store_prefix_q = [&](const PreQ& src) {
    char* qs = reinterpret_cast<char*>(s_out);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int i = 0; i < C::kKSteps; ++i)
        *reinterpret_cast<u32x4*>(qs + (ct * 16 + col) * kQPitch + qk_dim<kB>(i, j) * 2) = src[ct][i];
    }
  };

  // store the segment that just ended: final output, or a partial piece.
  // Lane (col, j) holds rows 4j .. 4j + 3, head dim 16 nt + col. Through
  // the wave's LDS region (kTileRows rows at a time: all G rows when it
  // holds G x D floats, the append variant's, else half), the rows leave as
  // 4-element stores; otherwise (G < 4, the cascade) each lane stores its
  // elements (16 lanes write 16 consecutive dims). Cascade: a completed
  // segment leaves its partial (m, l, o) as state rows of its batch rows
  // (part 0: prefix, 1: tail), a cut one a piece of RW rows. begun: the
  // segment starts inside the range; prows: a cascade prefix segment's q
  // rows. The wave's q rows in LDS are overwritten.
  auto flush = [&](int seg_seq, int seg_hg, bool complete, bool ends_here, int slot, bool begun, int prows) {
    const int64_t pbase = ((static_cast<int64_t>(w) * p.piece_slots + slot) * HW + wave) * RW;
    if constexpr (CAS) {
      const bool pre = seg_seq < NG;
      const int nrows = pre ? prows : G;
      const int64_t gq = static_cast<int64_t>(seg_hg * HW + wave) * G;
      const int m0 = pre ? s_goff[seg_seq] : 0;
      const int64_t part = pre ? 0 : 1;
      // state row of wave row rr: (batch row, query head), or -1 (a member
      // id outside the batch)
      auto state_row = [&](int rr) -> int64_t {
        const int srow = pre ? s_mem[m0 + rr / G] : seg_seq - NG;
        if (static_cast<unsigned>(srow) >= static_cast<unsigned>(B)) return -1;
        return (part * B + srow) * p.num_q_heads + gq + rr % G;
      };
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if (ct > 0 && !pre) break;
        const float l_head = pair32_sum(pair16_sum(l_w[ct]));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = ct * 16 + 4 * j + r;
          const float lr = __shfl(l_head, 4 * j + r, 64);  // lane h (row 0) holds row h's sum
          if (rr < nrows) {
            const float inv = p.v_scale / lr;
            const int64_t row = complete ? state_row(rr) : pbase + rr;
            if (row >= 0) {
              float* po = (complete ? p.state_o : p.piece_o) + row * D + col;
#pragma unroll
              for (int nt = 0; nt < kNT; ++nt) po[nt * 16] = acc[ct][nt][r] * inv;
            }
          }
        }
        if (lane < 16 && ct * 16 + lane < nrows) {
          const int64_t row = complete ? state_row(ct * 16 + lane) : pbase + ct * 16 + lane;
          if (row >= 0) {
            (complete ? p.state_m : p.piece_m)[row] = m_w[ct];
            (complete ? p.state_l : p.piece_l)[row] = l_head;
          }
        }
      }
    } else {
      const float l_head = pair32_sum(pair16_sum(l_w[0]));
      const int64_t head0 =
          static_cast<int64_t>(seg_seq) * p.num_q_heads + static_cast<int64_t>(seg_hg * HW + wave) * G;
      // the rows' scales: v_scale / l on the lane holding row h's sum (lane
      // h < 16), then to the lanes holding the row's outputs (a segment end
      // is a short chain of dependent steps that every wave of the
      // workgroup runs at once: measured, it cost ~2 us per segment end
      // with a division per row and per-element conversions)
      const float inv_h = p.v_scale * __builtin_amdgcn_rcpf(l_head);
      float inv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) inv[r] = __shfl(inv_h, 4 * j + r, 64);
      if constexpr (kTileRows > 0) {
        // element type of the rows: fp32 (pieces, float output), bf16, f16
        const int odt = complete ? p.out_dtype : 2;
        float* const o32 = complete ? static_cast<float*>(p.out) + head0 * D : p.piece_o + pbase * D;
        uint16_t* const o16 = static_cast<uint16_t*>(p.out) + head0 * D;
        // 4 elements per lane per round: 16-byte LDS reads of consecutive
        // lanes are conflict free
        constexpr int kRounds = (kTileRows * D + 255) / 256;
#pragma unroll
        for (int h0 = 0; h0 < G; h0 += kTileRows) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = 4 * j + r;
            if (h >= h0 && h < h0 + kTileRows) {
#pragma unroll
              for (int nt = 0; nt < kNT; ++nt) s_out[(h - h0) * D + nt * 16 + col] = acc[0][nt][r] * inv[r];
            }
          }
          wave_lds_sync();
#pragma unroll
          for (int it = 0; it < kRounds; ++it) {
            const int i = it * 256 + lane * 4;
            if ((kTileRows * D) % 256 == 0 || i < kTileRows * D) {
              const f32x4 a = *reinterpret_cast<const f32x4*>(s_out + i);
              const int64_t e = static_cast<int64_t>(h0) * D + i;  // element of the rows
              if (odt == 2) {
                *reinterpret_cast<f32x4*>(o32 + e) = a;
              } else if (odt == 1) {
                *reinterpret_cast<u32x2*>(o16 + e) = u32x2{pack2<BF16>(a.x, a.y), pack2<BF16>(a.z, a.w)};
              } else {
                *reinterpret_cast<u32x2*>(o16 + e) = u32x2{pack2<F16>(a.x, a.y), pack2<F16>(a.z, a.w)};
              }
            }
          }
          wave_lds_sync();
        }
      } else {
        // one loop per element type: fp32 rows (pieces, or a float output),
        // bf16 or f16 output rows
        auto rows = [&](auto* o, auto cvt) {  // (G < 4)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = 4 * j + r;
            if (h < G) {
#pragma unroll
              for (int nt = 0; nt < kNT; ++nt) o[h * D + nt * 16 + col] = cvt(acc[0][nt][r] * inv[r]);
            }
          }
        };
        if (!complete || p.out_dtype == 2) {
          rows(complete ? static_cast<float*>(p.out) + head0 * D : p.piece_o + pbase * D, [](float v) { return v; });
        } else if (p.out_dtype == 1) {
          rows(static_cast<uint16_t*>(p.out) + head0 * D,
               [](float v) { return static_cast<uint16_t>(f32_to_bf16_bits(v)); });
        } else {
          rows(static_cast<uint16_t*>(p.out) + head0 * D,
               [](float v) { return static_cast<uint16_t>(f32_to_f16_bits(v)); });
        }
      }
      if (!complete && lane < G) {
        p.piece_m[pbase + lane] = m_w[0];
        p.piece_l[pbase + lane] = l_head;
      }
    }
    if (wave == 0 && lane == 0 && p.seg_desc != nullptr) {  // (none when no segment is cut)
      int32_t* desc = p.seg_desc + (static_cast<int64_t>(seg_hg) * NV + seg_seq) * 2;
      if (complete) {
        desc[0] = -1;
      } else {
        if (begun) desc[0] = static_cast<int32_t>(static_cast<uint32_t>(w) | (static_cast<uint32_t>(slot) << 31));
        if (ends_here) desc[1] = w;
      }
    }
  };

  // append: the new token's element v_new[d] (d = lane's dim) out of the
  // four-dim group its lane loaded
  auto virt_v = [&](const u32x2& grp) -> uint32_t {
    const uint32_t w2 = (col & 2) ? grp.y : grp.x;
    return (col & 1) ? (w2 >> 16) : (w2 & 0xffffu);
  };

  // staged: the wave's K rows of a unit in the QK operand layout, from the
  // unit's stage (lane (token col, j): the 16 bytes of dims qk_dim(i, j);
  // fp8: QK tile s row `col` is token 8 (col / 4) + col % 4 + 4 s)
  auto read_kop = [&](const char* stg, u32x4 (&kop)[STG ? kKP : 1]) {
    if constexpr (STG) {
      if constexpr (TT == 16) {
        const char* ks = stg + col * kpitch + wave * D * kB;
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) kop[i] = *reinterpret_cast<const u32x4*>(ks + qk_dim<2>(i, j) * kB);
      } else {
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
          const int row = 8 * (col >> 2) + (col & 3) + 4 * s;
#pragma unroll
          for (int a = 0; a < C::kKLoads; ++a)
            kop[s * C::kKLoads + a] =
                *reinterpret_cast<const u32x4*>(stg + st_k(row, wave * D + qk_dim<1>(2 * a, j)));
        }
      }
    }
  };

  auto compute = [&](int x, const SkUnit& un, const u32x4 (&qr)[kQL], const u32x4 (&kr)[kKP],
                     const VSlot (&vr)[kVL]) {
    const int tb = AP && un.virt ? 0 : un.tile * TT;
    const int L = un.len;
    const bool upre = CAS && un.pre;  // (uniform) a cascade prefix unit: both row tiles
    if constexpr (CAS) {
      if (un.qsrc == 2) {
        PreQ qt;
        pre_rows = fetch_prefix_q(un.seq, un.hg, qt);
        store_prefix_q(qt);
      }
    }
    char* const stg = stage + (NBUF == 2 && (x & 1) ? sbytes : 0);  // this unit's stage
    char* const stg_v = stg + (stage_v - stage);
    // ---- token-major V: the unit's rows go to the stage as loaded; after
    // the barrier each wave reads its head's K rows in the QK operand layout
    // (lane (token col, j): the 16 bytes of dims qk_dim(i, j)) and later its
    // V rows with the transposing read (lane (d, j): tokens 4j .. 4j + 3 of
    // head dim 16 nt + d, its group's lanes pointing at rows 4j + lane / 4,
    // dims 4 (lane % 4) ..)
    u32x4 kop[STG ? kKP : 1];
    u32x2 vpre[STG ? kNT : 1];  // staged: the unit's V operands (see below)
    const uint16_t* vt_src = nullptr;
    const char* v8_src = nullptr;
    char* const qs = reinterpret_cast<char*>(s_out);  // the wave's q rows (staged)
    if constexpr (STG) {
#pragma unroll
      for (int i = 0; i < kKP; ++i) {
        *reinterpret_cast<u32x4*>(stg + st_k(st_r(i), st_cb(i))) = kr[i];
        if constexpr (TV && kB == 2) {
          *reinterpret_cast<u32x4*>(stg_v + st_r(i) * vpitch + st_cb(i)) = vr[i];
        } else if constexpr (TV) {
          // fp8 token-major V: the codes as loaded, laid out like K
          *reinterpret_cast<u32x4*>(stg_v + st_k(st_r(i), st_cb(i))) = vr[i];
        } else {
          // dim-major V (fp8): chunk-major, [part][head][8-token chunk][dim]
          // [8 bytes], so the 16 lanes of an operand read (16 head dims, one
          // chunk) read 128 contiguous bytes
          const int f = st_f(i);
          const int off = f & (SV - 1);
          char* hb = stg_v + (f - off) + (off / (D * BS)) * (D * BS);
          const int rem = off % (D * BS);
          const int d = rem / BS, t = rem % BS;
          if constexpr (BS == 8) {
            *reinterpret_cast<u32x4*>(hb + d * 8) = vr[i];  // dims d, d + 1
          } else {
            *reinterpret_cast<u32x2*>(hb + (t / 8) * (D * 8) + d * 8) = u32x2{vr[i].x, vr[i].y};
            *reinterpret_cast<u32x2*>(hb + (t / 8 + 1) * (D * 8) + d * 8) = u32x2{vr[i].z, vr[i].w};
          }
        }
      }
      // append: the new token's row of the head group into its cache slot,
      // from the workgroup's pieces of row 0 (every row of the virtual tile
      // holds it). With two stages it waits for the next unit and is taken
      // from the previous unit's stage, intact until this unit's barrier.
      if constexpr (AP) {
        auto cache_row = [&](int blk, int off, int hg) {
          return static_cast<int64_t>(blk) * blk_bytes + off * tok_bytes + static_cast<int64_t>(hg) * S;
        };
        if constexpr (NBUF == 2) {
          if (ap_blk >= 0) {
            const char* ps = stage + (x & 1 ? 0 : sbytes);  // the previous unit's stage
            const int64_t dst = cache_row(ap_blk, ap_oh & 255, ap_oh >> 8);
#pragma unroll
            for (int i = 0; i < C::kKLoads; ++i) {
              if (st_r(i) == 0) {
                *reinterpret_cast<u32x4*>(const_cast<char*>(kbase) + dst + st_cb(i)) =
                    *reinterpret_cast<const u32x4*>(ps + st_k(0, st_cb(i)));
                *reinterpret_cast<u32x4*>(const_cast<char*>(vbase) + dst + st_cb(i)) =
                    *reinterpret_cast<const u32x4*>(ps + (stage_v - stage) + st_cb(i));
              }
            }
            ap_blk = -1;
          }
        }
        if (un.virt && static_cast<uint32_t>(un.sblk) < static_cast<uint32_t>(p.num_blocks)) {
          if (NBUF == 2 && x + 1 < u1) {
            ap_blk = un.sblk;
            ap_oh = un.soff | (un.hg << 8);
          } else {
            const int64_t dst = cache_row(un.sblk, un.soff, un.hg);
#pragma unroll
            for (int i = 0; i < C::kKLoads; ++i) {
              if (st_r(i) == 0) {
                *reinterpret_cast<u32x4*>(const_cast<char*>(kbase) + dst + st_cb(i)) = kr[i];
                *reinterpret_cast<u32x4*>(const_cast<char*>(vbase) + dst + st_cb(i)) = vr[i];
              }
            }
          }
        }
      }
      // the previous unit's segment end, then this unit's q rows (if it
      // starts a segment) into the wave's LDS region the end passed through.
      // Both come after the stage writes, which wait for the last of this
      // unit's loads: no store is issued before that wait, and the q rows
      // (loaded first) have landed by then.
      if (pf_seq >= 0) {
        flush(pf_seq, pf_hg, pf_bits & 1, (pf_bits >> 1) & 1, pf_bits >> 3, (pf_bits >> 2) & 1, pf_rows);
        reset_segment();
        pf_seq = -1;
      }
      if (!upre && un.qld) {
#pragma unroll
        for (int i = 0; i < kQL; ++i) {
          const int f = (64 * i + lane) * 16;
          if (f < kQBytes) *reinterpret_cast<u32x4*>(qs + (f / (D * 2)) * kQPitch + f % (D * 2)) = qr[i];
        }
      }
      lds_barrier();
      read_kop(stg, kop);
      if constexpr (TT == 16) {
        vt_src = reinterpret_cast<const uint16_t*>(stg_v + (4 * j + (col >> 2)) * vpitch + wave * D * kB) + 4 * (col & 3);
      } else {
        // fp8: the PV operand of lane (d, j) is the run of head dim d over
        // tokens 8j .. 8j + 7 (block part 8j / BS of the V stage)
        if constexpr (TV) {
          // one 8-bit transposing read per 16-dim tile: lane m of group j
          // points at row 8j + m / 2, dims 8 (m % 2) .. of the tile, and
          // lane `col` receives dim col of tokens 8j .. 8j + 7
          v8_src = stg_v + st_k(8 * j + (col >> 1), wave * D + 8 * (col & 1));
        } else {
          v8_src = stg_v + ((8 * j) / BS) * SV + wave * D * BS + (((8 * j) % BS) / 8) * (D * 8) + col * 8;
        }
      }
      // the V operands of every n-tile (both q tiles of a cascade prefix
      // unit use them), read with the K operands: issued one n-tile at a
      // time inside the PV loop, each read's latency sat between two pairs
      // of MFMAs
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        if constexpr (TT == 16) {
          vpre[nt] = lds_read_tr16(vt_src + 16 * nt);
        } else if constexpr (TV) {
          vpre[nt] = lds_read_tr8(v8_src + 16 * nt);
        } else {
          vpre[nt] = *reinterpret_cast<const u32x2*>(v8_src + nt * 16 * 8);
        }
      }
    }
    // ---- PV masks: V elements past the end are zeroed (the pool may hold
    // anything there, and 0 * NaN would poison the sum)
    uint32_t vmask[kE / 2];
#pragma unroll
    for (int e = 0; e < kE; e += 2) vmask[e / 2] = 0xffffffffu;
    if (tb + TT > L) {
      const int t = tb + kE * j;
#pragma unroll
      for (int e = 0; e < kE; e += 2)
        vmask[e / 2] = (t + e < L ? 0xffffu : 0u) | (t + e + 1 < L ? 0xffff0000u : 0u);
    }
    // ---- per q row tile ct: QK, online softmax, PV. A cascade prefix unit
    // runs both tiles on the same K and V operands, one after the other
    // (interleaving the two chains needs more than the 256 VGPRs of two
    // waves per SIMD: the build spilled 21-59 of them).
    // QK: S^T = K q^T, one 16-row tile per kSub; lane (row col, j) gets the
    // scores of tokens kE * j + e, e = 4 * tile + row
    auto qk = [&](auto ctc, f32x4 (&sacc)[kSub]) {
      constexpr int ct = decltype(ctc)::value;
      // the q rows as the QK B operand (a wave's G heads: columns >= G
      // repeat row 0; a prefix segment: rows 16 ct ..)
      u32x4 qb[C::kKSteps];
      if constexpr (STG) {
        const char* qsrc = qs + (upre ? ct * 16 + col : (col < G ? col : 0)) * kQPitch;
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) qb[i] = *reinterpret_cast<const u32x4*>(qsrc + qk_dim<kB>(i, j) * 2);
      } else {
#pragma unroll
        for (int i = 0; i < C::kKSteps; ++i) qb[i] = qr[i];
      }
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kB == 2) {
#pragma unroll
          for (int i = 0; i < C::kKSteps; ++i) sacc[s] = mfma_16x16x32<QT>(TV ? kop[i] : kr[i], qb[i], sacc[s]);
        } else {
#pragma unroll
          for (int a = 0; a < C::kKLoads; ++a) {
            const u32x4 kw = STG ? kop[s * C::kKLoads + a] : kr[s * C::kKLoads + a];
            const u32x2 b0 = e4m3x4_to_bf16x4(kw.x), b1 = e4m3x4_to_bf16x4(kw.y);
            const u32x2 b2 = e4m3x4_to_bf16x4(kw.z), b3 = e4m3x4_to_bf16x4(kw.w);
            sacc[s] = mfma_16x16x32<QT>(u32x4{b0.x, b0.y, b1.x, b1.y}, qb[2 * a], sacc[s]);
            sacc[s] = mfma_16x16x32<QT>(u32x4{b2.x, b2.y, b3.x, b3.y}, qb[2 * a + 1], sacc[s]);
          }
        }
      }
    };
    // online softmax (row = col); rows holding a q row: the wave's G heads,
    // or a prefix segment's rows. Weights as two 16-bit terms (hi + lo), the
    // PV A operand: row = q row, k = the lane's kE tokens. fp8 pools: one
    // f16 term, and V widened to f16: every E4M3 value is exact in f16
    // (4 significant bits, 2^-9 .. 448), so PV runs on the f16 MFMA with
    // the weight rounded once (relative error <= 2^-12 each, against 2^-9
    // for a single bf16 term), half the MFMAs of the two-term form (mixed
    // fp8 batch 184 -> 178 us per call).
    auto softmax = [&](auto ctc, const f32x4 (&sacc)[kSub], uint32_t (&phi)[kE / 2], uint32_t (&plo)[kE / 2]) {
      constexpr int ct = decltype(ctc)::value;
      const bool rok = CAS && upre ? ct * 16 + col < pre_rows : col < G;
      float sv[kE];
#pragma unroll
      for (int e = 0; e < kE; ++e) sv[e] = tb + kE * j + e < L ? sacc[e / 4][e % 4] * p.qk_scale_log2 : -INFINITY;
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < kE; ++e) mx = fmaxf(mx, sv[e]);
      mx = pair32_max(pair16_max(mx));
      const bool need = rok && mx > m_w[ct] + C::kSlack;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float a = need ? __builtin_amdgcn_exp2f(m_w[ct] - mx) : 1.0f;
        m_w[ct] = need ? mx : m_w[ct];
        l_w[ct] *= a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(a, 4 * j + r, 64);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) acc[ct][nt][r] *= ar;
        }
      }
      float pw[kE];
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        pw[e] = rok ? __builtin_amdgcn_exp2f(sv[e] - m_w[ct]) : 0.f;
        l_w[ct] += pw[e];
      }
#pragma unroll
      for (int e = 0; e < kE; e += 2) {
        if constexpr (kB == 1) {
          phi[e / 2] = pack2<F16>(pw[e], pw[e + 1]);
          plo[e / 2] = 0u;
        } else {
          phi[e / 2] = pack2<QT>(pw[e], pw[e + 1]);
          plo[e / 2] = pack2<QT>(pw[e] - half_lo<QT>(phi[e / 2]), pw[e + 1] - half_hi<QT>(phi[e / 2]));
        }
      }
    };
    // PV of tile 0. 16-token units: one v_mfma_f32_16x16x32 per n-tile
    // takes both weight terms, its k slots of lane group j holding the hi
    // and then the lo weights of tokens 4j .. 4j + 3 against the same V
    // values twice (the two 16x16x16 products in one instruction)
    auto pv = [&](auto ntc, const uint32_t (&phi)[CT][kE / 2], const uint32_t (&plo)[CT][kE / 2]) {
      constexpr int NT = decltype(ntc)::value;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        if constexpr (TT == 16) {
          u32x2 vop;
          if constexpr (TV) {
            vop = vpre[nt];
          } else {
            vop = vr[nt];
            if constexpr (AP) {
              if (un.virt) vop = u32x2{virt_v(vr[nt]), 0u};
            }
          }
          vop.x &= vmask[0];
          vop.y &= vmask[1];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            acc[ct][nt] = mfma_16x16x32<QT>(u32x4{phi[ct][0], phi[ct][1], plo[ct][0], plo[ct][1]},
                                            u32x4{vop.x, vop.y, vop.x, vop.y}, acc[ct][nt]);
          }
        } else {
          u32x2 b0, b1;  // the lane's 8 tokens of its head dim as bf16
          if constexpr (TV) {
            const u32x2 codes = vpre[nt];  // tokens 8j .. 8j + 7, dim col
            b0 = e4m3x4_to_f16x4(codes.x);
            b1 = e4m3x4_to_f16x4(codes.y);
          } else {
            u32x2 vv;
            if constexpr (STG) {
              vv = vpre[nt];
            } else {
              vv = vr[nt];
            }
            b0 = e4m3x4_to_f16x4(vv.x);
            b1 = e4m3x4_to_f16x4(vv.y);
          }
          const u32x4 vop = {b0.x & vmask[0], b0.y & vmask[1], b1.x & vmask[2], b1.y & vmask[3]};
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            acc[ct][nt] = mfma_16x16x32<F16>(u32x4{phi[ct][0], phi[ct][1], phi[ct][2], phi[ct][3]}, vop, acc[ct][nt]);
          }
        }
      }
    };
    // PV of tile 1 alone (the same V operands)
    auto pv1 = [&](const uint32_t (&phi)[CT][kE / 2], const uint32_t (&plo)[CT][kE / 2]) {
      if constexpr (CT > 1) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          if constexpr (TT == 16) {
            u32x2 vop;
            if constexpr (TV) {
              vop = vpre[nt];
            } else {
              vop = vr[nt];
            }
            vop.x &= vmask[0];
            vop.y &= vmask[1];
            acc[1][nt] = mfma_16x16x32<QT>(u32x4{phi[1][0], phi[1][1], plo[1][0], plo[1][1]},
                                           u32x4{vop.x, vop.y, vop.x, vop.y}, acc[1][nt]);
          } else {
            u32x2 b0, b1;
            if constexpr (TV) {
              const u32x2 codes = vpre[nt];
              b0 = e4m3x4_to_f16x4(codes.x);
              b1 = e4m3x4_to_f16x4(codes.y);
            } else {
              u32x2 vv;
              if constexpr (STG) {
                vv = vpre[nt];
              } else {
                vv = vr[nt];
              }
              b0 = e4m3x4_to_f16x4(vv.x);
              b1 = e4m3x4_to_f16x4(vv.y);
            }
            const u32x4 vop = {b0.x & vmask[0], b0.y & vmask[1], b1.x & vmask[2], b1.y & vmask[3]};
            acc[1][nt] = mfma_16x16x32<F16>(u32x4{phi[1][0], phi[1][1], phi[1][2], phi[1][3]}, vop, acc[1][nt]);
          }
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    uint32_t phi[CT][kE / 2], plo[CT][kE / 2];
    {
      f32x4 s0[kSub];
      qk(I0{}, s0);
      softmax(I0{}, s0, phi[0], plo[0]);
      pv(I1{}, phi, plo);
    }
    if constexpr (CAS) {
      if (upre) {
        // (the K operand is read again: holding it across the first tile's
        // softmax and PV costs more registers than the reads)
        read_kop(stg, kop);
        f32x4 s1[kSub];
        qk(I1{}, s1);
        softmax(I1{}, s1, phi[1], plo[1]);
        pv1(phi, plo);
      }
    }
    // ---- append (dim-major V): write the newest token's row into its cache
    // slot (token-major V: done with the stage write above)
    if constexpr (AP && !TV) {
      if (un.virt && static_cast<uint32_t>(un.sblk) < static_cast<uint32_t>(p.num_blocks)) {
        {
          const int g = un.hg * HW + wave;
          char* kdst = const_cast<char*>(kbase) + static_cast<int64_t>(un.sblk) * blk_bytes + un.soff * tok_bytes +
                       static_cast<int64_t>(g) * D * kB;
          if (col == 0) {
#pragma unroll
            for (int i = 0; i < C::kKLoads; ++i) *reinterpret_cast<u32x4*>(kdst + qk_dim<kB>(i, j) * kB) = kr[i];
          }
          uint16_t* vdst = reinterpret_cast<uint16_t*>(const_cast<char*>(vbase) + static_cast<int64_t>(un.sblk) * blk_bytes) +
                           (static_cast<int64_t>(g) * D + col) * BS + un.soff;
          if (j == 0) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) vdst[nt * 16 * BS] = static_cast<uint16_t>(virt_v(vr[nt]));
          }
        }
      }
    }
    // ---- end of a segment: store it (staged: with the next unit, see
    // above), then start the next one at x + 1
    const bool seq_end = AP ? un.virt != 0 : un.tile == (L + TT - 1) / TT - 1;
    if (seq_end || x + 1 == u1) {
      const bool complete = seg_begun && seq_end;
      const int slot = seg_first ? 0 : 1;
      if (STG && x + 1 < u1) {
        // (uniform values; kept in scalar registers, so the stores branch
        // on them as a wave)
        pf_seq = __builtin_amdgcn_readfirstlane(un.seq);
        pf_hg = __builtin_amdgcn_readfirstlane(un.hg);
        pf_bits = __builtin_amdgcn_readfirstlane((complete ? 1 : 0) | (seq_end ? 2 : 0) | (seg_begun ? 4 : 0) |
                                                 (slot << 3));
        pf_rows = __builtin_amdgcn_readfirstlane(pre_rows);
      } else {
        flush(un.seq, un.hg, complete, seq_end, slot, seg_begun, pre_rows);
        if (x + 1 < u1) reset_segment();
      }
    }
  };

  // after each unit: the waves stay in step (without it the oldest wave of
  // each SIMD takes most issue slots and finishes far ahead); with the
  // stage, every wave has also read the unit's rows before the next unit's
  // rows overwrite them
  auto unit_barrier = [&]() {
    if constexpr (STG) {
      if constexpr (NBUF == 1) lds_barrier();
    } else {
      __builtin_amdgcn_s_barrier();
    }
  };

  // ---- the ring: unit x + 1 in flight while x is computed (measured: a
  // third slot, two units in flight, was 1-5% slower on every workload and
  // held ~40 more VGPRs). Loads are unconditional: past the range they
  // repeat the last unit (an L2 hit; one location when staged), so every
  // path through the loop carries the same loads.
  // Batches: an outer step covers 62 units (31 ring iterations); its batch
  // holds the units it loads (uk + 1 .. uk + 64), and the next step's batch
  // is requested when the step starts.
  u32x4 q0[kQL], q1[kQL];
  u32x4 k0[kSub * C::kKLoads], k1[kSub * C::kKLoads];
  VSlot v0[kVL], v1[kVL];
  const int ulast = u1 - 1;
  Batch cur = resolve(u0);
  Batch nxt = resolve(min(u0 + 1, ulast));
  // cascade: the range's first unit, if a prefix unit, needs its segment's
  // q rows: loaded ahead of the ring's loads (so waiting for them waits
  // for nothing else) and stored once those are out
  PreQ q_first;
  const int v_first = CAS ? __builtin_amdgcn_readlane(cur.seq, 0) : 0;
  if constexpr (CAS) {
    if (v_first < NG) pre_rows = fetch_prefix_q(v_first, __builtin_amdgcn_readlane(cur.hg, 0), q_first);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the prologue issues its loads in the loop's order (K then V), so the
  // wait counts the compiler derives for the loop hold on entry too
  SkUnit n0 = load_unit(cur, u0, q0, k0, v0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (CAS) {
    if (v_first < NG) store_prefix_q(q_first);
  }
  seg_begun = CAS ? n0.first != 0 : n0.tile == 0;
  int uk = u0;
  do {
    cur = nxt;
    nxt = resolve(min(uk + 63, ulast));
    const int uend = min(uk + 62, u1);
    int u = uk;
    do {
      SkUnit n1 = load_unit(cur, u + 1, q1, k1, v1);
      compute(u, n0, q0, k0, v0);
      unit_barrier();
      n0 = load_unit(cur, u + 2, q0, k0, v0);
      if (u + 1 <= ulast) compute(u + 1, n1, q1, k1, v1);
      unit_barrier();
      u += 2;
    } while (u < uend);
    uk += 62;
  } while (uk <= ulast);
}

// One build of the balanced kernel (NBUF stages), or of its cascade variant.
template <typename KV, typename QT, int D, int BS, int G, bool AP, bool TV, int NBUF, bool CAS = false>
hipError_t launch_decode_sk_n(const SkParams& p, int cus, int max_wgs, hipStream_t stream, int* wgs) {
  const int HW = p.heads_per_wg;
  const size_t lds =
      sk_lds_bytes(p.batch, HW, G, D, TV || KV::kBytes == 1, KV::kBytes, TV, NBUF, AP, CAS ? p.num_groups : -1);
  const void* fn = reinterpret_cast<const void*>(paged_decode_sk_kernel<KV, QT, D, BS, G, AP, TV, NBUF, CAS>);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  // more than 64 KiB of dynamic LDS (the stage) must be allowed per kernel
  // and device; the grant only grows (host_cache.h)
  static LdsGrant grant(64 * 1024);  // per instantiation
  if (!grant.ensure(dev, static_cast<int>(lds), [&](int bytes) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        return e == hipSuccess;
      }))
    return e;
  // occupancy per (HW, LDS in 4 KiB steps)
  static IntTable<9, 41> occupancy;  // per instantiation
  const int lb = static_cast<int>((lds + 4095) / 4096);
  const int occ = occupancy.get(HW, lb, [&]() {
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, paged_decode_sk_kernel<KV, QT, D, BS, G, AP, TV, NBUF, CAS>,
                                                     64 * HW, lds);
    return e == hipSuccess ? n : 0;
  });
  if (e != hipSuccess) return e;
  if (occ <= 0) return hipErrorInvalidConfiguration;
  // balanced: the resident workgroups, less those of one CU in 32 (one
  // per XCD on MI355X; measured: the GQA batch's call 1% faster, long and
  // mixed batches unchanged); partition mode: one per partition
  const int used_cus = cus > 32 ? cus - cus / 32 : cus;
  int W = p.part_tiles > 0 ? max_wgs : used_cus * occ;
  W = W < max_wgs ? W : max_wgs;
  *wgs = W;
  hipLaunchKernelGGL((paged_decode_sk_kernel<KV, QT, D, BS, G, AP, TV, NBUF, CAS>), dim3(W), dim3(64 * HW), lds,
                     stream, p);
  return hipGetLastError();
}

// Launch of the balanced kernel: W = resident workgroups (occupancy x CUs),
// at most max_wgs. Writes the grid size used to *wgs. p.stage_bufs = 2
// takes the two-stage build (built for the staged path).
template <typename KV, typename QT, int D, int BS, int G, bool AP, bool TV>
hipError_t launch_decode_sk(const SkParams& p, int cus, int max_wgs, hipStream_t stream, int* wgs) {
  if constexpr (TV || KV::kBytes == 1) {
    if (p.stage_bufs > 1) return launch_decode_sk_n<KV, QT, D, BS, G, AP, TV, 2>(p, cus, max_wgs, stream, wgs);
  }
  return launch_decode_sk_n<KV, QT, D, BS, G, AP, TV, 1>(p, cus, max_wgs, stream, wgs);
}

template <typename KV, typename QT, int D, int BS, bool AP, bool TV>
SkLaunch select_decode_sk_g(int G) {
  switch (G) {
    case 1: return &launch_decode_sk<KV, QT, D, BS, 1, AP, TV>;
    case 2: return &launch_decode_sk<KV, QT, D, BS, 2, AP, TV>;
    case 4: return &launch_decode_sk<KV, QT, D, BS, 4, AP, TV>;
    case 8: return &launch_decode_sk<KV, QT, D, BS, 8, AP, TV>;
    default: return nullptr;
  }
}

template <typename KV, typename QT, int D, bool AP, bool TV>
SkLaunch select_decode_sk_bs(int BS, int G) {
  switch (BS) {
    case 8: return select_decode_sk_g<KV, QT, D, 8, AP, TV>(G);
    case 16: return select_decode_sk_g<KV, QT, D, 16, AP, TV>(G);
    case 32: return select_decode_sk_g<KV, QT, D, 32, AP, TV>(G);
    default: return nullptr;
  }
}

// append = the fused cache write (16-bit pools only); TV = token-major V
template <typename KV, typename QT, bool TV>
SkLaunch select_decode_sk(int D, int BS, int G, bool append) {
  {
    if (append) {
      if constexpr (KV::kBytes != 2) {
        return nullptr;
      } else {
        switch (D) {
          case 64: return select_decode_sk_bs<KV, QT, 64, true, TV>(BS, G);
          case 128: return select_decode_sk_bs<KV, QT, 128, true, TV>(BS, G);
          default: return nullptr;
        }
      }
    }
    switch (D) {
      case 64: return select_decode_sk_bs<KV, QT, 64, false, TV>(BS, G);
      case 128: return select_decode_sk_bs<KV, QT, 128, false, TV>(BS, G);
      default: return nullptr;
    }
  }
}

// ---- the cascade variant (pa_decode_shared)
template <typename KV, typename QT, int D, int BS, int G, bool TV>
hipError_t launch_decode_cas(const SkParams& p, int cus, int max_wgs, hipStream_t stream, int* wgs) {
  if constexpr (TV || KV::kBytes == 1) {
    if (p.stage_bufs > 1) return launch_decode_sk_n<KV, QT, D, BS, G, false, TV, 2, true>(p, cus, max_wgs, stream, wgs);
  }
  return launch_decode_sk_n<KV, QT, D, BS, G, false, TV, 1, true>(p, cus, max_wgs, stream, wgs);
}

// (built on the staged path: token-major V, or fp8 pools)
template <typename KV, typename QT, int D, int BS, bool TV>
SkLaunch select_decode_cas_g(int G) {
  static_assert(TV || KV::kBytes == 1, "the cascade is built on the staged path");
  switch (G) {
    case 1: return &launch_decode_cas<KV, QT, D, BS, 1, TV>;
    case 2: return &launch_decode_cas<KV, QT, D, BS, 2, TV>;
    case 4: return &launch_decode_cas<KV, QT, D, BS, 4, TV>;
    case 8: return &launch_decode_cas<KV, QT, D, BS, 8, TV>;
    default: return nullptr;
  }
}

template <typename KV, typename QT, bool TV>
SkLaunch select_decode_cas(int D, int BS, int G) {
  auto by_bs = [&](auto d) -> SkLaunch {
    constexpr int kD = decltype(d)::value;
    switch (BS) {
      case 8: return select_decode_cas_g<KV, QT, kD, 8, TV>(G);
      case 16: return select_decode_cas_g<KV, QT, kD, 16, TV>(G);
      case 32: return select_decode_cas_g<KV, QT, kD, 32, TV>(G);
      default: return nullptr;
    }
  };
  switch (D) {
    case 64: return by_bs(std::integral_constant<int, 64>{});
    case 128: return by_bs(std::integral_constant<int, 128>{});
    default: return nullptr;
  }
}

}  // namespace pa
