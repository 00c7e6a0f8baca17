// Host block manager: free stack, refcounts, per-sequence block tables,
// fork with copy-on-write, release.
//
// [course] = "PagedAttention", Phase 7 · Document 04 · Production Serving;
// [note] = "PagedAttention" LLM study note (lux-666-github-io.pages.dev).
//
// [course] §2 "The insight": a sequence gets a block only when it needs
// one and returns its blocks when it is done; its table names the physical
// block behind each logical block. [note] block-size section: ceil(L / block_size) blocks
// per sequence. [course] §2 "The bonus" and [note] prefix sharing section:
// forked sequences share blocks under refcounts; a block is copied only when
// a branch writes into it. The choices the pages leave open (LIFO order,
// writer-gets-the-copy, all-or-nothing) are documented in libpagedattn.h.
//
// Swapping ([course] §4 and §8: under memory pressure the scheduler may
// preempt a sequence by swapping its blocks out): a second, host-side pool
// of blocks with its own LIFO free stack (first pop = block 0). Swapping
// out moves every block of a sequence to a fresh host block (a block shared
// with other sequences loses this reference only; the others keep it on the
// device) and frees the device blocks; swapping in does the reverse into
// fresh device blocks. The caller copies the data with
// pa_copy_blocks_between using the reported pairs. A swapped sequence can
// only be swapped in, freed or queried.
//
// Prefix caching ([course] §4: prefix sharing across requests needs an
// identical prefix and prefix caching enabled; §11: enable prefix caching
// for common prompts; §9: RadixAttention extends block sharing into a
// prefix tree): when enabled, every full block a prompt fills through
// pa_alloc_prompt is registered under a 64-bit hash of the whole token
// prefix up to its end (chained block by block) together with its own
// tokens and its parent's hash. A later prompt walks its full blocks and
// reuses registered ones as long as hash, parent and tokens all match. A
// registered block whose refcount drops to 0 keeps its data and joins an
// evictable LRU (a released sequence's blocks join in reverse logical order,
// so a prefix's first blocks are evicted last); allocation takes the free
// stack first and then evicts the least recently released cached block.
//
// Every mutating entry point first plans the whole request against the
// current state (blocks needed, including copy-on-write copies, checked
// against the free count), and only then applies it, so a failure leaves
// the state untouched.
#include <algorithm>
#include <climits>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "internal.h"

struct pa_bm {
  struct Seq {
    int32_t len = 0;
    std::vector<int32_t> blocks;  // logical order; host-pool ids while swapped
    bool swapped = false;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is popped next
  std::vector<int32_t> refcnt;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t cow_copies = 0;
  int64_t forks = 0;
  int32_t num_host_blocks = 0;
  std::vector<int32_t> host_free;  // back() is popped next
  int64_t swap_outs = 0;
  int64_t swap_ins = 0;
  // prefix cache
  bool prefix_cache = false;
  std::unordered_map<uint64_t, int32_t> cached;  // prefix hash -> block
  std::vector<char> registered;                   // per block
  std::vector<uint64_t> block_hash, block_parent;
  std::vector<std::vector<int32_t>> block_tokens;
  std::list<int32_t> lru;  // evictable registered blocks (refcount 0), front = evicted next
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<char> in_lru;
  int64_t cache_hits = 0, cache_misses = 0, evictions = 0;

  int64_t blocks_for(int64_t len) const { return (len + block_size - 1) / block_size; }
  // blocks an allocation can take: free ones, then evictable cached ones
  int64_t available() const { return static_cast<int64_t>(free_stack.size()) + static_cast<int64_t>(lru.size()); }
  void unregister(int32_t b) {
    cached.erase(block_hash[b]);
    registered[b] = 0;
    block_tokens[b].clear();
  }
  void lru_remove(int32_t b) {
    lru.erase(lru_pos[b]);
    in_lru[b] = 0;
  }
  int32_t pop() {
    if (!free_stack.empty()) {
      int32_t b = free_stack.back();
      free_stack.pop_back();
      return b;
    }
    const int32_t b = lru.front();  // callers checked available()
    lru_remove(b);
    unregister(b);
    ++evictions;
    return b;
  }
  // the blocks of `blocks` (logical order) whose refcount just reached 0:
  // unregistered ones onto the free stack in logical order, registered ones
  // into the LRU in reverse logical order
  void release(const std::vector<int32_t>& dead) {
    for (int32_t b : dead)
      if (!registered[b]) free_stack.push_back(b);
    for (auto it = dead.rbegin(); it != dead.rend(); ++it)
      if (registered[*it]) {
        lru_pos[*it] = lru.insert(lru.end(), *it);
        in_lru[*it] = 1;
      }
  }
};

namespace {

using pa::fail;

#define PA_GUARD_BEGIN try {
#define PA_GUARD_END                                                        \
  }                                                                         \
  catch (const std::bad_alloc&) {                                           \
    return fail(PA_ERR_OUT_OF_HOST_MEMORY, "host memory allocation failed"); \
  }

pa_status plan_and_apply(pa_bm* bm, const int64_t* ids, int32_t n, const int32_t* ntok, int64_t* slots,
                         int32_t* cow_pairs, int32_t* num_cow) {
  const int32_t bs = bm->block_size;
  // ---- plan: validate and count blocks (growth + copy-on-write copies)
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  std::unordered_map<int32_t, int32_t> pending;  // shared tail -> copies already planned from it
  // every host allocation of the request happens in this phase, before any
  // state changes: entries of new sequences (moved into the table below
  // without allocating) and room for each table's growth
  std::unordered_map<int64_t, pa_bm::Seq> fresh;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (ntok[i] < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_new_tokens[%d] = %d is negative", i, ntok[i]);
    if (!seen.insert(ids[i]).second)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld appears twice in one batch", (long long)ids[i]);
    auto it = bm->seqs.find(ids[i]);
    if (it != bm->seqs.end() && it->second.swapped)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out", (long long)ids[i]);
    const int64_t len = it == bm->seqs.end() ? 0 : it->second.len;
    if (len + ntok[i] > INT32_MAX)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld would exceed INT32_MAX tokens", (long long)ids[i]);
    need += bm->blocks_for(len + ntok[i]) - bm->blocks_for(len);
    if (it == bm->seqs.end())
      fresh[ids[i]].blocks.reserve(static_cast<size_t>(bm->blocks_for(ntok[i])));
    else
      it->second.blocks.reserve(static_cast<size_t>(bm->blocks_for(len + ntok[i])));
    if (ntok[i] > 0 && len % bs != 0) {
      const int32_t tail = it->second.blocks.back();
      int32_t& already = pending[tail];
      if (bm->refcnt[tail] - already > 1) {
        ++need;
        ++already;
      }
    }
  }
  if (need > bm->available())
    return fail(PA_ERR_OUT_OF_BLOCKS, "request needs %lld blocks, %lld free of %d", (long long)need,
                (long long)bm->available(), bm->num_blocks);
  bm->seqs.reserve(bm->seqs.size() + fresh.size());  // no rehash while applying

  // ---- apply: cannot fail from here on (blocks and host memory reserved above)
  int32_t ncow = 0;
  int64_t out = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto found = bm->seqs.find(ids[i]);
    if (found == bm->seqs.end()) found = bm->seqs.insert(fresh.extract(ids[i])).position;
    pa_bm::Seq& s = found->second;
    const int32_t add = ntok[i];
    if (add > 0 && s.len % bs != 0 && bm->refcnt[s.blocks.back()] > 1) {
      const int32_t old = s.blocks.back();
      const int32_t fresh = bm->pop();
      --bm->refcnt[old];
      bm->refcnt[fresh] = 1;
      s.blocks.back() = fresh;
      cow_pairs[2 * ncow] = old;
      cow_pairs[2 * ncow + 1] = fresh;
      ++ncow;
      ++bm->cow_copies;
    }
    const int64_t want = bm->blocks_for(static_cast<int64_t>(s.len) + add);
    while (static_cast<int64_t>(s.blocks.size()) < want) {
      const int32_t b = bm->pop();
      bm->refcnt[b] = 1;
      s.blocks.push_back(b);
    }
    for (int32_t t = s.len; t < s.len + add; ++t)
      slots[out++] = static_cast<int64_t>(s.blocks[t / bs]) * bs + t % bs;
    s.len += add;
  }
  *num_cow = ncow;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order, pa_bm** out) {
  pa::clear_error();
  if (out == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks = %d must be positive", num_blocks);
  if (block_size <= 0 || block_size > (1 << 20))
    return fail(PA_ERR_INVALID_ARGUMENT, "block_size = %d must be in [1, 2^20]", block_size);
  PA_GUARD_BEGIN
  pa_bm* bm = new pa_bm();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcnt.assign(num_blocks, 0);
  bm->registered.assign(num_blocks, 0);
  bm->block_hash.assign(num_blocks, 0);
  bm->block_parent.assign(num_blocks, 0);
  bm->block_tokens.resize(num_blocks);
  bm->lru_pos.resize(num_blocks);
  bm->in_lru.assign(num_blocks, 0);
  bm->free_stack.resize(num_blocks);
  if (initial_free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return fail(PA_ERR_INVALID_ARGUMENT, "initial_free_order is not a permutation (entry %d = %d)", i, b);
      }
      seen[b] = 1;
    }
  }
  // the stack's top (back) is the first block handed out
  for (int32_t i = 0; i < num_blocks; ++i)
    bm->free_stack[num_blocks - 1 - i] = initial_free_order ? initial_free_order[i] : i;
  *out = bm;
  return PA_OK;
  PA_GUARD_END
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_alloc_batch(pa_bm* bm, const int64_t* seq_ids, int32_t n, const int32_t* num_new_tokens,
                         int64_t* slot_mapping, int32_t* cow_pairs, int32_t* num_cow) {
  pa::clear_error();
  if (bm == nullptr || num_cow == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or num_cow is NULL");
  if (n < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n = %d is negative", n);
  if (n > 0 && (seq_ids == nullptr || num_new_tokens == nullptr || cow_pairs == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "seq_ids, num_new_tokens or cow_pairs is NULL");
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) total += num_new_tokens[i] > 0 ? num_new_tokens[i] : 0;
  if (total > 0 && slot_mapping == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "slot_mapping is NULL");
  PA_GUARD_BEGIN
  return plan_and_apply(bm, seq_ids, n, num_new_tokens, slot_mapping, cow_pairs, num_cow);
  PA_GUARD_END
}

pa_status pa_alloc(pa_bm* bm, int64_t seq_id, int32_t num_new_tokens, int64_t* slot_mapping, int32_t* cow_src,
                   int32_t* cow_dst, int32_t* num_cow) {
  pa::clear_error();
  if (cow_src == nullptr || cow_dst == nullptr || num_cow == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "cow_src, cow_dst or num_cow is NULL");
  int32_t pair[2] = {-1, -1};
  const pa_status st = pa_alloc_batch(bm, &seq_id, 1, &num_new_tokens, slot_mapping, pair, num_cow);
  if (st == PA_OK) {
    *cow_src = pair[0];
    *cow_dst = pair[1];
  }
  return st;
}

pa_status pa_free(pa_bm* bm, int64_t seq_id) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_id);
  PA_GUARD_BEGIN
  if (it->second.swapped) {
    for (int32_t h : it->second.blocks) bm->host_free.push_back(h);
  } else {
    bm->free_stack.reserve(bm->num_blocks);
    std::vector<int32_t> dead;
    for (int32_t b : it->second.blocks)
      if (--bm->refcnt[b] == 0) dead.push_back(b);
    bm->release(dead);
  }
  bm->seqs.erase(it);
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  if (bm->seqs.count(child_id)) return fail(PA_ERR_SEQ_EXISTS, "sequence %lld is already live", (long long)child_id);
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)parent_id);
  if (it->second.swapped)
    return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out", (long long)parent_id);
  PA_GUARD_BEGIN
  pa_bm::Seq copy = it->second;
  for (int32_t b : copy.blocks) ++bm->refcnt[b];
  bm->seqs.emplace(child_id, std::move(copy));
  ++bm->forks;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_seq_info(const pa_bm* bm, int64_t seq_id, int32_t* context_len, int32_t* num_blocks) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_id);
  if (context_len) *context_len = it->second.len;
  if (num_blocks) *num_blocks = static_cast<int32_t>(it->second.blocks.size());
  return PA_OK;
}

pa_status pa_seq_blocks(const pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t capacity, int32_t* n) {
  pa::clear_error();
  if (bm == nullptr || n == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or n is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_id);
  const int32_t len = static_cast<int32_t>(it->second.blocks.size());
  if (capacity < len || (len > 0 && blocks == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "capacity %d < table length %d", capacity, len);
  if (len > 0) std::memcpy(blocks, it->second.blocks.data(), sizeof(int32_t) * len);
  *n = len;
  return PA_OK;
}

pa_status pa_pack_block_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks, int32_t pad,
                               int32_t* tables, int32_t* context_lens) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  if (n < 0 || max_blocks < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n = %d, max_blocks = %d", n, max_blocks);
  if (n > 0 && (seq_ids == nullptr || (tables == nullptr && max_blocks > 0)))
    return fail(PA_ERR_INVALID_ARGUMENT, "seq_ids or tables is NULL");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out", (long long)seq_ids[i]);
    const auto& blocks = it->second.blocks;
    const int32_t len = static_cast<int32_t>(blocks.size());
    if (len > max_blocks)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld holds %d blocks > max_blocks %d", (long long)seq_ids[i],
                  len, max_blocks);
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    if (len > 0) std::memcpy(row, blocks.data(), sizeof(int32_t) * len);
    for (int32_t j = len; j < max_blocks; ++j) row[j] = pad;
    if (context_lens) context_lens[i] = it->second.len;
  }
  return PA_OK;
}

pa_status pa_bm_shared_prefixes(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t granule,
                                int32_t* group_offsets, int32_t* group_members, int32_t* shared_len,
                                int32_t* num_groups, int32_t* max_group_size, int32_t* max_shared_len) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  if (n < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n = %d is negative", n);
  if (granule <= 0 || granule % bm->block_size != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "granule %d must be a positive multiple of block_size %d", granule,
                bm->block_size);
  if (num_groups == nullptr || max_group_size == nullptr || max_shared_len == nullptr || group_offsets == nullptr ||
      (n > 0 && (seq_ids == nullptr || group_members == nullptr || shared_len == nullptr)))
    return fail(PA_ERR_INVALID_ARGUMENT, "an output or seq_ids is NULL");
  PA_GUARD_BEGIN
  std::vector<const pa_bm::Seq*> seqs(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_ids[i]);
    if (it->second.swapped)
      return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out", (long long)seq_ids[i]);
    seqs[i] = &it->second;
  }
  // rows by first physical block, groups in order of first appearance
  std::unordered_map<int32_t, int32_t> group_of;  // first block -> group index
  std::vector<std::vector<int32_t>> rows;
  for (int32_t i = 0; i < n; ++i) {
    shared_len[i] = 0;
    if (seqs[i]->blocks.empty()) continue;
    auto ins = group_of.emplace(seqs[i]->blocks[0], static_cast<int32_t>(rows.size()));
    if (ins.second) rows.emplace_back();
    rows[ins.first->second].push_back(i);
  }
  int32_t ng = 0, used = 0, gmax = 0, smax = 0;
  group_offsets[0] = 0;
  for (const auto& r : rows) {
    if (r.size() < 2) continue;
    const auto& b0 = seqs[r[0]]->blocks;
    size_t lcp = b0.size();
    int32_t min_len = seqs[r[0]]->len;
    for (size_t m = 1; m < r.size(); ++m) {
      const auto& bm_ = seqs[r[m]]->blocks;
      size_t c = 0;
      while (c < lcp && c < bm_.size() && bm_[c] == b0[c]) ++c;
      lcp = c;
      min_len = std::min(min_len, seqs[r[m]]->len);
    }
    // whole granules inside the common blocks, leaving every member a token of its own
    const int64_t limit = std::min<int64_t>(static_cast<int64_t>(lcp) * bm->block_size, min_len - 1);
    const int32_t shared = static_cast<int32_t>(limit > 0 ? limit / granule * granule : 0);
    if (shared == 0) continue;
    for (int32_t row : r) {
      group_members[used++] = row;
      shared_len[row] = shared;
    }
    group_offsets[++ng] = used;
    gmax = std::max<int32_t>(gmax, static_cast<int32_t>(r.size()));
    smax = std::max(smax, shared);
  }
  *num_groups = ng;
  *max_group_size = gmax;
  *max_shared_len = smax;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_bm_set_host_pool(pa_bm* bm, int32_t num_host_blocks) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  if (num_host_blocks < 0) return fail(PA_ERR_INVALID_ARGUMENT, "num_host_blocks = %d is negative", num_host_blocks);
  if (static_cast<int32_t>(bm->host_free.size()) != bm->num_host_blocks)
    return fail(PA_ERR_INVALID_ARGUMENT, "host blocks are in use by swapped sequences");
  PA_GUARD_BEGIN
  std::vector<int32_t> fresh(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) fresh[i] = num_host_blocks - 1 - i;  // first pop = block 0
  bm->host_free.swap(fresh);
  bm->num_host_blocks = num_host_blocks;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_swap_out(pa_bm* bm, int64_t seq_id, int32_t* pairs, int32_t capacity, int32_t* num_pairs) {
  pa::clear_error();
  if (bm == nullptr || num_pairs == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or num_pairs is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_id);
  pa_bm::Seq& sq = it->second;
  if (sq.swapped) return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is already swapped out", (long long)seq_id);
  const int32_t n = static_cast<int32_t>(sq.blocks.size());
  if (n > 0 && (pairs == nullptr || capacity < n))
    return fail(PA_ERR_INVALID_ARGUMENT, "pairs holds %d pairs, %d needed", capacity, n);
  if (n > static_cast<int32_t>(bm->host_free.size()))
    return fail(PA_ERR_OUT_OF_BLOCKS, "swap-out needs %d host blocks, %zu free of %d", n, bm->host_free.size(),
                bm->num_host_blocks);
  PA_GUARD_BEGIN
  bm->free_stack.reserve(bm->num_blocks);
  std::vector<int32_t> dead;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = sq.blocks[i];
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    pairs[2 * i] = b;
    pairs[2 * i + 1] = h;
    sq.blocks[i] = h;
    if (--bm->refcnt[b] == 0) dead.push_back(b);
  }
  bm->release(dead);
  sq.swapped = true;
  ++bm->swap_outs;
  *num_pairs = n;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_swap_in(pa_bm* bm, int64_t seq_id, int32_t* pairs, int32_t capacity, int32_t* num_pairs) {
  pa::clear_error();
  if (bm == nullptr || num_pairs == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or num_pairs is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_id);
  pa_bm::Seq& sq = it->second;
  if (!sq.swapped) return fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is not swapped out", (long long)seq_id);
  const int32_t n = static_cast<int32_t>(sq.blocks.size());
  if (n > 0 && (pairs == nullptr || capacity < n))
    return fail(PA_ERR_INVALID_ARGUMENT, "pairs holds %d pairs, %d needed", capacity, n);
  if (n > bm->available())
    return fail(PA_ERR_OUT_OF_BLOCKS, "swap-in needs %d blocks, %lld free of %d", n, (long long)bm->available(),
                bm->num_blocks);
  PA_GUARD_BEGIN
  bm->host_free.reserve(bm->num_host_blocks);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t h = sq.blocks[i];
    const int32_t b = bm->pop();
    bm->refcnt[b] = 1;
    pairs[2 * i] = h;
    pairs[2 * i + 1] = b;
    sq.blocks[i] = b;
    bm->host_free.push_back(h);
  }
  sq.swapped = false;
  ++bm->swap_ins;
  *num_pairs = n;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_bm_swap_state(const pa_bm* bm, int64_t seq_id, int32_t* swapped) {
  pa::clear_error();
  if (bm == nullptr || swapped == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or swapped is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq_id);
  *swapped = it->second.swapped ? 1 : 0;
  return PA_OK;
}

pa_status pa_bm_host_stats(const pa_bm* bm, int32_t* num_host_blocks, int32_t* num_host_free, int32_t* num_swapped,
                           int64_t* swap_outs, int64_t* swap_ins) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  int32_t ns = 0;
  for (const auto& kv : bm->seqs) ns += kv.second.swapped ? 1 : 0;
  if (num_host_blocks) *num_host_blocks = bm->num_host_blocks;
  if (num_host_free) *num_host_free = static_cast<int32_t>(bm->host_free.size());
  if (num_swapped) *num_swapped = ns;
  if (swap_outs) *swap_outs = bm->swap_outs;
  if (swap_ins) *swap_ins = bm->swap_ins;
  return PA_OK;
}

pa_status pa_bm_host_free_stack(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* n) {
  pa::clear_error();
  if (bm == nullptr || n == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or n is NULL");
  const int32_t k = static_cast<int32_t>(bm->host_free.size());
  if (k > 0 && (out == nullptr || capacity < k))
    return fail(PA_ERR_INVALID_ARGUMENT, "capacity %d < %d host free blocks", capacity, k);
  for (int32_t i = 0; i < k; ++i) out[i] = bm->host_free[i];
  *n = k;
  return PA_OK;
}

namespace {

// 64-bit mix of a token into a running prefix hash (splitmix64 finaliser)
uint64_t mix_token(uint64_t h, int32_t t) {
  uint64_t z = h + 0x9E3779B97F4A7C15ull * (static_cast<uint64_t>(static_cast<uint32_t>(t)) + 1ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

pa_status pa_bm_set_prefix_cache(pa_bm* bm, int32_t enable) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  PA_GUARD_BEGIN
  if (!enable && bm->prefix_cache) {
    // forget every registration; evictable blocks become free (in LRU order)
    for (int32_t b : bm->lru) {
      bm->in_lru[b] = 0;
      bm->free_stack.push_back(b);
    }
    bm->lru.clear();
    for (int32_t b = 0; b < bm->num_blocks; ++b)
      if (bm->registered[b]) bm->unregister(b);
  }
  bm->prefix_cache = enable != 0;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_alloc_prompt(pa_bm* bm, int64_t seq_id, const int32_t* token_ids, int32_t n, int64_t* slot_mapping,
                          int32_t* num_cached) {
  pa::clear_error();
  if (bm == nullptr || num_cached == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or num_cached is NULL");
  if (n < 0) return fail(PA_ERR_INVALID_ARGUMENT, "n = %d is negative", n);
  if (n > 0 && (token_ids == nullptr || slot_mapping == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "token_ids or slot_mapping is NULL");
  if (bm->seqs.count(seq_id)) return fail(PA_ERR_SEQ_EXISTS, "sequence %lld is already live", (long long)seq_id);
  const int32_t bs = bm->block_size;
  const int32_t nfull = n / bs;
  PA_GUARD_BEGIN
  // ---- plan: the longest run of registered leading blocks, then capacity
  std::vector<uint64_t> key(nfull);
  uint64_t h = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    for (int32_t t = i * bs; t < (i + 1) * bs; ++t) h = mix_token(h, token_ids[t]);
    key[i] = h;
  }
  std::vector<int32_t> hit;
  int64_t hits_in_lru = 0;
  if (bm->prefix_cache) {
    uint64_t parent = 0;
    for (int32_t i = 0; i < nfull; ++i) {
      auto f = bm->cached.find(key[i]);
      if (f == bm->cached.end()) break;
      const int32_t b = f->second;
      if (bm->block_parent[b] != parent ||
          !std::equal(bm->block_tokens[b].begin(), bm->block_tokens[b].end(), token_ids + static_cast<int64_t>(i) * bs))
        break;
      hit.push_back(b);
      hits_in_lru += bm->in_lru[b];
      parent = key[i];
    }
  }
  const int32_t nhit = static_cast<int32_t>(hit.size());
  const int64_t need = bm->blocks_for(n) - nhit;
  if (need > bm->available() - hits_in_lru)
    return fail(PA_ERR_OUT_OF_BLOCKS, "prompt needs %lld new blocks, %lld free of %d", (long long)need,
                (long long)(bm->available() - hits_in_lru), bm->num_blocks);
  // ---- apply
  pa_bm::Seq sq;
  sq.len = n;
  sq.blocks.reserve(static_cast<size_t>(bm->blocks_for(n)));
  for (int32_t b : hit) {
    if (bm->in_lru[b]) bm->lru_remove(b);
    ++bm->refcnt[b];
    sq.blocks.push_back(b);
  }
  for (int64_t i = nhit; i < bm->blocks_for(n); ++i) {
    const int32_t b = bm->pop();
    bm->refcnt[b] = 1;
    sq.blocks.push_back(b);
    if (bm->prefix_cache && i < nfull && !bm->cached.count(key[i])) {
      bm->cached.emplace(key[i], b);
      bm->registered[b] = 1;
      bm->block_hash[b] = key[i];
      bm->block_parent[b] = i > 0 ? key[i - 1] : 0;
      bm->block_tokens[b].assign(token_ids + i * bs, token_ids + (i + 1) * bs);
    }
  }
  for (int32_t t = 0; t < n; ++t) slot_mapping[t] = static_cast<int64_t>(sq.blocks[t / bs]) * bs + t % bs;
  bm->seqs.emplace(seq_id, std::move(sq));
  if (bm->prefix_cache) {
    bm->cache_hits += nhit;
    bm->cache_misses += nfull - nhit;
  }
  *num_cached = nhit * bs;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_bm_prefix_cache_stats(const pa_bm* bm, int32_t* num_cached_blocks, int32_t* num_evictable,
                                   int64_t* hits, int64_t* misses, int64_t* evictions) {
  pa::clear_error();
  if (bm == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm is NULL");
  if (num_cached_blocks) *num_cached_blocks = static_cast<int32_t>(bm->cached.size());
  if (num_evictable) *num_evictable = static_cast<int32_t>(bm->lru.size());
  if (hits) *hits = bm->cache_hits;
  if (misses) *misses = bm->cache_misses;
  if (evictions) *evictions = bm->evictions;
  return PA_OK;
}

pa_status pa_bm_evictable(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* n) {
  pa::clear_error();
  if (bm == nullptr || n == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or n is NULL");
  const int32_t k = static_cast<int32_t>(bm->lru.size());
  if (k > 0 && (out == nullptr || capacity < k))
    return fail(PA_ERR_INVALID_ARGUMENT, "capacity %d < %d evictable blocks", capacity, k);
  int32_t i = 0;
  for (int32_t b : bm->lru) out[i++] = b;
  *n = k;
  return PA_OK;
}

pa_status pa_bm_usage_get(const pa_bm* bm, int32_t max_context_len, pa_bm_usage* out) {
  pa::clear_error();
  if (bm == nullptr || out == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or out is NULL");
  if (max_context_len <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "max_context_len = %d must be positive", max_context_len);
  PA_GUARD_BEGIN
  const int32_t bs = bm->block_size;
  std::vector<int32_t> fill(bm->num_blocks, 0);  // slots of each block some resident sequence fills
  pa_bm_usage u{};
  int64_t resident = 0;
  for (const auto& kv : bm->seqs) {
    const pa_bm::Seq& sq = kv.second;
    if (sq.swapped) continue;
    ++resident;
    u.tokens += sq.len;
    for (size_t j = 0; j < sq.blocks.size(); ++j) {
      const int64_t f = std::min<int64_t>(bs, static_cast<int64_t>(sq.len) - static_cast<int64_t>(j) * bs);
      fill[sq.blocks[j]] = std::max<int32_t>(fill[sq.blocks[j]], static_cast<int32_t>(f));
    }
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b)
    if (bm->refcnt[b] > 0) {
      ++u.used_blocks;
      u.filled_slots += fill[b];
    }
  u.used_slots = static_cast<int64_t>(u.used_blocks) * bs;
  u.naive_slots = resident * max_context_len;
  u.capacity = static_cast<int32_t>(bm->num_blocks / bm->blocks_for(max_context_len));
  u.usage = static_cast<double>(u.used_blocks) / bm->num_blocks;
  u.paged_waste = u.used_slots ? 1.0 - static_cast<double>(u.filled_slots) / u.used_slots : 0.0;
  u.naive_waste = u.naive_slots ? 1.0 - static_cast<double>(u.tokens) / u.naive_slots : 0.0;
  *out = u;
  return PA_OK;
  PA_GUARD_END
}

pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out) {
  pa::clear_error();
  if (bm == nullptr || out == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or out is NULL");
  pa_bm_stats_t s{};
  s.num_blocks = bm->num_blocks;
  s.num_free = static_cast<int32_t>(bm->free_stack.size());
  for (int32_t r : bm->refcnt) {
    s.num_used += r > 0;
    s.num_shared += r > 1;
  }
  s.num_seqs = static_cast<int32_t>(bm->seqs.size());
  s.cow_copies = bm->cow_copies;
  s.forks = bm->forks;
  *out = s;
  return PA_OK;
}

pa_status pa_bm_refcounts(const pa_bm* bm, int32_t* out) {
  pa::clear_error();
  if (bm == nullptr || out == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or out is NULL");
  std::memcpy(out, bm->refcnt.data(), sizeof(int32_t) * bm->num_blocks);
  return PA_OK;
}

pa_status pa_bm_free_stack(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* n) {
  pa::clear_error();
  if (bm == nullptr || n == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "bm or n is NULL");
  const int32_t len = static_cast<int32_t>(bm->free_stack.size());
  if (capacity < len || (len > 0 && out == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "capacity %d < free count %d", capacity, len);
  if (len > 0) std::memcpy(out, bm->free_stack.data(), sizeof(int32_t) * len);
  *n = len;
  return PA_OK;
}

}  // extern "C"
