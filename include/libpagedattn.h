/*
 * libpagedattn — paged KV cache and PagedAttention decode for AMD MI355X (gfx950).
 *
 * A plain C ABI: host pointers, device pointers and sizes only. Device
 * memory is always owned by the caller; the library never allocates device
 * memory. Host block-manager state is owned by the library behind an opaque
 * handle.
 *
 * Pages cited (by title and section):
 *   [course] "PagedAttention" — Phase 7 · Document 04 · Production Serving
 *            (ai-engineer-zt0.pages.dev, llm-mastery/07-production-serving)
 *   [note]   "PagedAttention" — LLM study note in Chinese
 *            (lux-666-github-io.pages.dev)
 *   [intent] "Building Intent-Aware Configuration for LLM Serving"
 *            (marcusacosta.dev)
 *
 * Error convention ([intent] "Enforcing policy at the device boundary",
 * "Extending the Rust SDK contract"): an explicit request either does what
 * it asks or returns a specific status with a message from pa_last_error();
 * nothing silently falls back to another path. Unsupported shapes or dtypes
 * return PA_ERR_UNSUPPORTED, never a slower substitute. Every status-
 * returning call validates its arguments before it touches any state or
 * launches any kernel; on an error return no state has changed.
 *
 * Threading: a pa_bm handle is not thread-safe (the caller serialises
 * calls on one handle). Device calls are thread-safe and asynchronous on
 * the caller's stream (a hipStream_t passed as void*; NULL = the default
 * stream). They never synchronise the host unless the environment
 * variable PA_DEBUG=1 is set, in which case device-side inputs are copied
 * back and validated before launch (slow; for debugging only).
 * PA_SK_WGS=n caps the grid of the balanced decode split at n workgroups
 * (for tests of the split itself; the result is the same up to rounding).
 * PA_PARTITION_PATH=staged|wave picks, for partitioned pa_decode calls
 * where both exist, the staged kernel or the one-wave partition kernels
 * (normally chosen from the batch shape; for tests and measurements).
 * PA_SK_STAGES=1 keeps the staged kernel at one LDS stage where it would
 * take two (for measurements; same result).
 */
#ifndef LIBPAGEDATTN_H
#define LIBPAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 6

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad shape, misaligned pointer */
  PA_ERR_OUT_OF_BLOCKS = 2,    /* the pool cannot hold the request; nothing changed */
  PA_ERR_UNKNOWN_SEQ = 3,      /* the sequence id is not live */
  PA_ERR_SEQ_EXISTS = 4,       /* fork target already live */
  PA_ERR_UNSUPPORTED = 5,      /* dtype / head_dim / block_size / group combination not built */
  PA_ERR_DEVICE = 6,           /* a HIP call failed (launch error, bad stream) */
  PA_ERR_OUT_OF_HOST_MEMORY = 7, /* a host allocation of the block manager failed: pa_alloc and
                                    pa_alloc_batch changed nothing; after another call the manager
                                    may be partly updated and should be destroyed */
} pa_status;

typedef enum pa_dtype {
  PA_F16 = 0,      /* IEEE binary16 */
  PA_BF16 = 1,     /* bfloat16 */
  PA_F32 = 2,      /* IEEE binary32 */
  PA_FP8_E4M3 = 3, /* OCP FP8 E4M3 (e4m3fn: bias 7, max 448, no inf), per-tensor scale */
} pa_dtype;

/* Static string for a status code. */
const char* pa_status_string(pa_status status);
/* Detail of the last error on the calling thread ("" if none). Valid until
 * the next library call on this thread. */
const char* pa_last_error(void);
/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

/* ------------------------------------------------------------------------
 * Host block manager.
 *
 * [course] §2 "The insight": the KV cache lives in a pool of physical
 * blocks of one size; a sequence takes a block only when its tokens need
 * one and returns all of them when it is done; its block table names the
 * physical block behind each logical block. [note] 最小模型: growth takes one
 * more block, release returns the sequence's own blocks; [note] block-size
 * section: a sequence of L tokens holds ceil(L / block_size) blocks.
 * [course] §2 "The bonus: block sharing (copy-on-write)" and [note] prefix
 * sharing section: forked sequences share physical blocks under reference
 * counts, and a block is copied only when a branch writes into it.
 *
 * Choices the pages leave open, fixed here:
 *  - Free blocks form a LIFO stack. A fresh manager pops
 *    initial_free_order[0] first (NULL = 0, 1, 2, ...). pa_free pushes a
 *    sequence's blocks in logical order as their refcount reaches zero.
 *  - Copy-on-write: when a sequence appends to a partially filled last
 *    block whose refcount is > 1, the writer receives a fresh block (popped
 *    before any growth blocks) and a (src, dst) pair is reported; the
 *    caller must run pa_copy_blocks on those pairs before
 *    pa_reshape_and_cache writes into dst (same stream order suffices).
 *  - Allocation is all-or-nothing: PA_ERR_OUT_OF_BLOCKS leaves every
 *    table, refcount and the free stack unchanged; the caller queues,
 *    rejects or preempts ([course] §11 "at the limit: queue/reject").
 *  - A slot is phys_block * block_size + offset_in_block (int64).
 * ---------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

/* Counters of a manager ([note] section "prefix sharing 的边界": production
 * monitoring should track how many blocks are shared and how many
 * copy-on-write copies happen; [course] §4: pool occupancy is the capacity
 * signal). num_seqs (live sequences) is one field more than the counters
 * those passages name; `reserved` keeps the 64-bit fields aligned. */
typedef struct pa_bm_stats_s {
  int32_t num_blocks; /* pool size */
  int32_t num_free;   /* blocks on the free stack */
  int32_t num_used;   /* blocks with refcount > 0 */
  int32_t num_shared; /* blocks with refcount > 1 */
  int32_t num_seqs;   /* live sequences */
  int32_t reserved;
  int64_t cow_copies; /* copy-on-write pairs reported so far */
  int64_t forks;      /* successful pa_fork calls */
} pa_bm_stats_t;

/* Create a manager for a pool of num_blocks blocks of block_size tokens.
 * initial_free_order: host int32[num_blocks], a permutation of
 * 0..num_blocks-1 (copied), or NULL. *out receives the handle. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                       pa_bm** out);
/* Destroy a manager (NULL is a no-op). */
void pa_bm_destroy(pa_bm* bm);

/* Make room for num_new_tokens (>= 0) more tokens of seq_id, creating the
 * sequence if it is not live. slot_mapping: host int64[num_new_tokens]
 * receives the slots of the new tokens in token order (may be NULL when
 * num_new_tokens == 0). If the write needs a copy-on-write, *num_cow = 1
 * and (*cow_src, *cow_dst) is the pair; otherwise *num_cow = 0. */
pa_status pa_alloc(pa_bm* bm, int64_t seq_id, int32_t num_new_tokens, int64_t* slot_mapping,
                   int32_t* cow_src, int32_t* cow_dst, int32_t* num_cow);

/* pa_alloc for n distinct sequences at once, applied in array order and
 * all-or-nothing as a whole. seq_ids: host int64[n]; num_new_tokens: host
 * int32[n]; slot_mapping: host int64[sum(num_new_tokens)] receives each
 * sequence's new slots, concatenated in array order; cow_pairs: host
 * int32[n][2] receives (src, dst) pairs; *num_cow receives their count.
 * A sequence id may appear only once (PA_ERR_INVALID_ARGUMENT). */
pa_status pa_alloc_batch(pa_bm* bm, const int64_t* seq_ids, int32_t n, const int32_t* num_new_tokens,
                         int64_t* slot_mapping, int32_t* cow_pairs, int32_t* num_cow);

/* Release seq_id: every block loses one reference ([note] 最小模型, release). */
pa_status pa_free(pa_bm* bm, int64_t seq_id);

/* child_id becomes a live sequence sharing every block of parent_id
 * (refcount + 1 each); [course] §2 "The bonus", parallel sampling / beam. */
pa_status pa_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);

/* Context length and block count of a live sequence (either may be NULL). */
pa_status pa_seq_info(const pa_bm* bm, int64_t seq_id, int32_t* context_len, int32_t* num_blocks);

/* Copy a live sequence's block table (logical order) into host
 * int32[capacity]; *n receives its length. capacity < length ->
 * PA_ERR_INVALID_ARGUMENT. */
pa_status pa_seq_blocks(const pa_bm* bm, int64_t seq_id, int32_t* blocks, int32_t capacity, int32_t* n);

/* Pack the tables of n live sequences into host int32[n][max_blocks]
 * (row i = seq_ids[i], padded with `pad`) and their lengths into host
 * int32[n]. A table longer than max_blocks -> PA_ERR_INVALID_ARGUMENT
 * (outputs unspecified). context_lens may be NULL. */
pa_status pa_pack_block_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                               int32_t pad, int32_t* tables, int32_t* context_lens);

/* ------------------------------------------------------------------------
 * Swapping ([course] §4 and §8: under memory pressure the scheduler may
 * preempt a sequence by evicting and recomputing it or by swapping its
 * blocks out; a preemption is a latency event worth counting). The manager
 * keeps a second pool of host blocks with its own LIFO free stack (first
 * pop = host block 0). The data move is the caller's: pa_copy_blocks_between
 * with the reported pairs, between the device pool and a host pool of the
 * same geometry (pinned host memory the device can address), on the stream
 * of the decode work, before any later write to the freed blocks.
 * ---------------------------------------------------------------------- */

/* Size the host pool (num_host_blocks >= 0; 0 = no swapping). Only while no
 * sequence is swapped out (else PA_ERR_INVALID_ARGUMENT); resets its free
 * stack. */
pa_status pa_bm_set_host_pool(pa_bm* bm, int32_t num_host_blocks);

/* Swap out live sequence seq_id: each block of its table, in logical order,
 * moves to a freshly popped host block; pairs[i] = (device block, host
 * block) (host int32[capacity][2], capacity >= table length); the device
 * block loses this sequence's reference (and returns to the free stack at
 * 0; a block shared with other sequences stays theirs). Afterwards the
 * sequence is swapped: pa_alloc / pa_fork / pa_pack_block_tables /
 * pa_bm_shared_prefixes on it fail with PA_ERR_INVALID_ARGUMENT,
 * pa_seq_blocks reports host block ids, pa_free returns them to the host
 * pool. All-or-nothing: PA_ERR_OUT_OF_BLOCKS when the host pool lacks
 * blocks; PA_ERR_UNKNOWN_SEQ; PA_ERR_INVALID_ARGUMENT (already swapped,
 * capacity). *num_pairs = table length. */
pa_status pa_swap_out(pa_bm* bm, int64_t seq_id, int32_t* pairs, int32_t capacity, int32_t* num_pairs);

/* Swap a swapped sequence back in: each host block, in logical order, moves
 * to a freshly popped device block (refcount 1); pairs[i] = (host block,
 * device block); the host blocks return to the host free stack in logical
 * order. All-or-nothing: PA_ERR_OUT_OF_BLOCKS when the device pool lacks
 * blocks; PA_ERR_INVALID_ARGUMENT (not swapped, capacity). */
pa_status pa_swap_in(pa_bm* bm, int64_t seq_id, int32_t* pairs, int32_t capacity, int32_t* num_pairs);

/* *swapped = 1 if the live sequence is swapped out, else 0. */
pa_status pa_bm_swap_state(const pa_bm* bm, int64_t seq_id, int32_t* swapped);

/* Host pool size, free host blocks, swapped sequences, and the numbers of
 * swap-outs and swap-ins so far (any output may be NULL). */
pa_status pa_bm_host_stats(const pa_bm* bm, int32_t* num_host_blocks, int32_t* num_host_free, int32_t* num_swapped,
                           int64_t* swap_outs, int64_t* swap_ins);

/* Host free stack from bottom to top (the top is popped next): host
 * int32[capacity]; *n receives the count. */
pa_status pa_bm_host_free_stack(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* n);

/* ------------------------------------------------------------------------
 * Prefix caching across requests ([course] §4: sharing across users needs
 * an identical prefix and prefix caching enabled; §11: enable prefix
 * caching for common prompts; §9: RadixAttention extends block sharing into
 * a prefix tree).
 *
 * With the cache on, every full block a prompt fills through
 * pa_alloc_prompt is registered under a 64-bit hash of the token prefix up
 * to the block's end (the hash chains block by block), with its own tokens
 * and its parent's hash. A registered block whose refcount drops to 0 keeps
 * its K/V and becomes evictable (an LRU; a released sequence's registered
 * blocks enter it in reverse logical order, so the first blocks of a
 * prefix go last). Every allocation (pa_alloc, pa_alloc_prompt, copy-on-
 * write, pa_swap_in) takes the free stack first, then evicts the least
 * recently released cached block (unregistering it). Blocks filled by
 * decode growth are not registered (their tokens are unknown here).
 * ---------------------------------------------------------------------- */

/* Turn the prefix cache on or off (off by default). Turning it off forgets
 * every registration; evictable blocks go onto the free stack in LRU
 * order. */
pa_status pa_bm_set_prefix_cache(pa_bm* bm, int32_t enable);

/* Create sequence seq_id for a prompt of n tokens (token_ids: host
 * int32[n]). Its leading full blocks are reused from the cache while hash,
 * parent hash and tokens all match (refcount + 1, taken out of the LRU);
 * the rest are allocated, and its new full blocks registered (a hash
 * already registered keeps its block). slot_mapping: host int64[n], the
 * slot of every token; *num_cached = tokens covered by reused blocks — the
 * caller writes K/V only for tokens num_cached .. n - 1. All-or-nothing:
 * PA_ERR_OUT_OF_BLOCKS (free + evictable blocks, not counting reused ones,
 * are too few), PA_ERR_SEQ_EXISTS, PA_ERR_INVALID_ARGUMENT. With the cache
 * off it is pa_alloc of a new sequence and *num_cached = 0. A 64-bit hash
 * collision between different prefixes (probability ~2^-64 per lookup)
 * would share a wrong block; the block's own tokens and its parent hash are
 * compared exactly. */
pa_status pa_alloc_prompt(pa_bm* bm, int64_t seq_id, const int32_t* token_ids, int32_t n, int64_t* slot_mapping,
                          int32_t* num_cached);

/* Registered blocks, evictable ones, and the numbers of full prompt blocks
 * found / not found in the cache and of evictions so far (any output may
 * be NULL). */
pa_status pa_bm_prefix_cache_stats(const pa_bm* bm, int32_t* num_cached_blocks, int32_t* num_evictable,
                                   int64_t* hits, int64_t* misses, int64_t* evictions);

/* Evictable blocks, the next to be evicted first: host int32[capacity];
 * *n receives the count. */
pa_status pa_bm_evictable(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* n);

/* Groups of the batch rows seq_ids[0..n) whose block tables begin with the
 * same physical blocks — forks of one prompt ([course] §2 "The bonus":
 * parallel samples share the prompt's blocks; [note] prefix-sharing
 * section) — for pa_decode_shared. Rows are grouped by their first block;
 * a group's shared length is the longest run of leading table entries that
 * all members hold, in whole `granule`-token units (granule = the decode's
 * partition size, a positive multiple of block_size), and below every
 * member's length, so each member keeps at least one token of its own.
 * Groups of one row or with a shared length of 0 are left out; their rows
 * get shared_len 0. Outputs (host, caller-owned): group_offsets[groups + 1]
 * (capacity n / 2 + 1 suffices), group_members (batch rows, grouped;
 * capacity n), shared_len[n] (tokens, per row), *num_groups,
 * *max_group_size, *max_shared_len. Errors: PA_ERR_UNKNOWN_SEQ,
 * PA_ERR_INVALID_ARGUMENT. */
pa_status pa_bm_shared_prefixes(const pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t granule,
                                int32_t* group_offsets, int32_t* group_members, int32_t* shared_len,
                                int32_t* num_groups, int32_t* max_group_size, int32_t* max_shared_len);

/* The manager's counters (pa_bm_stats_t above) into *out (host).
 * Errors: PA_ERR_INVALID_ARGUMENT (NULL bm or out). */
pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out);

/* KV memory use of the resident sequences, and the two baselines the pages
 * compare ([course] §2 primer and "The insight": a contiguous max-context
 * reservation per request wastes most of it, paging wastes at most the
 * tail of each sequence's last block; §4 and §11: the pool still caps
 * concurrency, seqs ~ pool blocks / blocks per sequence; the KV usage
 * fraction is the capacity signal to watch). */
typedef struct pa_bm_usage {
  int64_t tokens;         /* sum of the resident sequences' lengths (shared tokens counted per sequence) */
  int64_t used_slots;     /* block_size x blocks with refcount > 0 */
  int64_t filled_slots;   /* slots of those blocks some resident sequence fills */
  int64_t naive_slots;    /* resident sequences x max_context_len (a contiguous reservation each) */
  int32_t used_blocks;    /* blocks with refcount > 0 */
  int32_t capacity;       /* sequences of max_context_len tokens the whole pool holds: num_blocks / ceil(max_context_len / block_size) */
  double usage;           /* used_blocks / num_blocks */
  double paged_waste;     /* 1 - filled_slots / used_slots (0 when no block is used) */
  double naive_waste;     /* 1 - tokens / naive_slots (0 when no sequence is resident) */
} pa_bm_usage;

/* Fill *out for a reservation size of max_context_len tokens (> 0). Swapped
 * sequences are not resident. Errors: PA_ERR_INVALID_ARGUMENT. */
pa_status pa_bm_usage_get(const pa_bm* bm, int32_t max_context_len, pa_bm_usage* out);
/* Refcount of every block: host int32[num_blocks]. */
pa_status pa_bm_refcounts(const pa_bm* bm, int32_t* out);
/* Free stack from bottom to top (the top is popped next): host
 * int32[capacity]; *n receives the count. */
pa_status pa_bm_free_stack(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* n);

/* ------------------------------------------------------------------------
 * Device KV pool descriptor (caller-owned device memory).
 *
 * [course] §2 "The insight": each physical block holds BLOCK tokens of K
 * and V laid out K[BLOCK][HEADS][HEAD_DIM], V[BLOCK][HEADS][HEAD_DIM].
 * K always uses that token-major layout: element (blk, t, h, d) of K is at
 *   k[blk * block_stride + (t * num_kv_heads + h) * head_dim + d].
 * V uses the layout named by v_layout:
 *   PA_LAYOUT_TOKEN_MAJOR (the page's V[BLOCK][HEADS][HEAD_DIM]):
 *     v[blk * block_stride + (t * num_kv_heads + h) * head_dim + d]
 *   PA_LAYOUT_DIM_MAJOR (V[HEADS][HEAD_DIM][BLOCK], the tokens of one head
 *     dimension contiguous; the V-cache layout vLLM uses for the same reason):
 *     v[blk * block_stride + (h * head_dim + d) * block_size + t]
 * The softmax-weighted sum contracts over tokens, so the matrix cores want
 * the tokens of one head dimension together: the dim-major layout stores
 * them so; with the token-major layout the kernels load V rows like K rows
 * and transpose each V tile through LDS ([note] block-size
 * section: the best block granularity depends on the attention kernel's
 * vectorisation). Both layouts are supported explicitly; neither falls
 * back to the other.
 * block_stride (elements) >= block_size * num_kv_heads * head_dim; separate
 * K and V pools use exactly that, the page's interleaved KVBlock uses twice
 * that with v = k + block_size * num_kv_heads * head_dim.
 * Requirements: k and v 16-byte aligned; head_dim a multiple of 16;
 * block_stride * element size a multiple of 16 bytes.
 * fp8 pools store E4M3 codes of value / scale with one fp32 scale per
 * tensor (k_scale, v_scale > 0); 16-bit pools ignore the scales.
 * ---------------------------------------------------------------------- */
typedef enum pa_layout {
  PA_LAYOUT_TOKEN_MAJOR = 0, /* [block][heads][head_dim] */
  PA_LAYOUT_DIM_MAJOR = 1,   /* [heads][head_dim][block] (V only) */
} pa_layout;

typedef struct pa_kv_cache {
  void* k;
  void* v;
  int64_t block_stride;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pa_dtype dtype;     /* PA_F16, PA_BF16 or PA_FP8_E4M3 */
  pa_layout v_layout; /* in-block layout of V */
  float k_scale;
  float v_scale;
} pa_kv_cache;

/* Write the K/V rows of T new tokens into their slots ([course] §2 primer:
 * each decode step adds one token's K/V; [course] §2 "The insight").
 * k_new, v_new: device [T][num_kv_heads][head_dim], contiguous, 16-byte
 * aligned, of src_dtype. slot_mapping: device int64[T]; token i goes to
 * block slot/block_size, row slot%block_size; a negative slot skips the
 * token; a slot >= num_blocks*block_size is skipped as well (PA_DEBUG=1
 * reports it as PA_ERR_INVALID_ARGUMENT). 16-bit pools take sources of
 * the same dtype and store the bits unchanged. fp8 pools take F16, BF16 or
 * F32 sources and store encode(float32(x) * (1.0f / scale)): round to
 * nearest even, saturating to +-448, NaN kept. Slots must be distinct
 * (two tokens writing one slot race). */
pa_status pa_reshape_and_cache(const pa_kv_cache* cache, const void* k_new, const void* v_new,
                               pa_dtype src_dtype, const int64_t* slot_mapping, int32_t T, void* stream);

/* Copy whole blocks, K and V: block pairs[i][1] := block pairs[i][0]
 * ([course] §2 "The bonus": only the differing block is copied; [note]
 * prefix sharing section: copy-on-write when a branch writes). pairs:
 * device int32[N][2] (src, dst). Pairs run concurrently: every dst must be
 * distinct and no dst may be a src of the same call. Pairs with an id
 * outside [0, num_blocks) are skipped (PA_DEBUG=1 reports them). N == 0 is
 * a no-op. */
pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* pairs, int32_t N, void* stream);

/* Whole-block copies between two pools of the same geometry (block_size,
 * num_kv_heads, head_dim, dtype, v_layout; block strides may differ):
 * dst block pairs[i][1] <- src block pairs[i][0], K and V, for i < N. Used
 * to swap blocks between the device pool and a host pool (pinned host
 * memory the device can address). pairs: device (or device-addressable)
 * int32[N][2]; destinations must be distinct and no destination may be a
 * source of the same call when the pools are the same memory. Pairs with an
 * id outside its pool are skipped (PA_DEBUG=1 reports them). Errors:
 * PA_ERR_INVALID_ARGUMENT (descriptors, geometry mismatch, N < 0, NULL
 * pairs with N > 0), PA_ERR_DEVICE. Asynchronous on `stream`. */
pa_status pa_copy_blocks_between(const pa_kv_cache* dst, const pa_kv_cache* src, const int32_t* pairs, int32_t N,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Decode attention through the block tables ([course] §2 "The insight":
 * keys and values are looked up through the table as attention runs;
 * [note] 最小模型: physical blocks are read in logical token order; [note]
 * "why it works": the result is ordinary attention).
 *
 * For each sequence s < B with L = context_lens[s] and each query head h
 * (KV head g = h / (Hq / num_kv_heads)):
 *   z_t = scale * q[s][h] . K_t[g]          for t in [0, L)
 *   out[s][h] = sum_t softmax(z)_t * V_t[g]  (zeros when L == 0)
 * where token t of s is row t % block_size of physical block
 * block_tables[s][t / block_size]. fp8 pools use K = code value * k_scale
 * and V = code value * v_scale.
 *
 * q: device [B][Hq][head_dim] of q_dtype (F16 or BF16; for F16/BF16 pools
 * it must equal the pool dtype). out: device [B][Hq][head_dim] of
 * out_dtype (F16, BF16 or F32). block_tables: device int32[B][max_blocks];
 * entries past ceil(L / block_size) are never read. context_lens: device
 * int32[B]. max_context_len: an upper bound on every context_lens[s]
 * (sizes the launch); it must be <= max_blocks * block_size. A sequence
 * whose length exceeds it is processed only up to it (PA_DEBUG=1 reports
 * it). Table entries outside [0, num_blocks) are read as block 0 (no
 * out-of-bounds access; PA_DEBUG=1 reports them).
 *
 * partition_size: how the work is divided over workgroups (the result is
 * the same up to fp32 rounding order):
 *   0      one workgroup per (sequence, KV head) walks the whole context;
 *   > 0    (a multiple of 16) each context is cut into partitions of that
 *          many tokens, one workgroup each, merged by a log-sum-exp
 *          reduction (a workgroup per partition and KV head, or, for
 *          batches of few long sequences with token-major V or fp8 pools,
 *          per partition and group of up to 4 KV heads; either way a
 *          row's result does not depend on the rest of the batch);
 *   PA_PARTITION_BALANCED  the batch's tiles (16 tokens; 32 for fp8 pools)
 *          of all sequences and KV heads are divided evenly over the
 *          workgroups the device holds at once, each walking its share
 *          across sequence boundaries;
 *          sequences cut between workgroups are merged as above. Either V
 *          layout, every pool dtype. A workgroup serves HW KV heads (the largest
 *          divisor of num_kv_heads up to 8; with token-major V or an fp8
 *          pool the largest such power of two) and keeps B + 1 ints and HW
 *          per-wave regions of G * head_dim floats in LDS; with token-major
 *          V also the unit's K and V rows (2 x 16 rows of HW * head_dim
 *          16-bit elements, padded by 16 and 32 bytes), with an fp8 pool
 *          the unit's 32 K rows (padded) and its V (about 64 * HW *
 *          head_dim bytes in all; token-major V widened to bf16, about 96
 *          * HW * head_dim). The LDS bounds B: 64 KiB for 16-bit
 *          pools with dim-major V (B <= 12287 for 8 KV heads, G = 4,
 *          head_dim 128), otherwise the device's LDS per workgroup (at
 *          most 160 KiB; token-major V: B <= 20287 for the same shapes on
 *          a 160 KiB device); beyond it PA_ERR_UNSUPPORTED. The grid
 *          depends on the current device's CU count, so size the workspace
 *          on the device that runs the call.
 * Splits need a workspace of pa_decode_workspace_size(...) bytes (device,
 * 256-byte aligned, contents need no initialisation); 0 bytes otherwise
 * (workspace may be NULL).
 *
 * Supported (else PA_ERR_UNSUPPORTED): head_dim 64 or 128; block_size 8,
 * 16 or 32; Hq / num_kv_heads in {1, 2, 4, 8}; pool F16 with q F16, pool
 * BF16 with q BF16, pool FP8_E4M3 with q BF16.
 * ---------------------------------------------------------------------- */
#define PA_PARTITION_BALANCED (-1)

/* Workspace bytes pa_decode needs for these sizes and partition_size (0
 * when no workspace is needed or the sizes are invalid). For
 * PA_PARTITION_BALANCED it reads the current device's CU count.
 * num_kv_heads is needed because the sizes depend on the grouping: the
 * balanced split keeps G = num_q_heads / num_kv_heads rows per wave and
 * per piece, and both splits keep num_kv_heads x B merge descriptors; a
 * size taken without it would have to assume G = num_q_heads. */
size_t pa_decode_workspace_size(int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size);

/* Workspace bytes pa_decode_shared needs (0 when partition_size <= 0 or the
 * sizes are invalid): at least pa_decode_workspace_size(...), and what its
 * cascade needs for any grouping of the B rows on the current device (per
 * row the two partial states, per CU the partial pieces of one workgroup
 * of up to 8 KV heads x 32 query rows). A deviation from the proposed
 * boundary, which has no shared-prefix call. */
size_t pa_decode_shared_workspace_size(int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size);

pa_status pa_decode(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                    int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, result and errors as pa_decode, without the workspace:
 * the partial results of a split go to a scratch array the library holds on
 * every GPU it runs on (64 MiB each, kept until the process ends; its
 * address is looked up once per device, on the first call there). Nothing
 * is allocated: no hipMalloc / hipFree, no library allocation.
 *
 * Limits: PA_PARTITION_BALANCED sizes its partial results for the
 * workgroups it launches (far below 64 MiB for every supported shape on
 * MI355X); a partitioned call (partition_size >= 0) whose
 * pa_decode_workspace_size exceeds 64 MiB returns PA_ERR_INVALID_ARGUMENT
 * before any launch. No scratch content carries over between calls: every
 * location a call reads it wrote itself earlier in the same call.
 *
 * Calls that overlap on one GPU (two streams, or two host threads without
 * ordering between their streams) share that GPU's scratch and race: order
 * them on one stream. PA_ERR_DEVICE if the scratch address cannot be read.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_noalloc(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                            int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                            void* stream);

/* ------------------------------------------------------------------------
 * One decode step's cache write and attention in a single launch: the
 * effect of pa_reshape_and_cache(cache, k_new, v_new, src_dtype,
 * slot_mapping, B) followed by pa_decode(..., PA_PARTITION_BALANCED, ...)
 * ([course] §2 primer: the cache grows by one token per decode step, and
 * that token takes part in the step's own attention). For each sequence s
 * with L = context_lens[s] >= 1, token L - 1 is the new one: the attention
 * reads its K/V from k_new[s] / v_new[s] ([B][num_kv_heads][head_dim],
 * device, the pool's dtype) instead of from the cache, and writes that row
 * into the cache at slot_mapping[s] (device int64[B]; < 0: no write).
 * slot_mapping[s] must be the slot of token L - 1 under block_tables[s]
 * (what pa_alloc returned for it; PA_DEBUG=1 checks it). Run any
 * copy-on-write pa_copy_blocks of the step first, on the same stream.
 *
 * The other arguments, the workspace and the errors are those of pa_decode
 * with partition_size = PA_PARTITION_BALANCED. F16 and BF16 pools, either
 * V layout (else PA_ERR_UNSUPPORTED); k_new / v_new 16-byte
 * aligned, slot_mapping 8-byte aligned (else PA_ERR_INVALID_ARGUMENT).
 * ---------------------------------------------------------------------- */
pa_status pa_decode_append(const pa_kv_cache* cache, const void* k_new, const void* v_new, pa_dtype src_dtype,
                           const int64_t* slot_mapping, void* out, pa_dtype out_dtype, const void* q,
                           pa_dtype q_dtype, const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, int32_t B, int32_t num_q_heads, int32_t max_context_len,
                           float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention with shared prefixes read once per group ([course] §2
 * "The bonus": forked sequences share the prompt's blocks; [note]
 * prefix-sharing section). The result is that of pa_decode on the same
 * batch (up to rounding); what differs is the K/V traffic: a group's
 * shared prefix is read once for all the group's query rows, instead of
 * once per member.
 *
 * Groups (device arrays, typically from pa_bm_shared_prefixes): group gi's
 * batch rows are group_members[group_offsets[gi] .. group_offsets[gi + 1]);
 * shared_len[s] (device int32[B]) = tokens at the start of row s that its
 * whole group shares: the same value for every member, a multiple of
 * partition_size, below context_lens[s], and the members' tables identical
 * over those tokens' blocks; 0 for rows in no group. max_group_size >= the
 * largest group, max_shared_len >= every shared_len (and < max_context_len)
 * and min_shared_len <= every shared_len (multiples of partition_size; 0
 * when some row is in no group) size the launch. PA_DEBUG=1 checks all of this; otherwise a violation
 * gives wrong results for the rows involved (no out-of-bounds access).
 *
 * partition_size: a positive multiple of 16 and of block_size (the unit
 * of shared_len); the workspace is pa_decode_shared_workspace_size(...,
 * partition_size) bytes. Either V layout, any pool dtype. Other arguments
 * and errors as pa_decode.
 *
 * Two implementations, the same attention up to rounding:
 *  - the cascade (token-major V or fp8 pools, groups of at most 32 / G
 *    rows, the batch's plan in LDS): the balanced split runs over the
 *    groups' prefixes (each read once, with all the group's query rows) and
 *    the rows' own tokens as one workload, then each row's two partial
 *    softmax states are merged (log-sum-exp; [note] prefix-sharing
 *    section: the shared part is computed once and reused);
 *  - otherwise, or with a workspace of only pa_decode_workspace_size(...)
 *    bytes, partitions of partition_size tokens: each partition of a
 *    group's shared prefix is read once for all its rows, the rest per
 *    row, merged by the partition reduce.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_shared(const pa_kv_cache* cache, void* out, pa_dtype out_dtype, const void* q, pa_dtype q_dtype,
                           const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens, int32_t B,
                           int32_t num_q_heads, int32_t max_context_len, float scale, int32_t partition_size,
                           const int32_t* group_offsets, const int32_t* group_members, const int32_t* shared_len,
                           int32_t num_groups, int32_t max_group_size, int32_t max_shared_len,
                           int32_t min_shared_len, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Measurement aid (not part of the method): the device's attainable read
 * bandwidth, the reference the decode's K/V bytes per second are compared
 * with. Reads buf[0 .. bytes) once: 16-byte non-temporal loads, a
 * grid-stride loop over `grid` workgroups of 256 threads, every word read
 * XOR-folded into sink[grid * 256] (device uint32, caller-owned; its
 * contents are meaningless). buf: device, 16-byte aligned, bytes a positive
 * multiple of 16. Asynchronous on `stream`. Errors: PA_ERR_INVALID_ARGUMENT
 * (checked before the launch), PA_ERR_DEVICE.
 * ---------------------------------------------------------------------- */
pa_status pa_ref_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBPAGEDATTN_H */
