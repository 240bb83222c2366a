/*
 * pkv.h -- C ABI of libpkv: attention over a paged KV cache on MI355X (gfx950).
 *
 * The method (PagedAttention with continuous batching) is described on these pages:
 *   [P17] "Project 17: Production Serving: Continuous Batching and PagedAttention"
 *         (llm-under-the-hood), sections "The Concept", "Step 4: Implement the paged
 *         KV cache", "Step 6: Implement attention over paged storage".
 *   [CB]  "Continuous Batching" (infra.pidoku inference-engineering notes), sections
 *         "4. Tiny example", "5. Technical explanation", "6. Under the hood".
 *   [PY]  "Build a pure-Python continuous batching LLM serving engine from scratch",
 *         "Step 2: Implement the PagedAttention KV Cache Manager".
 *   [TV]  tiny-vllm code reading, part 7 (jaehun.me), "Uploading the active arrays to
 *         the GPU", "Termination and returning blocks".
 *
 * Conventions for every entry point:
 *   - Return 0 (PKV_OK) or a negative status; nothing is thrown across the ABI.
 *     On an error return no host state has changed and no kernel was launched;
 *     pkv_last_error() gives a message (per thread).
 *   - "host" pointers are CPU memory owned by the caller; "device" pointers are GPU
 *     memory owned by the caller (the library never allocates device memory).
 *   - `stream` is a hipStream_t (NULL = the default stream). Device work is
 *     asynchronous on that stream; PKV_ERR_HIP reports a failed launch.
 *   - KV cache layout, per layer: two planes, K and V, each row-major
 *     [num_blocks][block_size][num_kv_heads][head_dim] (the [P17] Step 6 pool axes with
 *     the K/V axis hoisted into separate planes). Flat slot = block * block_size + offset.
 *   - Dtype codes: PKV_F32, PKV_BF16 (raw bfloat16), PKV_FP8_E4M3 (OCP E4M3, cache only;
 *     value = code * per-tensor scale).
 *   - Query head h uses KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_ERR_INVALID (-1)
#define PKV_ERR_OUT_OF_BLOCKS (-2)
#define PKV_ERR_HIP (-3)
#define PKV_ERR_UNSUPPORTED (-4)

#define PKV_F32 0
#define PKV_BF16 1
#define PKV_FP8_E4M3 2

typedef struct pkv_pool pkv_pool;

/* Layer batching. The layers of a model run the same step over the same metadata (block
 * tables, lengths, plans, work lists) with planes, queries and outputs of their own; a
 * *_layers entry point covers num_layers of them in one launch per kernel (the layer is
 * a grid dimension). The call's pointers are layer 0's; layer l's tensors sit l strides
 * further. Strides may be 0 only when num_layers is 1 (layers must not alias their
 * outputs). Read during the call only. */
typedef struct pkv_layers {
  int32_t num_layers;   /* >= 1 */
  int64_t in_bytes;     /* between layers of the inputs: q (attention), k and v (cache write) */
  int64_t out_bytes;    /* between layers of out (attention; unused by the cache write) */
  int64_t cache_bytes;  /* between layers of k_cache and of v_cache */
  int64_t lse_floats;   /* between layers of lse_out (unused when lse_out is NULL) */
} pkv_layers;

/* Library version string (static storage). */
const char* pkv_version(void);
/* Message of the last error returned on this thread (static per-thread storage). */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------------------
 * Host block pool and per-sequence block tables.
 * [P17] "Step 4": one pool of fixed-size pages and a free list; a page is taken from
 * the END of the free list and a freed page is appended; a finished sequence returns
 * its pages in page-table order. [PY] "Step 2": a multi-block request is
 * all-or-nothing and fails when fewer blocks are free. The pool is host state only
 * (no device memory); it is not thread-safe.
 * ---------------------------------------------------------------------------- */

/* Create a pool of num_blocks ids. initial_free_order (host, num_blocks ids, a
 * permutation of 0..num_blocks-1) is the initial free list, popped from its end;
 * NULL means 0..num_blocks-1. plane_bytes (nullable) receives the byte size of one
 * K or V plane of one layer for this geometry. Errors: INVALID on bad sizes,
 * dtype or a non-permutation. */
int pkv_alloc_pool(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, int32_t cache_dtype, const int32_t* initial_free_order,
                   pkv_pool** out, int64_t* plane_bytes);
void pkv_destroy_pool(pkv_pool* pool);

/* Pop n ids from the end of the free list into out_ids (host, n entries), in pop
 * order. OUT_OF_BLOCKS (nothing taken) if fewer than n are free. */
int pkv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids);
/* Append ids (host, n entries) to the free list in the given order. INVALID (nothing
 * freed) if an id is out of range, not allocated, repeated, or held by a sequence. */
int pkv_pool_free(pkv_pool* pool, const int32_t* ids, int32_t n);
/* Counters: free blocks, sequences holding a table (either pointer nullable). */
int pkv_pool_stats(const pkv_pool* pool, int32_t* free_blocks, int32_t* live_seqs);
/* Copy the free list, bottom to top (the next pop is the last entry), into out
 * (host, capacity entries); *count = its length. INVALID if capacity is too small. */
int pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t capacity, int32_t* count);

/* Grow sequence seq_id's table to ceil(total_tokens / block_size) blocks (never
 * shrinks; creates the sequence if new). New ids are popped as by pkv_pool_alloc,
 * appended to the table and held once. OUT_OF_BLOCKS: nothing changes. */
int pkv_seq_reserve(pkv_pool* pool, int64_t seq_id, int32_t total_tokens);
/* Forget seq_id's table: each of its blocks loses one reference, and those no other
 * table holds go back to the free list in table order (a table nobody shares frees its
 * whole table in table order). INVALID if unknown. */
int pkv_seq_release(pkv_pool* pool, int64_t seq_id);
/* Prefix sharing ([P17] "Step 8: Prefix caching"; reference counts as in [PY] "Step 2"):
 * start seq_id's table (new or empty) with n blocks (host array) that other tables hold,
 * each gaining a reference; later pkv_seq_reserve calls append own blocks after them.
 * INVALID (nothing changed) if seq_id already holds blocks or a block is not held by a
 * sequence or repeated. The caller must never write into a shared block. */
int pkv_seq_share(pkv_pool* pool, int64_t seq_id, const int32_t* blocks, int32_t n);
/* Copy the reference count of every block (host, capacity >= num_blocks entries): the
 * number of tables holding it (0 for free and pkv_pool_alloc blocks). */
int pkv_block_refs(const pkv_pool* pool, int32_t* refs, int32_t capacity);
/* Copy seq_id's table (host, capacity entries); *count = its length. */
int pkv_seq_table(const pkv_pool* pool, int64_t seq_id, int32_t* out, int32_t capacity,
                  int32_t* count);

/* Per-step metadata ([CB] "6. Under the hood": cu_seqlens, block_tables
 * (num_seqs, max_blocks), seq_lens; [P17] "Step 4": position p lives in page p/bs at
 * slot p%bs). For sequence s (host arrays of num_seqs entries): seq_lens[s] counts its
 * tokens after this step's q_lens[s] new tokens are written ([TV]: the current token's
 * K/V is stored before attention), the new tokens being positions
 * seq_lens[s]-q_lens[s] .. seq_lens[s]-1. Outputs (host):
 *   block_tables [num_seqs][table_width] int32: table[s][j] for j < ceil(seq_lens[s]/bs),
 *                 -1 elsewhere;
 *   cu_seqlens_q [num_seqs+1] int32: exclusive prefix sum of q_lens;
 *   slot_mapping [sum q_lens] int64: table[s][p/bs]*bs + p%bs for each new token.
 * INVALID if a sequence is unknown, q_len > seq_len, its table is shorter than
 * ceil(seq_len/bs), or table_width is too small. */
int pkv_build_block_table(const pkv_pool* pool, int32_t num_seqs, const int64_t* seq_ids,
                          const int32_t* q_lens, const int32_t* seq_lens, int32_t table_width,
                          int32_t* block_tables, int32_t* cu_seqlens_q, int64_t* slot_mapping);

/* ------------------------------------------------------------------------------
 * Device kernels.
 * ---------------------------------------------------------------------------- */

/* Cache write ([P17] "Step 4", append): for each new token i < num_tokens and KV head
 * h, k_cache[slot_i][h][:] = enc(k[i][h][:]) and the same for v, slot_i =
 * slot_mapping[i]. k, v: device [num_tokens][num_kv_heads][head_dim] in in_dtype.
 * k_cache, v_cache: device planes (layout above, num_blocks blocks) in cache_dtype.
 * slot_mapping: device int64 [num_tokens]; a slot < 0 or >= num_blocks*block_size
 * skips the token. enc: bit copy when in_dtype == cache_dtype (f32, bf16); for an
 * E4M3 cache, y = fl32(x * fl32(1/scale)) rounded to nearest-even E4M3, |y| >= 448
 * saturating to 448 with y's sign, NaN -> 0x7F with y's sign. Supported
 * (in, cache): (f32,f32), (bf16,bf16), (bf16,fp8), (f32,fp8); else UNSUPPORTED.
 * Two tokens mapped to one slot race (the result is one of them).
 * Per-head E4M3 scales (all attention calls take the same pair): k_head_scales /
 * v_head_scales are host float [num_kv_heads] or NULL (factors of 1); head h's scale is
 * k_scale * k_head_scales[h] (the product in double), so scale above is that product
 * for head h's elements. Each factor must be finite and > 0; with per-head factors
 * num_kv_heads is at most 16 and head_dim a multiple of 8 (INVALID otherwise). They are
 * read during the call only. */
int pkv_kv_cache_write(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens,
                       int32_t num_kv_heads, int32_t head_dim, void* k_cache, void* v_cache,
                       int32_t cache_dtype, int32_t num_blocks, int32_t block_size,
                       const int64_t* slot_mapping, float k_scale, float v_scale,
                       const float* k_head_scales, const float* v_head_scales, void* stream);
/* pkv_kv_cache_write for layers->num_layers layers in one launch (pkv_layers above): layer
 * l writes its k and v (in_bytes apart) into its planes (cache_bytes apart) at the same
 * slots. Errors as for pkv_kv_cache_write, and INVALID for a NULL layers, num_layers < 1,
 * or strides that are negative, not multiples of 16, or 0 with num_layers > 1. */
int pkv_kv_cache_write_layers(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, void* k_cache, void* v_cache,
                              int32_t cache_dtype, int32_t num_blocks, int32_t block_size,
                              const int64_t* slot_mapping, float k_scale, float v_scale,
                              const float* k_head_scales, const float* v_head_scales,
                              const pkv_layers* layers, void* stream);

/* Decode work list (host): one item per non-empty (sequence, context partition), so the
 * decode launch has no idle workgroups. seq_lens: host int32 [num_seqs] (the values the
 * device copy holds). partition_size: as for pkv_paged_attention_decode (0 = one item per
 * sequence). items: host int32 [capacity][4] receiving (seq, partition, partitions of
 * that sequence, end token of the partition); a sequence of length 0 still gets one item
 * (it writes zeros). Order: longest item first (full partitions in sequence order, then
 * the shorter last partitions by decreasing length). *count = number of items. INVALID
 * if capacity is too small (nothing written) or partition_size < 0. */
int pkv_build_decode_work(int32_t num_seqs, const int32_t* seq_lens, int32_t partition_size,
                          int32_t* items, int32_t capacity, int32_t* count);

/* Bytes of device workspace that pkv_paged_attention_decode needs for this shape
 * (0 when partition_size is 0 or no sequence can span two partitions). */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_seq_len, int32_t partition_size);

/* Decode attention, one query token per sequence ([P17] "Step 6": walk the page table,
 * score each key against the query scaled by `scale`, softmax, sum the values).
 * q: device [num_seqs][num_q_heads][head_dim] (q_dtype f32 or bf16); out: device,
 * same shape and dtype. The query of sequence s sits at position seq_lens[s]-1 and
 * sees keys 0..seq_lens[s]-1. block_tables: device int32 [num_seqs][table_width];
 * seq_lens: device int32 [num_seqs], each in 0..min(max_seq_len, table_width*bs)
 * (a sequence with seq_len 0 gets zeros and log-sum-exp -inf; larger values are
 * clamped to that bound); table entries outside 0..num_blocks-1 are skipped.
 * Keys are decoded as code * k_scale (values * v_scale) for an E4M3 cache, times
 * k_head_scales[h] (v_head_scales[h]) for KV head h when those host arrays
 * [num_kv_heads] are given (NULL: 1; at most 16 KV heads with them; as in
 * pkv_kv_cache_write); pass 1.0 and NULL otherwise. The same scale arguments, with the
 * same meaning, are taken by the split decode, the varlen and the chunk launches. Supported: (q, cache) in {(f32,f32), (bf16,bf16), (bf16,fp8)};
 * head_dim 64 or 128; block_size 16 or 32; num_q_heads/num_kv_heads in {1,2,4,8}.
 * partition_size 0 processes each sequence in one pass; otherwise (a multiple of
 * block_size) the context is split into partitions of that many tokens whose partial
 * results are merged by log-sum-exp in a second kernel, using `workspace` (device,
 * >= pkv_decode_workspace_bytes). lse_out (device float [num_seqs][num_q_heads],
 * nullable) receives the natural-log log-sum-exp of the scaled scores.
 * work_items (device int32 [num_work][4], nullable): the list pkv_build_decode_work
 * returns for these seq_lens and partition_size; with it the launch covers exactly the
 * listed items (a sequence missing from the list is not computed), without it every
 * (sequence, possible partition) gets a workgroup that exits when empty. */
int pkv_paged_attention_decode(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                               const void* v_cache, int32_t cache_dtype,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t table_width, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_seq_len, float scale,
                               float k_scale, float v_scale, const float* k_head_scales,
                               const float* v_head_scales, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, float* lse_out,
                               const int32_t* work_items, int32_t num_work, void* stream);

/* Balanced split plan (host) for pkv_paged_attention_decode_split. The context of each
 * sequence is cut into 16-token tiles (the last one partial) and the tiles of all
 * sequences are laid end to end; slot j of the launch streams tiles
 * [slot_lo[j], slot_lo[j + 1]). The boundaries make every slot take the same time under
 * a cost model: a slot costs its tiles plus piece_cost_tokens / 16 tiles for each piece
 * (a sequence, or part of one, that it streams: entering it and writing its output or
 * partial), so a slot that crosses many short sequences gets fewer tiles. Slots are
 * filled in order, each to the remaining cost over the remaining slots; at most
 * min(num_slots, total tiles / ceil(min_piece_tokens / 16)) slots are used (at least one
 * when there is any context; fewer when a slot would cost more in pieces than it saves),
 * the rest are empty. seq_lens: host int32 [num_seqs] (the
 * values the device copy holds). plan: host int32 [capacity], capacity >=
 * 3 * num_seqs + 2 * num_slots + 2, receiving in order: the tile offsets [num_seqs + 1]
 * (offset of sequence s = tiles of sequences 0..s-1); the first sequence with a tile at
 * or past each slot's start [num_slots]; slot_lo [num_slots + 1] (non-decreasing, the
 * last entry the total); and for each sequence its first slot and number of pieces
 * [num_seqs][2] (pieces 0 for an empty sequence). *tiles_per_slot = the most tiles in
 * one slot; *max_pieces = the most slots one sequence spans. INVALID on a bad argument, a
 * short capacity or more than 2^31 - 2 tiles (nothing useful written). */
int pkv_build_decode_split(int32_t num_seqs, const int32_t* seq_lens, int32_t min_piece_tokens,
                           int32_t piece_cost_tokens, int32_t num_slots, int32_t* plan,
                           int32_t capacity, int32_t* tiles_per_slot, int32_t* max_pieces);

/* Slots that fill the current device with resident workgroups of the balanced-split
 * decode kernel for this cache dtype and shape (any value >= 1 is correct; this one
 * keeps every compute unit busy for one wave of workgroups). UNSUPPORTED for shapes
 * pkv_paged_attention_decode_split does not take; PKV_ERR_HIP if the query fails. */
int pkv_decode_split_slots(int32_t cache_dtype, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t* slots);

/* Bytes of device workspace pkv_paged_attention_decode_split needs for a plan over
 * num_slots slots: float32 partial outputs [num_slots][2][num_q_heads][head_dim] and
 * log-sum-exps [num_slots][2][num_q_heads] (a slot holds at most two pieces of sequences
 * that span several slots: its first and its last), so the size does not depend on the
 * batch; 0 when max_pieces <= 1 (no sequence spans two slots). */
size_t pkv_decode_split_workspace_bytes(int32_t num_slots, int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_pieces);

/* Decode attention with a balanced split of the context over a fixed number of slots
 * (the attention of [P17] "Step 6", as for pkv_paged_attention_decode; the split and
 * its log-sum-exp merge are this library's scheduling, not the pages'). Arguments from
 * `out` to `v_scale` and `lse_out`: as for pkv_paged_attention_decode (num_seqs = the
 * batch's sequences, the rows of block_tables and seq_lens), with bf16 queries and a
 * bf16 or E4M3 cache, head_dim 64/128, block_size 16/32, at most 16 query heads per KV
 * head. Which rows are decoded: rows (device int32 [num_rows], nullable) gives the batch
 * sequence of each plan row, e.g. the decode rows of a mixed step; NULL means every
 * sequence in order (num_rows must equal num_seqs). Where queries and outputs live:
 * with cu_seqlens_q (device int32 [num_seqs + 1], nullable) q and out are
 * [total_q][num_q_heads][head_dim] and sequence b's row is its last new token,
 * cu_seqlens_q[b + 1] - 1 (for a decode row, its only one); with NULL they are
 * [num_seqs][...] and total_q must equal num_seqs. lse_out follows the same rows. plan:
 * device int32, the array pkv_build_decode_split returned for the plan rows' seq_lens
 * (in plan-row order) and num_slots (tiles_per_slot and max_pieces likewise); the launch
 * has num_slots workgroups per group of KV heads. A plan row inside one slot's range is
 * written directly, as are zeros (log-sum-exp -inf) for rows without context; the
 * pieces of one spanning several slots leave partials in the workspace, merged by
 * log-sum-exp in a second kernel (one workgroup per plan row and 256 output chunks;
 * rows held by one slot leave at once; not launched when max_pieces <= 1). workspace: device, >=
 * pkv_decode_split_workspace_bytes(num_slots, num_q_heads, head_dim, max_pieces);
 * nothing in it needs to start at zero, and calls that share one workspace must not
 * overlap. A plan or row map that does not match the batch
 * reads no memory out of bounds: a piece whose row falls outside the batch or that does
 * not fit is masked and not written. */
int pkv_paged_attention_decode_split(void* out, const void* q, int32_t q_dtype,
                                     const void* k_cache, const void* v_cache,
                                     int32_t cache_dtype, const int32_t* block_tables,
                                     const int32_t* seq_lens, int32_t table_width,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_seq_len, float scale, float k_scale,
                                     float v_scale, const float* k_head_scales,
                                     const float* v_head_scales, const int32_t* rows, int32_t num_rows,
                                     const int32_t* cu_seqlens_q, int32_t total_q,
                                     const int32_t* plan, int32_t num_slots,
                                     int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
                                     size_t workspace_bytes, float* lse_out, void* stream);
/* pkv_paged_attention_decode_split for layers->num_layers layers in one launch of each
 * kernel (pkv_layers above): the plan, rows and tables are shared; layer l reads its q
 * and planes and writes its out and lse_out. workspace_bytes must cover num_layers
 * times pkv_decode_split_workspace_bytes (layer l's partials at l times that size).
 * Errors as for pkv_paged_attention_decode_split, and INVALID for a NULL layers,
 * num_layers < 1, or strides that are negative, not multiples of 16 bytes (4 floats for
 * lse_floats), or 0 with num_layers > 1. */
int pkv_paged_attention_decode_split_layers(void* out, const void* q, int32_t q_dtype,
                                            const void* k_cache, const void* v_cache,
                                            int32_t cache_dtype, const int32_t* block_tables,
                                            const int32_t* seq_lens, int32_t table_width,
                                            int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t block_size, int32_t num_blocks,
                                            int32_t max_seq_len, float scale, float k_scale,
                                            float v_scale, const float* k_head_scales,
                                            const float* v_head_scales, const int32_t* rows,
                                            int32_t num_rows, const int32_t* cu_seqlens_q,
                                            int32_t total_q, const int32_t* plan, int32_t num_slots,
                                            int32_t tiles_per_slot, int32_t max_pieces,
                                            void* workspace, size_t workspace_bytes, float* lse_out,
                                            const pkv_layers* layers, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): pkv_paged_attention_decode_split
 * with its partials in a fixed device array of the library (pkv_decode_split_noalloc_
 * max_bytes() bytes, one per device, held until the process ends) instead of a
 * workspace argument. Arguments and results as for pkv_paged_attention_decode_split
 * without workspace / workspace_bytes; the current device must be the stream's. The
 * call allocates nothing (the array's device address is looked up once per device, on
 * the first call there). INVALID, with nothing launched, when
 * pkv_decode_split_workspace_bytes(num_slots, num_q_heads, head_dim, max_pieces) exceeds
 * the array. Every call on one device shares its array: calls that overlap on a device
 * (other streams, other threads) race and must be serialised by the caller. */
size_t pkv_decode_split_noalloc_max_bytes(void);
int pkv_paged_attention_decode_split_noalloc(void* out, const void* q, int32_t q_dtype,
                                             const void* k_cache, const void* v_cache,
                                             int32_t cache_dtype, const int32_t* block_tables,
                                             const int32_t* seq_lens, int32_t table_width,
                                             int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks,
                                             int32_t max_seq_len, float scale, float k_scale,
                                             float v_scale, const float* k_head_scales,
                                             const float* v_head_scales, const int32_t* rows,
                                             int32_t num_rows, const int32_t* cu_seqlens_q,
                                             int32_t total_q, const int32_t* plan,
                                             int32_t num_slots, int32_t tiles_per_slot,
                                             int32_t max_pieces, float* lse_out, void* stream);

/* Varlen work list (host) for pkv_paged_attention_prefill_varlen. For each sequence s
 * with q = q_lens[s] new tokens and seq_len L = seq_lens[s] (host int32 arrays):
 * q == 1 gives one decode item per KV head; q > 1 gives one prefill item
 * per KV head and per block of 128/G new tokens (G = group = num_q_heads/num_kv_heads),
 * whose keys end at the block's last position + 1; q == 0 gives none. items: host int32
 * [capacity][4] = (seq, kind << 24 | KV head or head group, first new token of the
 * block, keys to visit); longest first (by keys to visit). *count = number of items. INVALID if
 * q > L or capacity is too small; UNSUPPORTED unless G is 1, 2, 4, 8 or 16. */
int pkv_build_varlen_work(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                          int32_t num_kv_heads, int32_t group, int32_t* items, int32_t capacity,
                          int32_t* count);

/* Attention for a mixed step of prefill chunks and decode rows in one launch ([CB]
 * "5. Technical explanation", mixed batching: varlen kernels over cu_seqlens; [P17]
 * "Step 6" per row). Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
 * (device int32 [num_seqs+1], total_q rows in all); its new row i sits at position
 * seq_lens[s] - q_s + i and sees keys 0 .. that position (bottom-right causal; the step's
 * K/V are already in the cache). q, out: device bf16 [total_q][num_q_heads][head_dim].
 * Cache, block_tables, seq_lens, scales, num_blocks, max_seq_len: as for decode, except
 * that table entries outside 0..num_blocks-1 (never dereferenced) read as zero keys and
 * values here, where decode skips their keys.
 * work_items: device int32 [num_work][4] from pkv_build_varlen_work for the same q_lens
 * and seq_lens (rows not covered by an item are not written). lse_out: device float
 * [total_q][num_q_heads], nullable (natural log). Supported: bf16 queries with a bf16
 * or E4M3 cache, head_dim 64/128, block_size 16/32, group 1/2/4/8/16. */
int pkv_paged_attention_prefill_varlen(void* out, const void* q, int32_t q_dtype,
                                       const void* k_cache, const void* v_cache,
                                       int32_t cache_dtype, const int32_t* block_tables,
                                       const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                                       int32_t table_width, int32_t num_seqs, int32_t total_q,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                                       float scale, float k_scale, float v_scale,
                                       const float* k_head_scales, const float* v_head_scales,
                                       const int32_t* work_items, int32_t num_work, float* lse_out,
                                       void* stream);

/* Chunk work list (host) for pkv_paged_attention_prefill_chunks. For each sequence s with
 * q = q_lens[s] >= 2 new tokens and seq_len L = seq_lens[s] (host int32 arrays; q < 2 gives
 * nothing: decode rows go to the split decode), one row block per KV head g and per 128/G
 * new tokens q0.. (G = group), whose keys end at the block's last position + 1 ([P17]
 * "Step 6", causal). With T the 64-key tiles of all blocks and num_slots > 0 (for
 * instance pkv_chunk_slots), a block of more than
 * max_tiles = max(1, min_piece_tiles, ceil(T / num_slots)) tiles is cut into
 * np = ceil(tiles / max_tiles) pieces of whole tiles whose sizes differ by at most one
 * tile (num_slots <= 0: nothing is cut); each piece writes a partial into its own workspace slot and one merge
 * record combines the block's pieces by log-sum-exp (the decomposition of [P17] "Step 6"
 * over disjoint key ranges). items: host int32 [capacity][8] = (seq, KV head, first new
 * token of the block, first key, key end, slot or -1, 0, 0), most tiles first;
 * merges: host int32 [merge_capacity][4] = (seq, KV head, first new token, first slot |
 * np << 20); *count, *merge_count, *num_partials = items, merge records and workspace
 * slots (also set when a capacity is too small). INVALID if q > L, a capacity is too small
 * or the slots reach 2^20; UNSUPPORTED unless G is 1, 2, 4, 8 or 16. */
int pkv_build_chunk_work(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                         int32_t num_kv_heads, int32_t group, int32_t num_slots,
                         int32_t min_piece_tiles, int32_t* items,
                         int32_t capacity, int32_t* count, int32_t* merges, int32_t merge_capacity,
                         int32_t* merge_count, int32_t* num_partials);

/* Host plan of a mixed step ([CB] "5. Technical explanation", mixed batching): the
 * sequences with exactly one new token (decode rows) are listed in batch order in
 * decode_rows (host int32, capacity num_seqs; *num_decode = their count) and get a
 * balanced split plan over num_slots as pkv_build_decode_split would build from their
 * seq_lens (plan, plan_capacity >= 3 * num_seqs + 2 * num_slots + 2, *tiles_per_slot,
 * *max_pieces; left untouched, with both outputs 0, when there is no decode row); the
 * sequences with two or more get the chunk work of pkv_build_chunk_work (items ..
 * num_partials, same meaning and capacities). The decode rows go to
 * pkv_paged_attention_decode_split as its row map, the chunk work to
 * pkv_paged_attention_prefill_chunks. Errors as for the two builders. */
int pkv_build_mixed_step(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                         int32_t num_kv_heads, int32_t group, int32_t num_slots,
                         int32_t min_piece_tokens, int32_t piece_cost_tokens, int32_t chunk_slots,
                         int32_t min_piece_tiles, int32_t* decode_rows, int32_t* num_decode,
                         int32_t* plan, int32_t plan_capacity, int32_t* tiles_per_slot,
                         int32_t* max_pieces, int32_t* items, int32_t capacity, int32_t* count,
                         int32_t* merges, int32_t merge_capacity, int32_t* merge_count,
                         int32_t* num_partials);

/* Decode slots per layer for the one launch of pkv_paged_attention_mixed (num_layers 1) or
 * pkv_paged_attention_mixed_layers: the number of balanced-split slots over which a mixed
 * step's decode rows (q_lens[s] == 1) finish together with its chunk items (q_lens[s] >= 2,
 * the pkv_build_chunk_work items) running on the other compute units. q_lens, seq_lens:
 * host int32 [num_seqs]. With L = ceil(pkv_decode_split_slots / num_layers) (the layers
 * share the units): for a shape the mixed kernel covers (bf16 or E4M3 cache, head_dim
 * 64/128, block_size 16/32, num_kv_heads a multiple of 8) and rows of both kinds, *slots
 * is the slot count at which the decode rows' 16-token tiles and the items' 64-key tiles,
 * at per-unit rates measured on MI355X for these kernels and shapes, end soonest, in
 * [1, L]; otherwise (one kind of row, or a shape that runs as two launches) *slots = L.
 * Pass it to pkv_build_mixed_step as num_slots.
 * INVALID on a bad argument or q > L, and the errors of pkv_decode_split_slots. */
int pkv_mixed_decode_slots(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                           int32_t cache_dtype, int32_t num_kv_heads, int32_t group, int32_t head_dim,
                           int32_t block_size, int32_t num_layers, int32_t* slots);

/* The attention of a mixed continuous-batching step ([CB] "5. Technical explanation",
 * mixed batching: decode rows and prefill chunks in one batch; every row's attention as
 * in [P17] "Step 6") in one kernel launch plus the log-sum-exp merges. The arguments from
 * out to v_head_scales and lse_out are those of pkv_paged_attention_prefill_chunks (q and
 * out [total_q][num_q_heads][head_dim], rows delimited by cu_seqlens_q); the plan is
 * pkv_build_mixed_step's for the same q_lens and seq_lens: decode_rows (device int32
 * [num_decode_rows]), split_plan / split_slots / tiles_per_slot / max_pieces and
 * split_workspace (>= pkv_decode_split_workspace_bytes; not needed when max_pieces <= 1) as
 * for pkv_paged_attention_decode_split's row map, chunk_items / chunk_merges /
 * num_chunk_partials and chunk_workspace as for pkv_paged_attention_prefill_chunks;
 * num_decode_rows or num_chunk_items may be 0. With a bf16 or E4M3 cache at head_dim 64
 * or 128, block size 16 or 32 and num_kv_heads a multiple of 8, one kernel runs both kinds of
 * workgroup: the first split_slots x num_kv_heads / 8 run the decode pass (one per compute
 * unit, for the whole pass), the rest the chunk items, on the units the decode leaves
 * free, so the memory-bound decode and the MFMA-bound chunks run at the same time (with
 * split_slots from pkv_mixed_decode_slots they end together); then the merges of split
 * decode rows and of cut chunk blocks. Other shapes run the two kernels one after the
 * other (the same results). Every row with q_lens = 1 and every row of a sequence with
 * q_lens >= 2 is written (with its log-sum-exp when lse_out is given). Errors: those of
 * the two calls it combines. Calls sharing a workspace must not overlap. */
int pkv_paged_attention_mixed(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                              const void* v_cache, int32_t cache_dtype, const int32_t* block_tables,
                              const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t table_width,
                              int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                              float scale, float k_scale, float v_scale, const float* k_head_scales,
                              const float* v_head_scales, const int32_t* decode_rows,
                              int32_t num_decode_rows, const int32_t* split_plan, int32_t split_slots,
                              int32_t tiles_per_slot, int32_t max_pieces, void* split_workspace,
                              size_t split_workspace_bytes, const int32_t* chunk_items,
                              int32_t num_chunk_items, const int32_t* chunk_merges,
                              int32_t num_chunk_merges, int32_t num_chunk_partials,
                              void* chunk_workspace, int64_t chunk_workspace_bytes, float* lse_out,
                              void* stream);

/* pkv_paged_attention_mixed for layers->num_layers layers of one step in one launch (the
 * decode workgroups of every layer first, then every layer's chunk items, longest first),
 * with q, out, the cache planes and lse_out strided by layer as for
 * pkv_paged_attention_decode_split_layers; the workspaces hold one plan's partials per layer
 * (num_layers x the bytes of one). Errors as for pkv_paged_attention_mixed, and INVALID for
 * a NULL layers, num_layers < 1 or a bad stride. */
int pkv_paged_attention_mixed_layers(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                     const void* v_cache, int32_t cache_dtype,
                                     const int32_t* block_tables, const int32_t* seq_lens,
                                     const int32_t* cu_seqlens_q, int32_t table_width, int32_t num_seqs,
                                     int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                     const float* k_head_scales, const float* v_head_scales,
                                     const int32_t* decode_rows, int32_t num_decode_rows,
                                     const int32_t* split_plan, int32_t split_slots,
                                     int32_t tiles_per_slot, int32_t max_pieces, void* split_workspace,
                                     size_t split_workspace_bytes, const int32_t* chunk_items,
                                     int32_t num_chunk_items, const int32_t* chunk_merges,
                                     int32_t num_chunk_merges, int32_t num_chunk_partials,
                                     void* chunk_workspace, int64_t chunk_workspace_bytes,
                                     float* lse_out, const pkv_layers* layers, void* stream);

/* Slots to balance chunk work over on the current device (its compute units: a second
 * resident workgroup shares a unit's issue slots, so it adds little throughput): the
 * num_slots of pkv_build_chunk_work. UNSUPPORTED for a cache dtype / head_dim /
 * block_size the kernel does not cover, HIP if the device query fails. */
int pkv_chunk_slots(int32_t cache_dtype, int32_t head_dim, int32_t block_size, int32_t* slots);

/* Device workspace bytes for num_partials slots of pkv_build_chunk_work's split pieces
 * (128 rows of fp32 head_dim outputs plus one log-sum-exp each); 0 when none. */
int64_t pkv_chunk_workspace_bytes(int32_t num_partials, int32_t head_dim);

/* Prefill chunks of a mixed step: new row i of sequence s sits at position
 * seq_lens[s] - q_s + i and attends keys 0 .. that position ([P17] "Step 6", [CB]
 * "5. Technical explanation"; rows delimited by cu_seqlens_q as for
 * pkv_paged_attention_prefill_varlen, whose cache, table, scale and lse_out arguments
 * this shares). work_items: device int32 [num_work][8], merges: device int32
 * [num_merges][4], both from pkv_build_chunk_work for the same q_lens and seq_lens, with
 * num_partials its slot count; workspace: device, at least pkv_chunk_workspace_bytes
 * bytes, 16-byte aligned (not needed when num_partials is 0). The chunk kernel runs one
 * workgroup per item (128 GQA-packed query rows; two groups of 4 waves take the first and
 * the second half of the item's 64-key tiles on MFMA and merge their softmax states), then
 * a merge kernel writes the rows of split blocks. Rows of sequences with q < 2 are not
 * written (with a bf16 cache at head_dim 128 the two groups run in opposite phases,
 * one on the MFMAs while the other computes its softmax). Supported: bf16 queries with a
 * bf16 or E4M3 cache, head_dim 64/128, block_size 16/32, group 1/2/4/8/16. Calls sharing a
 * workspace must not overlap. */
int pkv_paged_attention_prefill_chunks(void* out, const void* q, int32_t q_dtype,
                                       const void* k_cache, const void* v_cache,
                                       int32_t cache_dtype, const int32_t* block_tables,
                                       const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                                       int32_t table_width, int32_t num_seqs, int32_t total_q,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                                       float scale, float k_scale, float v_scale,
                                       const float* k_head_scales, const float* v_head_scales,
                                       const int32_t* work_items, int32_t num_work,
                                       const int32_t* merges, int32_t num_merges, int32_t num_partials,
                                       void* workspace, int64_t workspace_bytes, float* lse_out,
                                       void* stream);
/* pkv_paged_attention_prefill_chunks for layers->num_layers layers in one launch of each
 * kernel (pkv_layers above): the work items and merges are shared; layer l reads its q
 * and planes and writes its out and lse_out. workspace_bytes must cover num_layers
 * times pkv_chunk_workspace_bytes (layer l's partials at l times that size). Errors as
 * for pkv_paged_attention_prefill_chunks, and INVALID for a NULL layers, num_layers < 1,
 * or strides that are negative, not multiples of 16 bytes (4 floats for lse_floats), or
 * 0 with num_layers > 1. */
int pkv_paged_attention_prefill_chunks_layers(void* out, const void* q, int32_t q_dtype,
                                              const void* k_cache, const void* v_cache,
                                              int32_t cache_dtype, const int32_t* block_tables,
                                              const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                                              int32_t table_width, int32_t num_seqs, int32_t total_q,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                              int32_t max_seq_len, float scale, float k_scale,
                                              float v_scale, const float* k_head_scales,
                                              const float* v_head_scales, const int32_t* work_items,
                                              int32_t num_work, const int32_t* merges, int32_t num_merges,
                                              int32_t num_partials, void* workspace,
                                              int64_t workspace_bytes, float* lse_out,
                                              const pkv_layers* layers, void* stream);

/* Continuous-batching scheduler step (host) over a pool ([CB] "4. Tiny example",
 * the engine loop: admit, one mixed forward pass, update; [CB] "5. Technical
 * explanation", preemption by recompute). Each request's id is its sequence id in the
 * pool (the scheduler reserves and releases its table). One step is:
 *   pkv_sched_schedule: requests whose arrival step <= the current step join the back of
 *     the waiting queue in (arrival, id) order; then, while fewer than max_running run,
 *     the head of the queue is admitted if ceil((prompt + outputs so far) / block_size)
 *     blocks can be reserved for it, else admission stops (strict first come, first
 *     served). Reports the step's rows, new tokens and widest table.
 *   pkv_sched_plan (any number of times): the rows in running order -- id, stage (0
 *     prefill: prompt + outputs so far new tokens at positions 0..; 1 decode: one new
 *     token, the last output, at position prompt + outputs - 1), q_len, seq_len -- and
 *     their block_tables / cu_seqlens_q / slot_mapping as pkv_build_block_table makes
 *     them (host arrays; block_tables [rows][table_width], slot_mapping [total q]).
 *   pkv_sched_update: in running order, one output token per decode row and per prefill
 *     row that completes its context (see chunked prefill below); a request with
 *     max_tokens outputs finishes and frees its table at once; one whose next token needs
 *     a new block reserves one, or, if none is free, is preempted: its table is freed and
 *     it goes to the front of the waiting queue (several preempted in one step end up in
 *     reverse order), to be re-prefilled with its outputs. The step number advances.
 * Calls out of this order are INVALID. pkv_sched_add_requests: host arrays [n]; ids unique
 * and without a table in the pool, prompt >= 1, max_tokens >= 1, arrival >= the current
 * step, and prompt + max_tokens - 1 tokens must fit the pool (else the queue could stall);
 * INVALID otherwise (nothing added). pkv_sched_counters: out int64 [8] = step, free
 * blocks, running, waiting, preemptions so far, finished so far, requests added, prompt
 * tokens served from the prefix cache so far. The scheduler does not own the pool, which
 * must outlive it; not thread-safe.
 * Prefix caching ([P17] "Step 8: Prefix caching"), off unless enabled before the first
 * step: at admission, the longest whole-page prefix of a request's prompt tokens (at
 * most prompt - 1 tokens for a fresh request, which must compute its last prompt token;
 * at most the prompt for a recompute) that the cache maps to still-held pages is shared
 * (pkv_seq_share), the rest reserved, and the request admitted if that rest fits; its
 * prefill row then holds only the uncached tokens (q = context - cached, positions from
 * the cached length). At each update, the whole prompt pages of the step's prefill rows
 * are registered (an existing usable entry stays). An entry dies with its pages: a block
 * freed since it was registered makes it unusable.
 * Chunked prefill under a token budget ([CB] "5. Technical explanation", mixed batching),
 * off unless set before the first step: the rows of a step then carry at most
 * max_batched_tokens new tokens. Every decode row is kept (one token each, even beyond
 * the budget); what is left goes to the prefill rows in running order, each taking the
 * least of its uncomputed context, chunk_tokens and the budget left. A running request
 * that gets 0 tokens has no row in that step (rows are the running requests with tokens,
 * in running order). A prefill row holds positions done..done+q-1 of the context (done:
 * tokens computed by its earlier chunks or found in the prefix cache) with seq_len =
 * done + q; the request gets its first output, and its prompt pages enter the prefix
 * cache, only at the update of the step that computes its last chunk. Blocks for the
 * whole context are still reserved at admission. */
typedef struct pkv_sched pkv_sched;
int pkv_sched_create(pkv_pool* pool, int32_t max_running, pkv_sched** out);
void pkv_sched_destroy(pkv_sched* sched);
int pkv_sched_add_requests(pkv_sched* sched, int32_t n, const int64_t* ids, const int32_t* arrival,
                           const int32_t* prompt, const int32_t* max_tokens);
int pkv_sched_schedule(pkv_sched* sched, int32_t* num_rows, int32_t* total_q, int32_t* max_blocks);
int pkv_sched_plan(const pkv_sched* sched, int32_t table_width, int64_t* ids, int32_t* stages,
                   int32_t* q_lens, int32_t* seq_lens, int32_t* block_tables, int32_t* cu_seqlens_q,
                   int64_t* slot_mapping);
int pkv_sched_update(pkv_sched* sched);
int pkv_sched_counters(const pkv_sched* sched, int64_t* out);
/* Turn prefix caching on (before the first step; see above). */
int pkv_sched_enable_prefix_cache(pkv_sched* sched);
/* Prompt token ids of request id (host int32 [n], n = its prompt length), before the first
 * step; requests without tokens neither hit nor fill the prefix cache. */
int pkv_sched_set_prompt_tokens(pkv_sched* sched, int64_t id, const int32_t* tokens, int32_t n);
/* Token budget per step and prefill chunk size (before the first step; see above); 0 for
 * either means no limit (the default, which gives every prefill its whole context in one
 * row). Negative values are INVALID. */
int pkv_sched_set_token_budget(pkv_sched* sched, int32_t max_batched_tokens, int32_t chunk_tokens);

/* Preemption by swap ([CB] "5. Technical explanation", Preemption: the SWAP strategy),
 * off unless enabled before the first step with a host space of host_blocks >= 1 blocks
 * (host block ids 0..host_blocks-1, handed out from the end of a free list that starts
 * 0, 1, ..., like the device pool). In pkv_sched_update, a request that cannot grow is
 * swapped out when the host space has as many free blocks as its table: each of its
 * blocks, in table order, is paired with a host block popped from the list; its device
 * blocks are freed and it goes to the front of the queue. Otherwise it is preempted by
 * recompute, as without swap. In pkv_sched_schedule, a swapped request at the head of
 * the queue is admitted when ceil((prompt + outputs) / block_size) blocks are free: its
 * table is reserved, host block j is paired with the table's block j, its host blocks
 * return to the free list in table order, and its row in that step is a decode row (no
 * prefill, no prefix lookup). pkv_sched_swap_pairs reports the pairs of the last update
 * (swap-outs, (device block, host block) as int32 [num_out][2]) and of the last schedule
 * (swap-ins, (host block, device block) [num_in][2]); any of the pointers may be NULL.
 * The caller copies the swap-outs (pkv_swap_out) after the update and before the next
 * step's kernels, and the swap-ins (pkv_swap_in) before the step's attention.
 * pkv_sched_swap_counters: out int64 [4] = requests swapped out so far, blocks swapped
 * out, blocks swapped in, free host blocks. */
int pkv_sched_enable_swap(pkv_sched* sched, int32_t host_blocks);

/* Victim policies ([CB] "5. Technical explanation", Preemption: victim selection; the
 * pure-Python engine's preemption of the request with the fewest generated tokens),
 * set before the first step. PKV_VICTIM_SELF (default): the one-pass update above, where
 * a request that cannot grow preempts itself. PKV_VICTIM_LIFO / PKV_VICTIM_FEWEST:
 * pkv_sched_update first appends every row's output and retires finished requests (in
 * running order), then walks the running requests in order; one that produced an output
 * and needs a block for its next token preempts victims until it gets one: the running
 * request admitted last (LIFO) or with the fewest outputs (FEWEST; the earliest admitted
 * on ties), among those of the least important priority class present, itself included
 * (then it stops). Victims are preempted by swap or recompute as above and requeued as
 * above; a swapped victim in the middle of a chunked prefill resumes with its next chunk.
 * Priority admission ([CB] "5. Technical explanation", admission policies):
 * pkv_sched_set_priorities gives requests (by id; host arrays [n]) a class >= 0, 0 the
 * most important, others keep 0, before the first step; the waiting queue is then kept in
 * (class, arrival step, id) order, preempted requests included (they take their place by
 * that key instead of the front), and admission still stops at the first head that does
 * not fit. INVALID: unknown ids, negative classes, calls after the first step. */
enum { PKV_VICTIM_SELF = 0, PKV_VICTIM_LIFO = 1, PKV_VICTIM_FEWEST = 2 };
/* Static batching (enabled != 0, before the first step), the baseline continuous
 * batching is measured against ([CB] "1. What is it?", "2. Why does it exist?": a batch
 * is decided and run to completion): pkv_sched_schedule admits only when nothing is
 * running, so finished requests leave their slots empty (their blocks are still freed at
 * once) and arrivals wait for the whole batch. Everything else is unchanged. */
int pkv_sched_set_static_batching(pkv_sched* sched, int32_t enabled);
int pkv_sched_set_victim_policy(pkv_sched* sched, int32_t policy);
int pkv_sched_set_priorities(pkv_sched* sched, int32_t n, const int64_t* ids, const int32_t* classes);
/* The copies of preemption by swap ([CB] "5. Technical explanation", Preemption: SWAP):
 * a pair moves every layer's K and V block, as the cache's bytes. Layouts: k_cache and
 * v_cache are device planes [num_layers][num_blocks][block_bytes] (block_bytes =
 * block_size * num_kv_heads * head_dim * element size, a positive multiple of 16, both
 * 16-byte aligned); host_space is host memory [host_capacity][num_layers][2 (K, V)]
 * [block_bytes] and should be pinned (hipHostMalloc; pageable memory makes the copies
 * synchronous); workspace is device memory, 16-byte aligned, of at least
 * pkv_swap_workspace_bytes(n, num_layers, block_bytes) bytes (the pairs are staged
 * there). dev_blocks / host_blocks: host int32 [n], every device block in
 * 0..num_blocks-1 and every host block in 0..host_capacity-1, neither repeated
 * (INVALID otherwise, nothing enqueued). pkv_swap_out: a copy kernel gathers the device
 * blocks into the workspace, then DMA copies move them to their host blocks;
 * pkv_swap_in: DMA copies bring the host blocks into the workspace, then a copy kernel
 * scatters them into the device blocks. Both are asynchronous on `stream` (hipStream_t,
 * NULL = default): the host space must not be read (after a swap-out) or rewritten
 * (before a swap-in completes) until the stream has reached that point; n = 0 is a
 * no-op. pkv_swap_out's copy_stream (NULL: `stream`) takes the DMA copies, ordered after
 * the gather by an event, so the transfer overlaps later work on `stream` (whose writes
 * into the freed blocks come after the gather); the workspace and the host blocks are
 * then busy until copy_stream reaches that point, which the caller must wait for before
 * reusing the workspace or reading those host blocks (a later pkv_swap_in included).
 * Errors: INVALID (sizes, pointers, ids), HIP (launch, ordering or copy failure). */
int64_t pkv_swap_workspace_bytes(int32_t n, int32_t num_layers, int64_t block_bytes);
int pkv_swap_out(const void* k_cache, const void* v_cache, int32_t num_layers, int32_t num_blocks,
                 int64_t block_bytes, const int32_t* dev_blocks, const int32_t* host_blocks, int32_t n,
                 void* host_space, int32_t host_capacity, void* workspace, int64_t workspace_bytes,
                 void* stream, void* copy_stream);
int pkv_swap_in(void* k_cache, void* v_cache, int32_t num_layers, int32_t num_blocks, int64_t block_bytes,
                const int32_t* host_blocks, const int32_t* dev_blocks, int32_t n, const void* host_space,
                int32_t host_capacity, void* workspace, int64_t workspace_bytes, void* stream);
int pkv_sched_swap_pairs(const pkv_sched* sched, int32_t* num_out, int32_t* num_in, int32_t* out_pairs,
                         int32_t* in_pairs);
int pkv_sched_swap_counters(const pkv_sched* sched, int64_t* out);

/* Admission without the memory check (enabled = 0), the sabotage of the "Break It"
 * experiment of [P17]: pkv_sched_schedule takes the head of the waiting queue off it and
 * allocates its blocks unchecked; when they do not fit it returns PKV_ERR_OUT_OF_BLOCKS
 * (the pool unchanged, that request out of every queue, the step not scheduled) and the
 * scheduler is not meant to be used further. enabled != 0 restores the check (default). */
int pkv_sched_set_admission_check(pkv_sched* sched, int32_t enabled);

/* Profiling hook (for timing the partition pass alone): while `hip_event` (a
 * hipEvent_t) is not NULL, every pkv_paged_attention_decode and
 * pkv_paged_attention_decode_split call made on this thread records it on its stream
 * right after the partition pass, before the merge kernel (if any). NULL turns the hook off. The caller owns the event. */
void pkv_decode_set_profile_event(void* hip_event);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
