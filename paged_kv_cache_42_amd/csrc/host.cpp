// Host side of libpkv: the block pool, per-sequence block tables and the per-step
// metadata build. Pure C++17, no device calls.
//
// Pool semantics follow "Project 17: Production Serving: Continuous Batching and
// PagedAttention", "Step 4: Implement the paged KV cache" (take from the end of the
// free list, append on free, return a finished sequence's pages in table order) and
// "Build a pure-Python continuous batching LLM serving engine from scratch", "Step 2"
// (a multi-block request is all-or-nothing and fails when too few blocks are free).
#include <algorithm>
#include <cstdint>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int dtype_bytes(int32_t dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

namespace {

bool positive_finite(double x) { return x > 0.0 && x < 1e300; }

// the product of the per-tensor scale and each head's factor (1 when NULL), checked
int head_products(const char* who, int32_t hkv, float base, const float* head, double* out) {
  if (head && hkv > kHeadScales)
    return fail(PKV_ERR_INVALID, "%s: per-head scales need at most %d KV heads, got %d", who, kHeadScales, hkv);
  if (!positive_finite(base) || !std::isfinite(base)) return fail(PKV_ERR_INVALID, "%s: scales must be finite and > 0", who);
  for (int h = 0; h < kHeadScales; ++h) {
    const double f = head && h < hkv ? double(head[h]) : 1.0;
    if (head && h < hkv && (!std::isfinite(head[h]) || !(head[h] > 0.f)))
      return fail(PKV_ERR_INVALID, "%s: per-head scale %d must be finite and > 0", who, h);
    out[h] = double(base) * f;
  }
  return PKV_OK;
}

}  // namespace

int layers_from(const char* who, const pkv_layers* desc, bool required, unsigned uses, Layers* out) {
  *out = Layers{};
  if (!desc) return required ? fail(PKV_ERR_INVALID, "%s: layers is NULL", who) : PKV_OK;
  if (desc->num_layers < 1) return fail(PKV_ERR_INVALID, "%s: num_layers %d < 1", who, desc->num_layers);
  const struct {
    unsigned bit;
    int64_t bytes;
    const char* name;
  } st[] = {{kLayerIn, desc->in_bytes, "in_bytes"},
            {kLayerOut, desc->out_bytes, "out_bytes"},
            {kLayerCache, desc->cache_bytes, "cache_bytes"},
            {kLayerLse, desc->lse_floats * 4, "lse_floats"}};
  for (const auto& x : st) {
    if (!(uses & x.bit)) continue;
    if (x.bytes < 0 || x.bytes % 16 != 0 || (desc->num_layers > 1 && x.bytes == 0))
      return fail(PKV_ERR_INVALID, "%s: layer stride %s must be a positive multiple of 16 bytes", who, x.name);
  }
  out->n = desc->num_layers;
  out->in = uses & kLayerIn ? desc->in_bytes : 0;
  out->out = uses & kLayerOut ? desc->out_bytes : 0;
  out->cache = uses & kLayerCache ? desc->cache_bytes : 0;
  out->lse = uses & kLayerLse ? desc->lse_floats : 0;
  return PKV_OK;
}

int head_scales(const char* who, int32_t num_kv_heads, float scale, float k_scale, float v_scale,
                const float* k_head, const float* v_head, float* zs, float* vs) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(PKV_ERR_INVALID, "%s: scales must be finite and > 0", who);
  double kp[kHeadScales], vp[kHeadScales];
  int rc = head_products(who, num_kv_heads, k_scale, k_head, kp);
  if (rc == PKV_OK) rc = head_products(who, num_kv_heads, v_scale, v_head, vp);
  if (rc != PKV_OK) return rc;
  for (int h = 0; h < kHeadScales; ++h) {
    zs[h] = float(double(scale) * kp[h] * 1.4426950408889634);
    vs[h] = float(vp[h]);
  }
  return PKV_OK;
}

int head_inverse_scales(const char* who, int32_t num_kv_heads, float k_scale, float v_scale,
                        const float* k_head, const float* v_head, float* ki, float* vi) {
  double kp[kHeadScales], vp[kHeadScales];
  int rc = head_products(who, num_kv_heads, k_scale, k_head, kp);
  if (rc == PKV_OK) rc = head_products(who, num_kv_heads, v_scale, v_head, vp);
  if (rc != PKV_OK) return rc;
  for (int h = 0; h < kHeadScales; ++h) {
    ki[h] = float(1.0 / kp[h]);
    vi[h] = float(1.0 / vp[h]);
  }
  return PKV_OK;
}

}  // namespace pkv

using pkv::fail;

#include "pool_internal.h"

namespace pkv {

bool pool_reserve(pkv_pool* p, int64_t id, int64_t tokens) {
  const int64_t want = (tokens + p->block_size - 1) / p->block_size;
  auto it = p->tables.find(id);
  const int64_t have = it == p->tables.end() ? 0 : int64_t(it->second.size());
  const int64_t need = want - have;
  if (need > int64_t(p->free_list.size())) return false;
  std::vector<int32_t>& t = p->tables[id];
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = p->free_list.back();
    p->free_list.pop_back();
    p->state[b] = kInSeq;
    p->ref[b] = 1;
    t.push_back(b);
  }
  return true;
}

void pool_release(pkv_pool* p, int64_t id) {
  auto it = p->tables.find(id);
  if (it == p->tables.end()) return;
  for (int32_t b : it->second) {                 // table order
    if (--p->ref[b] > 0) continue;               // still held by another table
    p->state[b] = kFree;
    ++p->gen[b];
    p->free_list.push_back(b);
  }
  p->tables.erase(it);
}

void pool_share(pkv_pool* p, int64_t id, const int32_t* blocks, int32_t n) {
  std::vector<int32_t>& t = p->tables[id];
  for (int32_t i = 0; i < n; ++i) {
    ++p->ref[blocks[i]];
    t.push_back(blocks[i]);
  }
}

}  // namespace pkv

extern "C" {

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

int pkv_alloc_pool(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, int32_t cache_dtype, const int32_t* initial_free_order,
                   pkv_pool** out, int64_t* plane_bytes) {
  if (!out) return fail(PKV_ERR_INVALID, "alloc_pool: out is NULL");
  if (num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID, "alloc_pool: bad sizes (blocks %d, block_size %d, kv heads %d, head_dim %d)",
                num_blocks, block_size, num_kv_heads, head_dim);
  const int eb = pkv::dtype_bytes(cache_dtype);
  if (eb == 0) return fail(PKV_ERR_INVALID, "alloc_pool: unknown cache dtype %d", cache_dtype);
  auto* p = new pkv_pool();
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->state.assign(num_blocks, kFree);
  p->ref.assign(num_blocks, 0);
  p->gen.assign(num_blocks, 0);
  p->free_list.resize(num_blocks);
  if (initial_free_order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return fail(PKV_ERR_INVALID, "alloc_pool: initial order is not a permutation (entry %d = %d)", i, b);
      }
      seen[b] = 1;
      p->free_list[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->free_list[i] = i;
  }
  if (plane_bytes)
    *plane_bytes = int64_t(num_blocks) * block_size * num_kv_heads * head_dim * eb;
  *out = p;
  return PKV_OK;
}

void pkv_destroy_pool(pkv_pool* pool) { delete pool; }

int pkv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids) {
  if (!pool || n < 0 || (n > 0 && !out_ids)) return fail(PKV_ERR_INVALID, "pool_alloc: bad arguments");
  if (int64_t(pool->free_list.size()) < n)
    return fail(PKV_ERR_OUT_OF_BLOCKS, "pool_alloc: need %d, %zu free", n, pool->free_list.size());
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = pool->free_list.back();
    pool->free_list.pop_back();
    pool->state[b] = kRaw;
    out_ids[i] = b;
  }
  return PKV_OK;
}

int pkv_pool_free(pkv_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !ids)) return fail(PKV_ERR_INVALID, "pool_free: bad arguments");
  std::vector<int32_t> seen;
  seen.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || b >= pool->num_blocks || pool->state[b] != kRaw)
      return fail(PKV_ERR_INVALID, "pool_free: id %d is not a block taken by pool_alloc", b);
    for (int32_t x : seen)
      if (x == b) return fail(PKV_ERR_INVALID, "pool_free: id %d repeated", b);
    seen.push_back(b);
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->state[ids[i]] = kFree;
    pool->free_list.push_back(ids[i]);
  }
  return PKV_OK;
}

int pkv_pool_stats(const pkv_pool* pool, int32_t* free_blocks, int32_t* live_seqs) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool_stats: pool is NULL");
  if (free_blocks) *free_blocks = int32_t(pool->free_list.size());
  if (live_seqs) *live_seqs = int32_t(pool->tables.size());
  return PKV_OK;
}

int pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t capacity, int32_t* count) {
  if (!pool || !count) return fail(PKV_ERR_INVALID, "pool_free_list: bad arguments");
  const int32_t n = int32_t(pool->free_list.size());
  *count = n;
  if (capacity < n || (n > 0 && !out))
    return fail(PKV_ERR_INVALID, "pool_free_list: capacity %d < %d", capacity, n);
  if (n) std::memcpy(out, pool->free_list.data(), sizeof(int32_t) * n);
  return PKV_OK;
}

int pkv_seq_reserve(pkv_pool* pool, int64_t seq_id, int32_t total_tokens) {
  if (!pool || total_tokens < 0) return fail(PKV_ERR_INVALID, "seq_reserve: bad arguments");
  if (!pkv::pool_reserve(pool, seq_id, total_tokens)) {
    const int64_t want = (int64_t(total_tokens) + pool->block_size - 1) / pool->block_size;
    auto it = pool->tables.find(seq_id);
    const int64_t have = it == pool->tables.end() ? 0 : int64_t(it->second.size());
    return fail(PKV_ERR_OUT_OF_BLOCKS, "seq_reserve: sequence %lld needs %lld more blocks, %zu free",
                (long long)seq_id, (long long)(want - have), pool->free_list.size());
  }
  return PKV_OK;
}

int pkv_seq_release(pkv_pool* pool, int64_t seq_id) {
  if (!pool) return fail(PKV_ERR_INVALID, "seq_release: pool is NULL");
  if (!pool->tables.count(seq_id))
    return fail(PKV_ERR_INVALID, "seq_release: unknown sequence %lld", (long long)seq_id);
  pkv::pool_release(pool, seq_id);
  return PKV_OK;
}

int pkv_seq_share(pkv_pool* pool, int64_t seq_id, const int32_t* blocks, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return fail(PKV_ERR_INVALID, "seq_share: bad arguments");
  auto it = pool->tables.find(seq_id);
  if (it != pool->tables.end() && !it->second.empty())
    return fail(PKV_ERR_INVALID, "seq_share: sequence %lld already holds blocks", (long long)seq_id);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (b < 0 || b >= pool->num_blocks || pool->state[b] != kInSeq || pool->ref[b] < 1)
      return fail(PKV_ERR_INVALID, "seq_share: block %d is not held by a sequence", b);
    for (int32_t j = 0; j < i; ++j)
      if (blocks[j] == b) return fail(PKV_ERR_INVALID, "seq_share: block %d repeated", b);
  }
  pkv::pool_share(pool, seq_id, blocks, n);
  return PKV_OK;
}

int pkv_block_refs(const pkv_pool* pool, int32_t* refs, int32_t capacity) {
  if (!pool || (pool->num_blocks > 0 && !refs) || capacity < pool->num_blocks)
    return fail(PKV_ERR_INVALID, "block_refs: bad arguments");
  if (pool->num_blocks) std::memcpy(refs, pool->ref.data(), sizeof(int32_t) * pool->num_blocks);
  return PKV_OK;
}

int pkv_seq_table(const pkv_pool* pool, int64_t seq_id, int32_t* out, int32_t capacity,
                  int32_t* count) {
  if (!pool || !count) return fail(PKV_ERR_INVALID, "seq_table: bad arguments");
  auto it = pool->tables.find(seq_id);
  if (it == pool->tables.end())
    return fail(PKV_ERR_INVALID, "seq_table: unknown sequence %lld", (long long)seq_id);
  const int32_t n = int32_t(it->second.size());
  *count = n;
  if (capacity < n || (n > 0 && !out))
    return fail(PKV_ERR_INVALID, "seq_table: capacity %d < %d", capacity, n);
  if (n) std::memcpy(out, it->second.data(), sizeof(int32_t) * n);
  return PKV_OK;
}

int pkv_build_block_table(const pkv_pool* pool, int32_t num_seqs, const int64_t* seq_ids,
                          const int32_t* q_lens, const int32_t* seq_lens, int32_t table_width,
                          int32_t* block_tables, int32_t* cu_seqlens_q, int64_t* slot_mapping) {
  if (!pool || num_seqs < 0 || table_width < 0 || !cu_seqlens_q ||
      (num_seqs > 0 && (!seq_ids || !q_lens || !seq_lens || (table_width > 0 && !block_tables))))
    return fail(PKV_ERR_INVALID, "build_block_table: bad arguments");
  const int64_t bs = pool->block_size;
  // validate everything before writing anything
  std::vector<const std::vector<int32_t>*> tabs(num_seqs);
  int64_t total_q = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    auto it = pool->tables.find(seq_ids[s]);
    if (it == pool->tables.end())
      return fail(PKV_ERR_INVALID, "build_block_table: unknown sequence %lld", (long long)seq_ids[s]);
    const int64_t L = seq_lens[s], q = q_lens[s];
    if (q < 0 || L < 0 || q > L)
      return fail(PKV_ERR_INVALID, "build_block_table: sequence %d q_len %lld outside 0..seq_len %lld", s,
                  (long long)q, (long long)L);
    const int64_t nblk = (L + bs - 1) / bs;
    if (nblk > int64_t(it->second.size()))
      return fail(PKV_ERR_INVALID, "build_block_table: sequence %d holds %zu blocks, needs %lld", s,
                  it->second.size(), (long long)nblk);
    if (nblk > table_width)
      return fail(PKV_ERR_INVALID, "build_block_table: sequence %d needs %lld blocks > width %d", s,
                  (long long)nblk, table_width);
    tabs[s] = &it->second;
    total_q += q;
  }
  if (total_q > 0 && !slot_mapping) return fail(PKV_ERR_INVALID, "build_block_table: slot_mapping is NULL");
  int64_t r = 0;
  cu_seqlens_q[0] = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const std::vector<int32_t>& t = *tabs[s];
    const int64_t L = seq_lens[s], q = q_lens[s];
    const int64_t nblk = (L + bs - 1) / bs;
    int32_t* row = block_tables + int64_t(s) * table_width;
    for (int64_t j = 0; j < table_width; ++j) row[j] = j < nblk ? t[j] : -1;
    for (int64_t p = L - q; p < L; ++p) slot_mapping[r++] = int64_t(t[p / bs]) * bs + p % bs;
    cu_seqlens_q[s + 1] = int32_t(r);
  }
  return PKV_OK;
}

int pkv_build_decode_work(int32_t num_seqs, const int32_t* seq_lens, int32_t partition_size,
                          int32_t* items, int32_t capacity, int32_t* count) {
  if (num_seqs < 0 || partition_size < 0 || !count || (num_seqs > 0 && !seq_lens))
    return fail(PKV_ERR_INVALID, "build_decode_work: bad arguments");
  struct Item {
    int32_t s, p, n, end, len;
  };
  std::vector<Item> full, tail;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s] < 0 ? 0 : seq_lens[s];
    if (partition_size == 0 || L <= partition_size) {
      tail.push_back({s, 0, 1, L, L});
      continue;
    }
    const int32_t n = int32_t((int64_t(L) + partition_size - 1) / partition_size);
    for (int32_t p = 0; p < n; ++p) {
      const int32_t b = p * partition_size;
      const int32_t e = std::min(L, b + partition_size);
      (e - b == partition_size ? full : tail).push_back({s, p, n, e, e - b});
    }
  }
  std::stable_sort(tail.begin(), tail.end(), [](const Item& x, const Item& y) { return x.len > y.len; });
  const int64_t total = int64_t(full.size()) + int64_t(tail.size());
  *count = int32_t(total);
  if (total > capacity || (total > 0 && !items))
    return fail(PKV_ERR_INVALID, "build_decode_work: %lld items, capacity %d", (long long)total, capacity);
  int32_t* o = items;
  for (const auto* v : {&full, &tail})
    for (const Item& it : *v) {
      o[0] = it.s;
      o[1] = it.p;
      o[2] = it.n;
      o[3] = it.end;
      o += 4;
    }
  return PKV_OK;
}

int pkv_build_decode_split(int32_t num_seqs, const int32_t* seq_lens, int32_t min_piece_tokens,
                           int32_t piece_cost_tokens, int32_t num_slots, int32_t* plan, int32_t capacity,
                           int32_t* tiles_per_slot, int32_t* max_pieces) {
  if (num_seqs < 0 || min_piece_tokens < 0 || piece_cost_tokens < 0 || num_slots < 1 || !tiles_per_slot ||
      !max_pieces || (num_seqs > 0 && !seq_lens))
    return fail(PKV_ERR_INVALID, "build_decode_split: bad arguments");
  const int64_t B = num_seqs, S = num_slots;
  const int64_t need = 3 * B + 2 * S + 2;
  if (need > capacity || !plan)
    return fail(PKV_ERR_INVALID, "build_decode_split: plan needs %lld entries, capacity %d", (long long)need,
                capacity);
  int32_t* cu = plan;                      // [B + 1] tile offsets
  int32_t* first_seq = plan + B + 1;       // [S] first sequence with a tile at or past the slot's start
  int32_t* slot_lo = first_seq + S;        // [S + 1] first tile of each slot, then the total
  int32_t* seq_slots = slot_lo + S + 1;    // [B][2] first slot and number of pieces of each sequence
  // tile offsets of the sequences laid end to end (16-token tiles, the last one partial)
  int64_t total = 0, nonempty = 0;
  cu[0] = 0;
  for (int64_t s = 0; s < B; ++s) {
    const int64_t L = seq_lens[s] < 0 ? 0 : seq_lens[s];
    total += (L + 15) / 16;
    nonempty += L > 0;
    if (total > INT32_MAX - 1) return fail(PKV_ERR_INVALID, "build_decode_split: context too long");
    cu[s + 1] = int32_t(total);
  }
  // Slot boundaries. A slot's time is modelled as its tiles plus `alpha` tiles for each
  // piece (a sequence, or part of one, it enters: queries, table row, softmax state and
  // the output or partial at the end). Slots are filled in stream order, each up to the
  // remaining cost divided by the remaining slots, so every slot ends near the same time
  // whatever the length mix. Slots past the active count (the context split into pieces
  // of at least min_piece_tokens) stay empty.
  const double alpha = piece_cost_tokens / 16.0;
  const int64_t min_tiles = std::max<int64_t>(1, (int64_t(min_piece_tokens) + 15) / 16);
  const int64_t active = total > 0 ? std::max<int64_t>(1, std::min<int64_t>(S, total / min_tiles)) : 0;
  int64_t j = 0;                           // slot being filled
  double cost = 0.0;                       // its cost so far
  int64_t seqs_left = nonempty;            // sequences not yet started
  slot_lo[0] = 0;
  for (int64_t s = 0; s < B && active > 0; ++s) {
    int64_t t = cu[s], end = cu[s + 1];
    if (t == end) continue;
    --seqs_left;
    while (t < end) {
      if (j == active - 1) {               // the last active slot takes the rest
        t = end;
        break;
      }
      const double rem = cost + double(total - t) + alpha * double(1 + seqs_left + (active - 1 - j));
      const double room = rem / double(active - j) - cost - alpha;
      if (room < 0.5 && cost > 0.0) {      // full: the sequence starts in the next slot
        slot_lo[++j] = int32_t(t);
        cost = 0.0;
        continue;
      }
      const int64_t take = std::min<int64_t>(end - t, std::max<int64_t>(1, std::llround(room)));
      cost += alpha + double(take);
      t += take;
      if (t < end) {                       // the sequence continues in the next slot
        slot_lo[++j] = int32_t(t);
        cost = 0.0;
      }
    }
  }
  for (int64_t k = j + 1; k <= S; ++k) slot_lo[k] = int32_t(total);
  // first sequence of each slot, and each sequence's slots
  int64_t s = 0, widest = 0;
  for (int64_t k = 0; k < S; ++k) {
    while (s < B && cu[s + 1] <= slot_lo[k]) ++s;
    first_seq[k] = int32_t(s);
    widest = std::max<int64_t>(widest, slot_lo[k + 1] - slot_lo[k]);
  }
  int32_t pieces_max = 0;
  int64_t k = 0;                           // slot holding tile cu[s]
  for (s = 0; s < B; ++s) {
    while (k + 1 < S && slot_lo[k + 1] <= cu[s]) ++k;
    int64_t np = 0;
    if (cu[s + 1] > cu[s]) {
      int64_t last = k;
      while (last + 1 < S && slot_lo[last + 1] < cu[s + 1]) ++last;
      np = last - k + 1;
    }
    seq_slots[2 * s] = int32_t(k);
    seq_slots[2 * s + 1] = int32_t(np);
    pieces_max = std::max<int32_t>(pieces_max, int32_t(np));
  }
  *tiles_per_slot = int32_t(std::max<int64_t>(widest, 1));
  *max_pieces = pieces_max;
  return PKV_OK;
}

int pkv_build_mixed_step(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens, int32_t num_kv_heads,
                         int32_t group, int32_t num_slots, int32_t min_piece_tokens, int32_t piece_cost_tokens,
                         int32_t chunk_slots, int32_t min_piece_tiles, int32_t* decode_rows, int32_t* num_decode,
                         int32_t* plan, int32_t plan_capacity, int32_t* tiles_per_slot, int32_t* max_pieces,
                         int32_t* items, int32_t capacity, int32_t* count, int32_t* merges, int32_t merge_capacity,
                         int32_t* merge_count, int32_t* num_partials) {
  if (num_seqs < 0 || (num_seqs > 0 && (!q_lens || !seq_lens || !decode_rows)) || !num_decode || !tiles_per_slot ||
      !max_pieces)
    return fail(PKV_ERR_INVALID, "build_mixed_step: bad arguments");
  // decode rows: the sequences with exactly one new token, in batch order
  std::vector<int32_t> lens;
  int32_t n = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (q_lens[s] != 1) continue;
    decode_rows[n++] = s;
    lens.push_back(seq_lens[s]);
  }
  *num_decode = n;
  *tiles_per_slot = 0;
  *max_pieces = 0;
  if (n > 0) {
    const int rc = pkv_build_decode_split(n, lens.data(), min_piece_tokens, piece_cost_tokens, num_slots, plan,
                                          plan_capacity, tiles_per_slot, max_pieces);
    if (rc != PKV_OK) return rc;
  }
  // the rows of sequences with two or more new tokens
  return pkv_build_chunk_work(num_seqs, q_lens, seq_lens, num_kv_heads, group, chunk_slots, min_piece_tiles, items,
                              capacity, count, merges, merge_capacity, merge_count, num_partials);
}

}  // extern "C"
