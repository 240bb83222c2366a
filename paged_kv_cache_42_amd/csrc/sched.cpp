// Host scheduler step of continuous batching, on top of the block pool.
//
// The loop is the engine step of "Continuous Batching" (infra.pidoku inference notes),
// section "4. Tiny example" (admit from the head of the waiting queue while a slot
// and the blocks are free, stopping at the first request that does not fit; run one
// mixed forward pass over every running request; then, in running order, append one
// output token, free a finished request's blocks at once, give a request that needs one
// a new block, and preempt it to the front of the queue when none is left), with the
// recompute preemption of "5. Technical explanation". Readings where the page leaves a
// step open: blocks at admission cover prompt + outputs so far (a preempted request
// re-prefills both); a prefill row holds those tokens at positions 0..; a decode row is
// the last output token; a request finishes at its output count; arrivals join the
// back of the queue at the start of their step in (arrival, id) order.
//
// Chunked prefill (the mixed batching of "5. Technical explanation", off by default): a
// step carries at most max_batched_tokens new tokens. Decode rows are never cut; the rest
// of the budget goes to prefill rows in running order, each taking the least of its
// uncomputed context, chunk_tokens and what is left, so a request may get no row. A
// request produces its first output at the step of its last chunk.
//
// Preemption by swap (the SWAP strategy of "5. Technical explanation", off by default):
// a victim's blocks go, in table order, to host blocks popped from a host free list, its
// device blocks are freed, and it waits at the front of the queue; when the host space
// is short it is preempted by recompute. Re-admitted, it gets blocks for prompt +
// outputs, its host blocks are copied back into the first of them and freed in table
// order, and it resumes with a decode row. The copies are listed per call: swap-outs by
// the update, swap-ins by the schedule.
//
// Policy variants ("5. Technical explanation": victim selection and admission policies):
// with the LIFO or fewest-generated victim policy the update first appends every row's
// output and retires finished requests, then gives each running request (in order) the
// block its next token needs, preempting victims until it gets one: the last admitted,
// or the one with the fewest outputs (earliest admitted on ties), among the least
// important priority class present, the request itself included. With priority classes
// the waiting queue is ordered by (class, arrival, id), preempted requests included.
//
// Static batching (the baseline of "1. What is it?": decide a batch, run it to
// completion): admission only at a step that starts with nothing running.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <tuple>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"
#include "pool_internal.h"

using pkv::fail;

namespace {

enum : int32_t { kPrefill = 0, kDecode = 1 };

struct Req {
  int64_t id;
  int32_t arrival, prompt, max_tokens;
  int32_t n_out = 0;
  int32_t stage = kPrefill;
  int32_t cached = 0;                  // prompt tokens of this prefill found in the cache
  int32_t done = 0;                    // context tokens of the current prefill computed so far
  int32_t q_step = 0;                  // new tokens of its row in the scheduled step (0: no row)
  int32_t prio = 0;                    // priority class, 0 most important
  bool swapped = false;                // its K/V waits in `host`
  std::vector<int32_t> host;           // host blocks holding its swapped-out K/V, in table order
  std::vector<int32_t> tokens;         // prompt token ids (prefix caching), else empty
};

using pkv::pool_release;
using pkv::pool_reserve;

// 64-bit mix (SplitMix64 finaliser) for the prefix keys.
uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Prefix cache ([P17] "Step 8: Prefix caching"): page-aligned prompt prefix -> the pages
// holding it. Keys chain a hash over whole pages; a hit is confirmed token by token
// against the request that registered the entry. An entry is usable while each of its
// blocks is still held and has not been freed since (generation unchanged).
struct PrefixEntry {
  int32_t owner;                       // request (index) whose tokens the key covers
  int32_t n_tokens;
  std::vector<std::pair<int32_t, uint32_t>> pages;   // (block, generation)
};

}  // namespace


struct pkv_sched {
  pkv_pool* pool = nullptr;
  int32_t max_running = 0;
  std::vector<Req> reqs;
  std::vector<int32_t> arrival_order;   // indices into reqs, by (arrival, id)
  size_t next_arrival = 0;
  std::deque<int32_t> waiting;
  std::vector<int32_t> running;
  int64_t step = 0;
  int64_t preempted = 0;
  int64_t finished = 0;
  bool scheduled = false;               // schedule() done, update() pending
  bool admission_check = true;          // false: admit without checking for free blocks
  bool prefix_cache = false;
  std::unordered_map<uint64_t, PrefixEntry> cache;
  std::unordered_map<int64_t, int32_t> index;   // request id -> index in reqs
  int64_t cached_tokens = 0;
  int32_t max_batched_tokens = 0;       // 0: no per-step token budget
  int32_t chunk_tokens = 0;             // 0: prefills are not cut into chunks
  std::vector<int32_t> rows;            // running requests with a row this step, in running order
  bool swap = false;                    // preemption by swap into the host space
  int32_t host_blocks = 0;
  std::vector<int32_t> host_free;       // LIFO free list of host blocks
  std::vector<int32_t> swap_out;        // (device, host) pairs of the last update
  std::vector<int32_t> swap_in;         // (host, device) pairs of the last schedule
  int64_t swapped_out = 0, blocks_out = 0, blocks_in = 0;
  int32_t victim = PKV_VICTIM_SELF;
  bool by_priority = false;
  bool static_batching = false;

  // waiting queue insertion: the back (arrivals) or front (preempted), or by
  // (class, arrival, id) with priority classes
  void enqueue(int32_t i, bool front) {
    if (!by_priority) {
      if (front) waiting.push_front(i);
      else waiting.push_back(i);
      return;
    }
    auto key = [&](int32_t j) { const Req& r = reqs[size_t(j)]; return std::make_tuple(r.prio, r.arrival, r.id); };
    auto it = waiting.begin();
    while (it != waiting.end() && key(*it) < key(i)) ++it;
    waiting.insert(it, i);
  }
  // preempt by swap when the host space holds the whole table, else by recompute
  void preempt(int32_t i) {
    Req& r = reqs[size_t(i)];
    const std::vector<int32_t>& t = pool->tables.at(r.id);
    if (swap && host_free.size() >= t.size()) {
      r.host.clear();
      for (int32_t b : t) {
        r.host.push_back(host_free.back());
        host_free.pop_back();
        swap_out.push_back(b);
        swap_out.push_back(r.host.back());
      }
      r.swapped = true;
      ++swapped_out;
      blocks_out += int64_t(t.size());
    }
    pool_release(pool, r.id);
    ++preempted;
    enqueue(i, true);
  }
  // victim among `alive` (running order) by the policy
  size_t pick_victim(const std::vector<int32_t>& alive) const {
    int32_t worst = 0;
    for (int32_t j : alive) worst = std::max(worst, reqs[size_t(j)].prio);
    size_t best = alive.size();
    for (size_t k = 0; k < alive.size(); ++k) {
      const Req& c = reqs[size_t(alive[k])];
      if (c.prio != worst) continue;
      if (victim == PKV_VICTIM_LIFO) best = k;                       // the last one
      else if (best == alive.size() || c.n_out < reqs[size_t(alive[best])].n_out) best = k;   // first minimum
    }
    return best;
  }

  // page-chained keys of tokens[0 : k * bs] for k = 1..pages
  std::vector<uint64_t> page_keys(const std::vector<int32_t>& tok, int64_t pages) const {
    std::vector<uint64_t> keys(size_t(std::max<int64_t>(pages, 0)));
    uint64_t h = 0x9E3779B97F4A7C15ull;
    const int64_t bs = pool->block_size;
    for (int64_t k = 0; k < pages; ++k) {
      for (int64_t i = k * bs; i < (k + 1) * bs; ++i) h = mix64(h ^ (uint64_t(uint32_t(tok[size_t(i)])) + 0x632BE59BD9B4E019ull));
      keys[size_t(k)] = h;
    }
    return keys;
  }
  bool valid(const PrefixEntry& e) const {
    for (const auto& pg : e.pages)
      if (pool->ref[pg.first] < 1 || pool->gen[pg.first] != pg.second) return false;
    return true;
  }
  // longest cached whole-page prefix of r's prompt within `limit` tokens
  int32_t lookup(const Req& r, int64_t limit, std::vector<int32_t>& pages) const {
    pages.clear();
    const int64_t bs = pool->block_size;
    const int64_t kmax = std::min<int64_t>(limit, int64_t(r.tokens.size())) / bs;
    const std::vector<uint64_t> keys = page_keys(r.tokens, kmax);
    for (int64_t k = kmax; k >= 1; --k) {
      auto it = cache.find(keys[size_t(k - 1)]);
      if (it == cache.end() || it->second.n_tokens != k * bs || !valid(it->second)) continue;
      const std::vector<int32_t>& ot = reqs[size_t(it->second.owner)].tokens;
      if (!std::equal(r.tokens.begin(), r.tokens.begin() + k * bs, ot.begin())) continue;   // hash collision
      for (const auto& pg : it->second.pages) pages.push_back(pg.first);
      return int32_t(k * bs);
    }
    return 0;
  }
  // register the whole pages of r's prompt (held by its table) that have no usable entry
  void insert(int32_t ri) {
    const Req& r = reqs[size_t(ri)];
    const int64_t bs = pool->block_size;
    const int64_t pages = int64_t(r.tokens.size()) / bs;
    const std::vector<uint64_t> keys = page_keys(r.tokens, pages);
    const std::vector<int32_t>& t = pool->tables.at(r.id);
    for (int64_t k = 1; k <= pages; ++k) {
      auto it = cache.find(keys[size_t(k - 1)]);
      if (it != cache.end() && valid(it->second)) continue;
      PrefixEntry e{ri, int32_t(k * bs), {}};
      for (int64_t j = 0; j < k; ++j) e.pages.emplace_back(t[size_t(j)], pool->gen[t[size_t(j)]]);
      cache[keys[size_t(k - 1)]] = std::move(e);
    }
  }
};

extern "C" {

int pkv_sched_create(pkv_pool* pool, int32_t max_running, pkv_sched** out) {
  if (!pool || !out || max_running < 1) return fail(PKV_ERR_INVALID, "sched_create: bad arguments");
  auto* s = new pkv_sched();
  s->pool = pool;
  s->max_running = max_running;
  *out = s;
  return PKV_OK;
}

void pkv_sched_destroy(pkv_sched* s) { delete s; }

int pkv_sched_add_requests(pkv_sched* s, int32_t n, const int64_t* ids, const int32_t* arrival,
                           const int32_t* prompt, const int32_t* max_tokens) {
  if (!s || n < 0 || (n > 0 && (!ids || !arrival || !prompt || !max_tokens)))
    return fail(PKV_ERR_INVALID, "sched_add_requests: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    if (prompt[i] < 1 || max_tokens[i] < 1 || arrival[i] < 0)
      return fail(PKV_ERR_INVALID, "sched_add_requests: request %lld needs prompt >= 1, max_tokens >= 1, "
                  "arrival >= 0", (long long)ids[i]);
    if (arrival[i] < s->step)
      return fail(PKV_ERR_INVALID, "sched_add_requests: request %lld arrives at step %d, before the current "
                  "step %lld", (long long)ids[i], arrival[i], (long long)s->step);
    const int64_t blocks = (int64_t(prompt[i]) + max_tokens[i] - 1 + s->pool->block_size - 1) / s->pool->block_size;
    if (blocks > s->pool->num_blocks)
      return fail(PKV_ERR_INVALID, "sched_add_requests: request %lld can need %lld blocks, the pool has %d",
                  (long long)ids[i], (long long)blocks, s->pool->num_blocks);
    if (s->pool->tables.count(ids[i]))
      return fail(PKV_ERR_INVALID, "sched_add_requests: id %lld already holds a table", (long long)ids[i]);
  }
  for (const Req& r : s->reqs)
    for (int32_t i = 0; i < n; ++i)
      if (r.id == ids[i]) return fail(PKV_ERR_INVALID, "sched_add_requests: id %lld repeated", (long long)ids[i]);
  for (int32_t i = 0; i < n; ++i) {
    for (int32_t j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return fail(PKV_ERR_INVALID, "sched_add_requests: id %lld repeated", (long long)ids[i]);
  }
  for (int32_t i = 0; i < n; ++i) {
    s->reqs.push_back(Req{ids[i], arrival[i], prompt[i], max_tokens[i]});
    s->arrival_order.push_back(int32_t(s->reqs.size() - 1));
    s->index[ids[i]] = int32_t(s->reqs.size() - 1);
  }
  // requests not yet arrived are kept sorted by (arrival, id)
  std::sort(s->arrival_order.begin() + s->next_arrival, s->arrival_order.end(), [&](int32_t a, int32_t b) {
    const Req &x = s->reqs[a], &y = s->reqs[b];
    return x.arrival != y.arrival ? x.arrival < y.arrival : x.id < y.id;
  });
  return PKV_OK;
}

int pkv_sched_schedule(pkv_sched* s, int32_t* num_rows, int32_t* total_q, int32_t* max_blocks) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_schedule: scheduler is NULL");
  if (s->scheduled) return fail(PKV_ERR_INVALID, "sched_schedule: the previous step was not updated");
  // arrivals
  while (s->next_arrival < s->arrival_order.size()) {
    const int32_t i = s->arrival_order[s->next_arrival];
    if (s->reqs[i].arrival > s->step) break;
    s->enqueue(i, false);
    ++s->next_arrival;
  }
  // strict first-come-first-served admission
  std::vector<int32_t> pages;
  s->swap_in.clear();
  const bool admit = !(s->static_batching && !s->running.empty());
  while (admit && !s->waiting.empty() && int32_t(s->running.size()) < s->max_running) {
    const int32_t head = s->waiting.front();
    Req& r = s->reqs[head];
    const int64_t ctx = int64_t(r.prompt) + r.n_out;
    if (r.swapped) {                      // its K/V comes back from the host: no prefill
      const int64_t need = (ctx + s->pool->block_size - 1) / s->pool->block_size;
      if (s->admission_check && need > int64_t(s->pool->free_list.size())) break;
      s->waiting.pop_front();
      if (!pool_reserve(s->pool, r.id, ctx))
        return fail(PKV_ERR_OUT_OF_BLOCKS, "sched_schedule: step %lld, request %lld does not fit and admission "
                    "does not check", (long long)s->step, (long long)r.id);
      const std::vector<int32_t>& t = s->pool->tables.at(r.id);
      for (size_t j = 0; j < r.host.size(); ++j) {
        s->swap_in.push_back(r.host[j]);
        s->swap_in.push_back(t[j]);
        s->host_free.push_back(r.host[j]);
      }
      s->blocks_in += int64_t(r.host.size());
      r.host.clear();
      r.swapped = false;                  // resumes in its stage
      s->running.push_back(head);
      continue;
    }
    // longest cached prefix; a fresh request computes at least its last prompt token
    const int32_t hit = s->prefix_cache && !r.tokens.empty()
                            ? s->lookup(r, std::min<int64_t>(r.prompt, ctx - 1), pages)
                            : (pages.clear(), 0);
    const int64_t need = (ctx + s->pool->block_size - 1) / s->pool->block_size - int64_t(pages.size());
    if (s->admission_check && need > int64_t(s->pool->free_list.size())) break;   // strict FCFS
    s->waiting.pop_front();
    if (!pages.empty()) pkv::pool_share(s->pool, r.id, pages.data(), int32_t(pages.size()));
    if (!pool_reserve(s->pool, r.id, ctx))    // only without the admission check
      return fail(PKV_ERR_OUT_OF_BLOCKS, "sched_schedule: step %lld, request %lld does not fit and admission "
                  "does not check", (long long)s->step, (long long)r.id);
    r.stage = kPrefill;
    r.cached = hit;
    r.done = hit;
    s->cached_tokens += hit;
    s->running.push_back(head);
  }
  // new tokens per running request: decode rows first, then prefill chunks in running
  // order within what the budget leaves
  int64_t left = INT64_MAX;
  if (s->max_batched_tokens > 0) {
    int64_t decodes = 0;
    for (int32_t i : s->running) decodes += s->reqs[i].stage == kDecode;
    left = std::max<int64_t>(0, s->max_batched_tokens - decodes);
  }
  s->rows.clear();
  int64_t q = 0, mb = 0;
  for (int32_t i : s->running) {
    Req& r = s->reqs[i];
    const int64_t ctx = int64_t(r.prompt) + r.n_out;
    int64_t qi = 1, len = ctx;
    if (r.stage == kPrefill) {
      qi = ctx - r.done;
      if (s->chunk_tokens > 0) qi = std::min<int64_t>(qi, s->chunk_tokens);
      qi = std::min(qi, left);
      left -= qi;
      len = r.done + qi;
    }
    r.q_step = int32_t(qi);
    if (qi == 0) continue;                // no row this step
    s->rows.push_back(i);
    q += qi;
    mb = std::max<int64_t>(mb, (len + s->pool->block_size - 1) / s->pool->block_size);
  }
  s->scheduled = true;
  if (num_rows) *num_rows = int32_t(s->rows.size());
  if (total_q) *total_q = int32_t(q);
  if (max_blocks) *max_blocks = int32_t(mb);
  return PKV_OK;
}

int pkv_sched_plan(const pkv_sched* s, int32_t table_width, int64_t* ids, int32_t* stages, int32_t* q_lens,
                   int32_t* seq_lens, int32_t* block_tables, int32_t* cu_seqlens_q, int64_t* slot_mapping) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_plan: scheduler is NULL");
  if (!s->scheduled) return fail(PKV_ERR_INVALID, "sched_plan: no step scheduled");
  const int32_t n = int32_t(s->rows.size());
  if (n > 0 && (!ids || !stages || !q_lens || !seq_lens))
    return fail(PKV_ERR_INVALID, "sched_plan: NULL row array");
  for (int32_t k = 0; k < n; ++k) {
    const Req& r = s->reqs[s->rows[k]];
    ids[k] = r.id;
    stages[k] = r.stage;
    q_lens[k] = r.q_step;
    seq_lens[k] = r.stage == kPrefill ? r.done + r.q_step : r.prompt + r.n_out;
  }
  return pkv_build_block_table(s->pool, n, ids, q_lens, seq_lens, table_width, block_tables, cu_seqlens_q,
                               slot_mapping);
}

namespace {

// the update of the LIFO / fewest-generated victim policies: outputs and retirements
// first, then the blocks for the next tokens in running order
int update_with_victims(pkv_sched* s) {
  std::vector<int32_t> alive;
  std::vector<uint8_t> grew;
  alive.reserve(s->running.size());
  for (int32_t i : s->running) {
    Req& r = s->reqs[i];
    const bool had_row = r.q_step > 0;
    r.q_step = 0;
    if (!had_row || (r.stage == kPrefill && r.done < r.prompt + r.n_out)) {
      alive.push_back(i);
      grew.push_back(0);
      continue;
    }
    r.cached = 0;
    r.n_out += 1;
    r.stage = kDecode;
    if (r.n_out >= r.max_tokens) {
      pool_release(s->pool, r.id);
      ++s->finished;
      continue;
    }
    alive.push_back(i);
    grew.push_back(1);
  }
  size_t k = 0;
  while (k < alive.size()) {
    const int32_t i = alive[k];
    const Req& r = s->reqs[size_t(i)];
    const int64_t need = int64_t(r.prompt) + r.n_out;
    bool self_preempted = false;
    if (grew[k]) {
      while (!pool_reserve(s->pool, r.id, need)) {
        const size_t v = s->pick_victim(alive);
        const int32_t vi = alive[v];
        alive.erase(alive.begin() + std::ptrdiff_t(v));
        grew.erase(grew.begin() + std::ptrdiff_t(v));
        if (v < k) --k;
        s->preempt(vi);
        if (vi == i) {
          self_preempted = true;
          break;
        }
      }
    }
    if (!self_preempted) ++k;
  }
  s->running.swap(alive);
  s->rows.clear();
  s->scheduled = false;
  ++s->step;
  return PKV_OK;
}

}  // namespace

int pkv_sched_update(pkv_sched* s) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_update: scheduler is NULL");
  if (!s->scheduled) return fail(PKV_ERR_INVALID, "sched_update: no step scheduled");
  s->swap_out.clear();
  for (int32_t i : s->running) {
    Req& r = s->reqs[i];
    if (r.stage == kPrefill) r.done += r.q_step;
  }
  if (s->prefix_cache)                  // prefills completed this step: their prompt pages
    for (int32_t i : s->running) {
      const Req& r = s->reqs[i];
      if (r.stage == kPrefill && r.done == r.prompt + r.n_out && !r.tokens.empty()) s->insert(i);
    }
  if (s->victim != PKV_VICTIM_SELF) return update_with_victims(s);
  std::vector<int32_t> still;
  still.reserve(s->running.size());
  for (int32_t i : s->running) {
    Req& r = s->reqs[i];
    const bool had_row = r.q_step > 0;
    r.q_step = 0;
    if (!had_row || (r.stage == kPrefill && r.done < r.prompt + r.n_out)) {
      still.push_back(i);                 // no output this step
      continue;
    }
    r.cached = 0;
    r.n_out += 1;
    r.stage = kDecode;
    if (r.n_out >= r.max_tokens) {            // finished: blocks freed at once
      pool_release(s->pool, r.id);
      ++s->finished;
      continue;
    }
    const int64_t need = int64_t(r.prompt) + r.n_out;   // tokens the next row writes up to
    if (!pool_reserve(s->pool, r.id, need)) {  // no block for the next token: it preempts itself
      s->preempt(i);
      continue;
    }
    still.push_back(i);
  }
  s->running.swap(still);
  s->rows.clear();
  s->scheduled = false;
  ++s->step;
  return PKV_OK;
}

int pkv_sched_set_admission_check(pkv_sched* s, int32_t enabled) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_set_admission_check: scheduler is NULL");
  s->admission_check = enabled != 0;
  return PKV_OK;
}

int pkv_sched_set_token_budget(pkv_sched* s, int32_t max_batched_tokens, int32_t chunk_tokens) {
  if (!s || max_batched_tokens < 0 || chunk_tokens < 0)
    return fail(PKV_ERR_INVALID, "sched_set_token_budget: bad arguments");
  if (s->step > 0 || s->scheduled)
    return fail(PKV_ERR_INVALID, "sched_set_token_budget: call before the first step");
  s->max_batched_tokens = max_batched_tokens;
  s->chunk_tokens = chunk_tokens;
  return PKV_OK;
}

int pkv_sched_set_static_batching(pkv_sched* s, int32_t enabled) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_set_static_batching: scheduler is NULL");
  if (s->step > 0 || s->scheduled)
    return fail(PKV_ERR_INVALID, "sched_set_static_batching: call before the first step");
  s->static_batching = enabled != 0;
  return PKV_OK;
}

int pkv_sched_set_victim_policy(pkv_sched* s, int32_t policy) {
  if (!s || policy < PKV_VICTIM_SELF || policy > PKV_VICTIM_FEWEST)
    return fail(PKV_ERR_INVALID, "sched_set_victim_policy: bad arguments");
  if (s->step > 0 || s->scheduled)
    return fail(PKV_ERR_INVALID, "sched_set_victim_policy: call before the first step");
  s->victim = policy;
  return PKV_OK;
}

int pkv_sched_set_priorities(pkv_sched* s, int32_t n, const int64_t* ids, const int32_t* classes) {
  if (!s || n < 0 || (n > 0 && (!ids || !classes))) return fail(PKV_ERR_INVALID, "sched_set_priorities: bad arguments");
  if (s->step > 0 || s->scheduled)
    return fail(PKV_ERR_INVALID, "sched_set_priorities: call before the first step");
  for (int32_t k = 0; k < n; ++k) {
    if (classes[k] < 0) return fail(PKV_ERR_INVALID, "sched_set_priorities: class %d < 0", classes[k]);
    if (!s->index.count(ids[k]))
      return fail(PKV_ERR_INVALID, "sched_set_priorities: unknown request %lld", (long long)ids[k]);
  }
  for (int32_t k = 0; k < n; ++k) s->reqs[size_t(s->index.at(ids[k]))].prio = classes[k];
  s->by_priority = true;
  return PKV_OK;
}

int pkv_sched_enable_swap(pkv_sched* s, int32_t host_blocks) {
  if (!s || host_blocks < 1) return fail(PKV_ERR_INVALID, "sched_enable_swap: bad arguments");
  if (s->step > 0 || s->scheduled) return fail(PKV_ERR_INVALID, "sched_enable_swap: call before the first step");
  s->swap = true;
  s->host_blocks = host_blocks;
  s->host_free.resize(size_t(host_blocks));
  for (int32_t i = 0; i < host_blocks; ++i) s->host_free[size_t(i)] = i;
  return PKV_OK;
}

int pkv_sched_swap_pairs(const pkv_sched* s, int32_t* num_out, int32_t* num_in, int32_t* out_pairs,
                         int32_t* in_pairs) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_swap_pairs: scheduler is NULL");
  if (num_out) *num_out = int32_t(s->swap_out.size() / 2);
  if (num_in) *num_in = int32_t(s->swap_in.size() / 2);
  if (out_pairs) std::copy(s->swap_out.begin(), s->swap_out.end(), out_pairs);
  if (in_pairs) std::copy(s->swap_in.begin(), s->swap_in.end(), in_pairs);
  return PKV_OK;
}

int pkv_sched_swap_counters(const pkv_sched* s, int64_t* out) {
  if (!s || !out) return fail(PKV_ERR_INVALID, "sched_swap_counters: bad arguments");
  out[0] = s->swapped_out;
  out[1] = s->blocks_out;
  out[2] = s->blocks_in;
  out[3] = int64_t(s->host_free.size());
  return PKV_OK;
}

int pkv_sched_counters(const pkv_sched* s, int64_t* out) {
  if (!s || !out) return fail(PKV_ERR_INVALID, "sched_counters: bad arguments");
  out[0] = s->step;
  out[1] = int64_t(s->pool->free_list.size());
  out[2] = int64_t(s->running.size());
  out[3] = int64_t(s->waiting.size());
  out[4] = s->preempted;
  out[5] = s->finished;
  out[6] = int64_t(s->reqs.size());
  out[7] = s->cached_tokens;
  return PKV_OK;
}

int pkv_sched_enable_prefix_cache(pkv_sched* s) {
  if (!s) return fail(PKV_ERR_INVALID, "sched_enable_prefix_cache: scheduler is NULL");
  if (s->step > 0 || s->scheduled)
    return fail(PKV_ERR_INVALID, "sched_enable_prefix_cache: call before the first step");
  s->prefix_cache = true;
  return PKV_OK;
}

int pkv_sched_set_prompt_tokens(pkv_sched* s, int64_t id, const int32_t* tokens, int32_t n) {
  if (!s || n < 0 || (n > 0 && !tokens)) return fail(PKV_ERR_INVALID, "sched_set_prompt_tokens: bad arguments");
  auto it = s->index.find(id);
  if (it == s->index.end())
    return fail(PKV_ERR_INVALID, "sched_set_prompt_tokens: unknown request %lld", (long long)id);
  Req& r = s->reqs[size_t(it->second)];
  if (n != r.prompt)
    return fail(PKV_ERR_INVALID, "sched_set_prompt_tokens: request %lld has a %d-token prompt, %d tokens given",
                (long long)id, r.prompt, n);
  if (s->step > 0 || s->scheduled)
    return fail(PKV_ERR_INVALID, "sched_set_prompt_tokens: call before the first step");
  r.tokens.assign(tokens, tokens + n);
  return PKV_OK;
}

}  // extern "C"
