// The host pool's state, shared by the pool entry points (host.cpp) and the scheduler
// step (sched.cpp). Host-only C++; not part of the C ABI.
#pragma once

#include <cstdint>
#include <unordered_map>
#include <vector>

enum : uint8_t { kFree = 0, kRaw = 1, kInSeq = 2 };

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;        // next pop = back()
  std::vector<uint8_t> state;            // per id: kFree / kRaw / kInSeq
  std::vector<int32_t> ref;              // per id in tables: the tables holding it
  std::vector<uint32_t> gen;             // per id: frees from tables so far
  std::unordered_map<int64_t, std::vector<int32_t>> tables;
};

namespace pkv {
// Grow id's table to ceil(tokens / block_size) blocks, all-or-nothing: false (nothing
// changed) when too few blocks are free. New blocks are held once.
bool pool_reserve(pkv_pool* p, int64_t id, int64_t tokens);
// Drop id's table: each block loses a reference; those left with none go back to the
// free list in table order. No-op for an unknown id.
void pool_release(pkv_pool* p, int64_t id);
// Start id's (empty or missing) table with blocks held by other tables, one more
// reference each.
void pool_share(pkv_pool* p, int64_t id, const int32_t* blocks, int32_t n);
}  // namespace pkv
