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
  std::unordered_map<int64_t, std::vector<int32_t>> tables;
};
