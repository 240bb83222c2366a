// Swap-out and swap-in of K/V blocks between the device cache and a host swap space.
//
// "Continuous Batching" (infra.pidoku inference notes), "5. Technical explanation",
// Preemption: the SWAP strategy copies a victim's K/V blocks to CPU memory and frees the
// GPU blocks, and copies them back when it resumes. A pair (device block b, host block
// h) moves every layer's K block b and V block b, bytes as they are in the cache.
//
// Layouts: each cache plane is [layers][num_blocks][block_bytes]; the host space is
// [host_blocks][layers][2 (K, V)][block_bytes]; the workspace stages the pairs of one
// call as [pairs][layers][2][block_bytes]. A host block is one contiguous run, so the
// PCIe leg is one DMA copy per run of consecutive host blocks (the pairs are staged in
// host-block order to make those runs long); the scattered device side is gathered or
// scattered by a copy kernel that moves 16 bytes per lane, one (pair, layer, plane)
// block per workgroup.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

using pkv::fail;

namespace {

constexpr int kIdsPerLaunch = 256;   // device block ids carried in the kernel arguments
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct SwapArgs {
  char* k;                      // cache planes (read by the gather, written by the scatter)
  char* v;
  char* staging;                // this launch's first staged pair
  int64_t block_bytes;          // multiple of 16
  int64_t layer_stride;         // num_blocks * block_bytes
  int32_t num_layers;
  int32_t num_blocks;
  int32_t ids[kIdsPerLaunch];   // device block of each staged pair
};

// One workgroup per (pair, layer, plane) block: blockIdx.x = (pair * layers + layer) * 2 + plane,
// matching the staging layout. TO_STAGING: cache -> staging (swap-out), else back.
template <bool TO_STAGING>
__global__ void __launch_bounds__(kThreads) swap_copy_kernel(SwapArgs a) {
  const int32_t c = int32_t(blockIdx.x);
  const int32_t pair = c / (2 * a.num_layers);
  const int32_t r = c - pair * 2 * a.num_layers;
  const int32_t layer = r >> 1;
  const int32_t b = a.ids[pair];
  if (b < 0 || b >= a.num_blocks) return;        // ids are checked on the host as well
  char* plane = (r & 1) ? a.v : a.k;
  uint4* cache = reinterpret_cast<uint4*>(plane + int64_t(layer) * a.layer_stride + int64_t(b) * a.block_bytes);
  uint4* stage = reinterpret_cast<uint4*>(a.staging + int64_t(c) * a.block_bytes);
  const uint4* src = TO_STAGING ? cache : stage;
  uint4* dst = TO_STAGING ? stage : cache;
  const int64_t n16 = a.block_bytes / 16;
  int64_t i = threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n16; i += kUnroll * kThreads) {
    uint4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = src[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * kThreads] = x[u];
  }
  for (; i < n16; i += kThreads) dst[i] = src[i];
}

struct Plan {
  std::vector<int32_t> order;   // pair indices sorted by host block
};

// Validate the pairs and order them by host block. Returns PKV_OK or an error.
int plan_pairs(const char* who, const int32_t* dev_blocks, const int32_t* host_blocks, int32_t n,
               int32_t num_blocks, int32_t host_capacity, Plan& p) {
  std::vector<uint8_t> seen_dev(size_t(num_blocks), 0);
  for (int32_t i = 0; i < n; ++i) {
    if (dev_blocks[i] < 0 || dev_blocks[i] >= num_blocks)
      return fail(PKV_ERR_INVALID, "%s: device block %d of pair %d outside 0..%d", who, dev_blocks[i], i,
                  num_blocks - 1);
    if (host_blocks[i] < 0 || host_blocks[i] >= host_capacity)
      return fail(PKV_ERR_INVALID, "%s: host block %d of pair %d outside 0..%d", who, host_blocks[i], i,
                  host_capacity - 1);
    if (seen_dev[size_t(dev_blocks[i])]++)
      return fail(PKV_ERR_INVALID, "%s: device block %d named twice", who, dev_blocks[i]);
  }
  p.order.resize(size_t(n));
  std::iota(p.order.begin(), p.order.end(), 0);
  std::sort(p.order.begin(), p.order.end(), [&](int32_t x, int32_t y) { return host_blocks[x] < host_blocks[y]; });
  for (int32_t i = 1; i < n; ++i)
    if (host_blocks[p.order[size_t(i)]] == host_blocks[p.order[size_t(i - 1)]])
      return fail(PKV_ERR_INVALID, "%s: host block %d named twice", who, host_blocks[p.order[size_t(i)]]);
  return PKV_OK;
}

int check_common(const char* who, const void* k, const void* v, int32_t num_layers, int32_t num_blocks,
                 int64_t block_bytes, int32_t n, const int32_t* dev_blocks, const int32_t* host_blocks,
                 const void* host_space, int32_t host_capacity, const void* workspace, int64_t workspace_bytes) {
  if (n < 0 || num_layers < 1 || num_blocks < 1 || host_capacity < 1 || block_bytes < 16 || block_bytes % 16 != 0)
    return fail(PKV_ERR_INVALID, "%s: bad sizes (block_bytes must be a positive multiple of 16)", who);
  if (n == 0) return PKV_OK;
  if (!k || !v || !dev_blocks || !host_blocks || !host_space || !workspace)
    return fail(PKV_ERR_INVALID, "%s: NULL pointer", who);
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(workspace)) % 16)
    return fail(PKV_ERR_INVALID, "%s: cache and workspace pointers must be 16-byte aligned", who);
  if (workspace_bytes < pkv_swap_workspace_bytes(n, num_layers, block_bytes))
    return fail(PKV_ERR_INVALID, "%s: workspace of %lld bytes, %lld needed", who, (long long)workspace_bytes,
                (long long)pkv_swap_workspace_bytes(n, num_layers, block_bytes));
  return PKV_OK;
}

// Launch the copy kernel over the staged pairs in `order`.
template <bool TO_STAGING>
int launch(const char* who, void* k, void* v, char* staging, int32_t num_layers, int32_t num_blocks,
           int64_t block_bytes, const int32_t* dev_blocks, const Plan& p, hipStream_t st) {
  const int64_t pair_bytes = int64_t(num_layers) * 2 * block_bytes;
  const int32_t n = int32_t(p.order.size());
  for (int32_t first = 0; first < n; first += kIdsPerLaunch) {
    const int32_t cnt = std::min(kIdsPerLaunch, n - first);
    SwapArgs a{};
    a.k = static_cast<char*>(k);
    a.v = static_cast<char*>(v);
    a.staging = staging + int64_t(first) * pair_bytes;
    a.block_bytes = block_bytes;
    a.layer_stride = int64_t(num_blocks) * block_bytes;
    a.num_layers = num_layers;
    a.num_blocks = num_blocks;
    for (int32_t i = 0; i < cnt; ++i) a.ids[i] = dev_blocks[p.order[size_t(first + i)]];
    swap_copy_kernel<TO_STAGING><<<dim3(uint32_t(cnt) * 2u * uint32_t(num_layers)), dim3(kThreads), 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  }
  return PKV_OK;
}

// One DMA copy per run of consecutive host blocks (the staging holds the pairs in
// host-block order). TO_HOST: staging -> host space, else host space -> staging.
template <bool TO_HOST>
int copy_runs(const char* who, char* host, char* staging, int64_t pair_bytes, const int32_t* host_blocks,
              const Plan& p, hipStream_t st) {
  const int32_t n = int32_t(p.order.size());
  for (int32_t i = 0; i < n;) {
    int32_t j = i + 1;
    while (j < n && host_blocks[p.order[size_t(j)]] == host_blocks[p.order[size_t(j - 1)]] + 1) ++j;
    char* h = host + int64_t(host_blocks[p.order[size_t(i)]]) * pair_bytes;
    char* s = staging + int64_t(i) * pair_bytes;
    const size_t bytes = size_t(int64_t(j - i) * pair_bytes);
    const hipError_t e = TO_HOST ? hipMemcpyAsync(h, s, bytes, hipMemcpyDeviceToHost, st)
                                 : hipMemcpyAsync(s, h, bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: copy failed: %s", who, hipGetErrorString(e));
    i = j;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int64_t pkv_swap_workspace_bytes(int32_t n, int32_t num_layers, int64_t block_bytes) {
  if (n <= 0 || num_layers <= 0 || block_bytes <= 0) return 0;
  return int64_t(n) * num_layers * 2 * block_bytes;
}

int pkv_swap_out(const void* k_cache, const void* v_cache, int32_t num_layers, int32_t num_blocks,
                 int64_t block_bytes, const int32_t* dev_blocks, const int32_t* host_blocks, int32_t n,
                 void* host_space, int32_t host_capacity, void* workspace, int64_t workspace_bytes, void* stream,
                 void* copy_stream) {
  const char* who = "swap_out";
  int rc = check_common(who, k_cache, v_cache, num_layers, num_blocks, block_bytes, n, dev_blocks, host_blocks,
                        host_space, host_capacity, workspace, workspace_bytes);
  if (rc != PKV_OK || n == 0) return rc;
  Plan p;
  rc = plan_pairs(who, dev_blocks, host_blocks, n, num_blocks, host_capacity, p);
  if (rc != PKV_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* staging = static_cast<char*>(workspace);
  rc = launch<true>(who, const_cast<void*>(k_cache), const_cast<void*>(v_cache), staging, num_layers, num_blocks,
                    block_bytes, dev_blocks, p, st);
  if (rc != PKV_OK) return rc;
  // the device blocks are free for reuse on `stream` once the gather is done; the PCIe leg
  // may run on a copy stream that waits for the gather only
  hipStream_t cs = copy_stream ? reinterpret_cast<hipStream_t>(copy_stream) : st;
  if (cs != st) {
    hipEvent_t ev;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: event creation failed: %s", who, hipGetErrorString(e));
    e = hipEventRecord(ev, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, ev, 0);
    hipEventDestroy(ev);                   // released once the recorded work completes
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: stream ordering failed: %s", who, hipGetErrorString(e));
  }
  return copy_runs<true>(who, static_cast<char*>(host_space), staging, int64_t(num_layers) * 2 * block_bytes,
                         host_blocks, p, cs);
}

int pkv_swap_in(void* k_cache, void* v_cache, int32_t num_layers, int32_t num_blocks, int64_t block_bytes,
                const int32_t* host_blocks, const int32_t* dev_blocks, int32_t n, const void* host_space,
                int32_t host_capacity, void* workspace, int64_t workspace_bytes, void* stream) {
  const char* who = "swap_in";
  int rc = check_common(who, k_cache, v_cache, num_layers, num_blocks, block_bytes, n, dev_blocks, host_blocks,
                        host_space, host_capacity, workspace, workspace_bytes);
  if (rc != PKV_OK || n == 0) return rc;
  Plan p;
  rc = plan_pairs(who, dev_blocks, host_blocks, n, num_blocks, host_capacity, p);
  if (rc != PKV_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* staging = static_cast<char*>(workspace);
  rc = copy_runs<false>(who, const_cast<char*>(static_cast<const char*>(host_space)), staging,
                        int64_t(num_layers) * 2 * block_bytes, host_blocks, p, st);
  if (rc != PKV_OK) return rc;
  return launch<false>(who, k_cache, v_cache, staging, num_layers, num_blocks, block_bytes, dev_blocks, p, st);
}

}  // extern "C"
