// pkv_paged_attention_decode_split_noalloc: the balanced-split decode for callers that
// cannot allocate device memory, its split partials kept in a device array of this file.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

// The partials live in this file's device array `scratch` (one copy per device, held
// until the process ends). Host code never passes the array's name to a kernel (on the
// host it only names a stand-in): the device address comes from hipGetSymbolAddress,
// once per device, and only that address is handed on.
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
int scratch_on_current_device(void** out) {
  using pkv::fail;
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return fail(PKV_ERR_HIP, "decode_split_noalloc: hipGetDevice: %s", hipGetErrorString(ge));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "decode_split_noalloc: device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "decode_split_noalloc: hipGetSymbolAddress on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" size_t pkv_decode_split_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int pkv_paged_attention_decode_split_noalloc(
    void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache, int32_t cache_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_seq_len, float scale, float k_scale, float v_scale, const float* k_head_scales,
    const float* v_head_scales, const int32_t* rows, int32_t num_rows, const int32_t* cu_seqlens_q, int32_t total_q,
    const int32_t* plan, int32_t num_slots, int32_t tiles_per_slot, int32_t max_pieces, float* lse_out,
    void* stream) {
  using pkv::fail;
  const size_t need = pkv_decode_split_workspace_bytes(num_slots, num_q_heads, head_dim, max_pieces);
  if (need > kNoAllocScratchBytes)
    return fail(PKV_ERR_INVALID,
                "decode_split_noalloc: %zu bytes of partials (%d slots x %d heads x head_dim %d) exceed the "
                "%zu-byte device scratch; use pkv_paged_attention_decode_split with a workspace",
                need, num_slots, num_q_heads, head_dim, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_on_current_device(&ws);
    if (rc != PKV_OK) return rc;
  }
  return pkv::decode_split(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, table_width,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                           k_scale, v_scale, k_head_scales, v_head_scales, rows, num_rows, cu_seqlens_q, total_q,
                           plan, num_slots, tiles_per_slot, max_pieces, ws, need > 0 ? kNoAllocScratchBytes : 0,
                           lse_out, pkv::Layers{}, stream);
}
