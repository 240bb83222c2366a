// kv_cache_write: scatter this step's new K/V rows into their cache slots.
//
// "Project 17: Production Serving: Continuous Batching and PagedAttention", "Step 4:
// Implement the paged KV cache": a token's K and V go to slot (length % page size) of
// its page. Here the host has already resolved every new token to a flat slot
// (slot_mapping); the kernel is a coalesced scatter copy. With the cache layout
// [block][slot][kv_head][d], one token's Hkv*d elements are contiguous in the input
// and in the cache, so each lane moves 16 contiguous bytes of input.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

using pkv::f32_to_bf16;
using pkv::f32_to_fp8;

// Layer blockIdx.y of a layer-batched launch: inputs in_ls bytes apart, planes cache_ls.
template <typename T>
__device__ __forceinline__ T* at_layer(T* p, int64_t ls) {
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(p) + uintptr_t(int64_t(blockIdx.y) * ls));
}

// Same dtype: bit copy, one uint4 (16 B) per lane.
__global__ void __launch_bounds__(256) write_copy16(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                    uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                    const int64_t* __restrict__ slots, int64_t num_tokens,
                                                    int64_t chunks_per_row, int64_t num_slots, int64_t in_ls,
                                                    int64_t cache_ls) {
  k = at_layer(k, in_ls);
  v = at_layer(v, in_ls);
  kc = at_layer(kc, cache_ls);
  vc = at_layer(vc, cache_ls);
  const int64_t total = num_tokens * chunks_per_row;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t tok = i / chunks_per_row;
    const int64_t c = i - tok * chunks_per_row;
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t dst = slot * chunks_per_row + c;
    kc[dst] = k[i];
    vc[dst] = v[i];
  }
}

// Inverse scales per KV head (every slot equal without per-head factors).
struct InvScales {
  float k[pkv::kHeadScales];
  float v[pkv::kHeadScales];
};

// To E4M3: 8 input elements (16 B of bf16 or 32 B of f32) -> 8 code bytes per lane;
// chunk c of a token row belongs to KV head c / chunks_per_head.
template <bool IN_BF16>
__global__ void __launch_bounds__(256) write_fp8(const void* __restrict__ k_, const void* __restrict__ v_,
                                                 uint2* __restrict__ kc, uint2* __restrict__ vc,
                                                 const int64_t* __restrict__ slots, int64_t num_tokens,
                                                 int64_t chunks_per_row, int64_t num_slots,
                                                 int64_t chunks_per_head, InvScales inv, int64_t in_ls,
                                                 int64_t cache_ls) {
  k_ = at_layer(k_, in_ls);
  v_ = at_layer(v_, in_ls);
  kc = at_layer(kc, cache_ls);
  vc = at_layer(vc, cache_ls);
  const int64_t total = num_tokens * chunks_per_row;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t tok = i / chunks_per_row;
    const int64_t c = i - tok * chunks_per_row;
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;
    float kx[8], vx[8];
    if constexpr (IN_BF16) {
      const uint4 a = reinterpret_cast<const uint4*>(k_)[i];
      const uint4 b = reinterpret_cast<const uint4*>(v_)[i];
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
      const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kx[2 * j] = pkv::bf16_lo(aw[j]);
        kx[2 * j + 1] = pkv::bf16_hi(aw[j]);
        vx[2 * j] = pkv::bf16_lo(bw[j]);
        vx[2 * j + 1] = pkv::bf16_hi(bw[j]);
      }
    } else {
      const float4* kf = reinterpret_cast<const float4*>(k_) + 2 * i;
      const float4* vf = reinterpret_cast<const float4*>(v_) + 2 * i;
      const float4 a0 = kf[0], a1 = kf[1], b0 = vf[0], b1 = vf[1];
      const float ka[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float va[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        kx[j] = ka[j];
        vx[j] = va[j];
      }
    }
    const int64_t hh = c / chunks_per_head;
    const int h = hh < pkv::kHeadScales ? int(hh) : pkv::kHeadScales - 1;
    const float k_inv = inv.k[h];
    const float v_inv = inv.v[h];
    uint32_t kw[2] = {0, 0}, vw[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kw[j >> 2] |= f32_to_fp8(kx[j] * k_inv) << (8 * (j & 3));
      vw[j >> 2] |= f32_to_fp8(vx[j] * v_inv) << (8 * (j & 3));
    }
    const int64_t dst = slot * chunks_per_row + c;
    kc[dst] = make_uint2(kw[0], kw[1]);
    vc[dst] = make_uint2(vw[0], vw[1]);
  }
}

int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  return int(g < 1 ? 1 : g);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

namespace {
int cache_write(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens, int32_t num_kv_heads,
                int32_t head_dim, void* k_cache, void* v_cache, int32_t cache_dtype, int32_t num_blocks,
                int32_t block_size, const int64_t* slot_mapping, float k_scale, float v_scale,
                const float* k_head_scales, const float* v_head_scales, const pkv::Layers& layers, void* stream) {
  using pkv::fail;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID, "kv_cache_write: bad sizes");
  if (layers.n < 1 || layers.n > 65535) return fail(PKV_ERR_INVALID, "kv_cache_write: bad layer count %d", layers.n);
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID, "kv_cache_write: NULL pointer");
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (row % 8 != 0) return fail(PKV_ERR_INVALID, "kv_cache_write: num_kv_heads*head_dim must be a multiple of 8");
  const int64_t num_slots = int64_t(num_blocks) * block_size;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (cache_dtype == in_dtype && (in_dtype == PKV_F32 || in_dtype == PKV_BF16)) {
    const int eb = pkv::dtype_bytes(in_dtype);
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
      return fail(PKV_ERR_INVALID, "kv_cache_write: pointers must be 16-byte aligned");
    const int64_t chunks = row * eb / 16;
    hipLaunchKernelGGL(write_copy16, dim3(grid_for(num_tokens * chunks), layers.n), dim3(256), 0, st,
                       static_cast<const uint4*>(k), static_cast<const uint4*>(v), static_cast<uint4*>(k_cache),
                       static_cast<uint4*>(v_cache), slot_mapping, int64_t(num_tokens), chunks, num_slots, layers.in,
                       layers.cache);
  } else if (cache_dtype == PKV_FP8_E4M3 && (in_dtype == PKV_BF16 || in_dtype == PKV_F32)) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f)) return fail(PKV_ERR_INVALID, "kv_cache_write: scales must be > 0");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 8) || !aligned(v_cache, 8))
      return fail(PKV_ERR_INVALID, "kv_cache_write: input pointers must be 16-byte, cache 8-byte aligned");
    if ((k_head_scales || v_head_scales) && head_dim % 8 != 0)
      return fail(PKV_ERR_INVALID, "kv_cache_write: per-head scales need head_dim a multiple of 8");
    InvScales inv;
    const int rc = pkv::head_inverse_scales("kv_cache_write", num_kv_heads, k_scale, v_scale, k_head_scales,
                                            v_head_scales, inv.k, inv.v);
    if (rc != PKV_OK) return rc;
    const int64_t chunks = row / 8;
    const int64_t per_head = head_dim % 8 == 0 ? head_dim / 8 : INT64_MAX;
    if (in_dtype == PKV_BF16)
      hipLaunchKernelGGL(write_fp8<true>, dim3(grid_for(num_tokens * chunks), layers.n), dim3(256), 0, st, k, v,
                         static_cast<uint2*>(k_cache), static_cast<uint2*>(v_cache), slot_mapping,
                         int64_t(num_tokens), chunks, num_slots, per_head, inv, layers.in, layers.cache);
    else
      hipLaunchKernelGGL(write_fp8<false>, dim3(grid_for(num_tokens * chunks), layers.n), dim3(256), 0, st, k, v,
                         static_cast<uint2*>(k_cache), static_cast<uint2*>(v_cache), slot_mapping,
                         int64_t(num_tokens), chunks, num_slots, per_head, inv, layers.in, layers.cache);
  } else {
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write: input dtype %d -> cache dtype %d not supported", in_dtype,
                cache_dtype);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_cache_write: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}
}  // namespace

extern "C" int pkv_kv_cache_write(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, void* k_cache, void* v_cache,
                                  int32_t cache_dtype, int32_t num_blocks, int32_t block_size,
                                  const int64_t* slot_mapping, float k_scale, float v_scale,
                                  const float* k_head_scales, const float* v_head_scales, void* stream) {
  return cache_write(k, v, in_dtype, num_tokens, num_kv_heads, head_dim, k_cache, v_cache, cache_dtype, num_blocks,
                     block_size, slot_mapping, k_scale, v_scale, k_head_scales, v_head_scales, pkv::Layers{},
                     stream);
}

extern "C" int pkv_kv_cache_write_layers(const void* k, const void* v, int32_t in_dtype, int32_t num_tokens,
                                         int32_t num_kv_heads, int32_t head_dim, void* k_cache, void* v_cache,
                                         int32_t cache_dtype, int32_t num_blocks, int32_t block_size,
                                         const int64_t* slot_mapping, float k_scale, float v_scale,
                                         const float* k_head_scales, const float* v_head_scales,
                                         const pkv_layers* layers, void* stream) {
  pkv::Layers ls;
  const int rc = pkv::layers_from("kv_cache_write_layers", layers, true, pkv::kLayerIn | pkv::kLayerCache, &ls);
  if (rc != PKV_OK) return rc;
  return cache_write(k, v, in_dtype, num_tokens, num_kv_heads, head_dim, k_cache, v_cache, cache_dtype, num_blocks,
                     block_size, slot_mapping, k_scale, v_scale, k_head_scales, v_head_scales, ls, stream);
}
