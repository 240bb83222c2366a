// Internal helpers shared by libpkv's host code and HIP kernels (not part of the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Record a message for pkv_last_error() and return `code`.
int fail(int code, const char* fmt, ...);
// Bytes per element of a PKV_* dtype code (0 if unknown).
int dtype_bytes(int32_t dt);

// Per-KV-head scale slots carried in kernel arguments: a kernel reads the slot of its
// KV head (h & (kHeadScales - 1)); without per-head factors every slot holds the same
// value, so any number of heads works, with them at most kHeadScales heads.
constexpr int kHeadScales = 16;

// Attention constants per KV head: zs[h] = scale * k_scale * k_head[h] * log2(e) and
// vs[h] = v_scale * v_head[h] (a NULL array means factors of 1), products in double.
// Checks that every scale is finite and > 0 and that per-head factors come with at most
// kHeadScales heads; returns PKV_OK or the error (message recorded under `who`).
int head_scales(const char* who, int32_t num_kv_heads, float scale, float k_scale, float v_scale,
                const float* k_head, const float* v_head, float* zs, float* vs);
// Cache-write inverses per KV head: ki[h] = fl32(1 / (k_scale * k_head[h])), likewise vi.
int head_inverse_scales(const char* who, int32_t num_kv_heads, float k_scale, float v_scale,
                        const float* k_head, const float* v_head, float* ki, float* vi);

// Layer batching of a *_layers call, checked: n layers and the byte (lse: float)
// strides between them. `uses` names the strides the call reads (kLayerIn | ...); each of
// those must be >= 0, a multiple of 16 bytes (4 floats) and non-zero when n > 1. A NULL
// descriptor is INVALID when `required`, else one layer.
struct Layers {
  int n = 1;
  int64_t in = 0, out = 0, cache = 0, lse = 0;
};
constexpr unsigned kLayerIn = 1, kLayerOut = 2, kLayerCache = 4, kLayerLse = 8;
int layers_from(const char* who, const pkv_layers* desc, bool required, unsigned uses, Layers* out);

// pkv_paged_attention_decode_split (the no-allocation entry point reuses it).
int decode_split(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                 int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width,
                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale, float v_scale,
                 const float* k_head_scales, const float* v_head_scales, const int32_t* rows, int32_t num_rows,
                 const int32_t* cu_seqlens_q, int32_t total_q, const int32_t* plan, int32_t num_slots,
                 int32_t tiles_per_slot, int32_t max_pieces, void* workspace, size_t workspace_bytes,
                 float* lse_out, const Layers& layers, void* stream);

}  // namespace pkv

#ifdef __HIPCC__
#include <hip/hip_runtime.h>

namespace pkv {

// ---- scalar conversions --------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN, quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  // v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN (quieted)
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// OCP E4M3 code (low 8 bits of c) -> float, exact. Relies on fp32 denormals being
// preserved (gfx950 default mode): the 7 magnitude bits placed at bit 20 form a
// float equal to the E4M3 magnitude times 2^-120 (subnormal codes included).
__device__ __forceinline__ float fp8_to_f32(uint32_t c) {
  const uint32_t em = c & 0x7fu;
  float mag = __uint_as_float(em << 20) * 0x1p120f;
  mag = (em == 0x7fu) ? __builtin_nanf("") : mag;
  return (c & 0x80u) ? -mag : mag;
}

// float y -> OCP E4M3 code: nearest-even, |y| >= 448 (inf included) saturates to
// 448, NaN -> 0x7F; the sign of y is always kept.
__device__ __forceinline__ uint32_t f32_to_fp8(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;           // 448.0f
  if (a >= 0x3c800000u) {                              // >= 2^-6: normal E4M3 range
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // round 23 -> 3 mantissa bits
    return sign | ((r >> 20) - (120u << 3));
  }
  // subnormal range: multiple of 2^-9, m in 0..8 (8 is the smallest normal, 0x08)
  const float t = __uint_as_float(a) * 512.0f;         // exact scaling
  return sign | uint32_t(__builtin_rintf(t));          // rint = round half to even
}

// ---- cross-lane reductions -----------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16,32); every lane of a group gets
// the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
#endif  // __HIPCC__
