// GPU twin of the counter-based value generator in workloads/__init__.py.
// Input generation only (test and benchmark infrastructure): element e of stream
// `key` is field e%3 of SplitMix64(key + (e/3 + 1) * golden gamma), three 6-bit
// uniforms summed (Irwin-Hall(3)), value = sigma * (2 * sum - 189) / 64, stored as
// float32 or bfloat16 (exact). Bit-identical to the NumPy implementation.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t finalize(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void __launch_bounds__(256) fill_values(void* out, int as_bf16, uint64_t key, int64_t e0,
                                                   int64_t count, float sigma) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint64_t e = uint64_t(e0 + i);
    const uint64_t n = e / 3;
    const uint32_t j = uint32_t(e - n * 3);
    const uint64_t h = finalize(key + (n + 1) * 0x9E3779B97F4A7C15ull);
    const uint32_t f = uint32_t((h >> (18 * j)) & 0x3FFFFull);
    const uint32_t s = (f & 63u) + ((f >> 6) & 63u) + (f >> 12);
    float v = float(s) * 0.03125f - 2.953125f;
    if (sigma != 1.0f) v *= sigma;
    if (as_bf16)
      static_cast<uint16_t*>(out)[i] = uint16_t(__float_as_uint(v) >> 16);
    else
      static_cast<float*>(out)[i] = v;
  }
}

}  // namespace

// out: device buffer of `count` float32 (as_bf16 = 0) or bfloat16 (1) values.
extern "C" int pkvgen_fill(void* out, int as_bf16, uint64_t key, int64_t e0, int64_t count, float sigma,
                           void* stream) {
  if (count <= 0) return 0;
  if (!out || e0 < 0) return -1;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_values, dim3(unsigned(blocks)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), out,
                     as_bf16, key, e0, count, sigma);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Many segments in one launch: segment r writes elements e0[r] .. e0[r] + n_r - 1 of
// stream keys[r] to out[off[r] .. off[r+1]) (off: int64 prefix of the segment sizes,
// off[0] = 0). Each thread finds its segment by binary search over off.
namespace {
__global__ void __launch_bounds__(256) fill_segments(void* out, int as_bf16, int nseg, const uint64_t* keys,
                                                     const int64_t* e0, const int64_t* off, float sigma) {
  const int64_t total = off[nseg];
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    int lo = 0, hi = nseg - 1;                 // last r with off[r] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const uint64_t e = uint64_t(e0[lo] + (i - off[lo]));
    const uint64_t n = e / 3;
    const uint32_t j = uint32_t(e - n * 3);
    const uint64_t h = finalize(keys[lo] + (n + 1) * 0x9E3779B97F4A7C15ull);
    const uint32_t f = uint32_t((h >> (18 * j)) & 0x3FFFFull);
    const uint32_t s = (f & 63u) + ((f >> 6) & 63u) + (f >> 12);
    float v = float(s) * 0.03125f - 2.953125f;
    if (sigma != 1.0f) v *= sigma;
    if (as_bf16)
      static_cast<uint16_t*>(out)[i] = uint16_t(__float_as_uint(v) >> 16);
    else
      static_cast<float*>(out)[i] = v;
  }
}
}  // namespace

// keys, e0: device [nseg]; off: device int64 [nseg + 1] (non-decreasing, off[0] = 0);
// out: device buffer of off[nseg] elements; total: off[nseg] (host copy, sizes the grid).
extern "C" int pkvgen_fill_segments(void* out, int as_bf16, int nseg, const void* keys, const void* e0,
                                    const void* off, int64_t total, float sigma, void* stream) {
  if (nseg <= 0 || total <= 0) return 0;
  if (!out || !keys || !e0 || !off) return -1;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_segments, dim3(unsigned(blocks)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     out, as_bf16, nseg, static_cast<const uint64_t*>(keys), static_cast<const int64_t*>(e0),
                     static_cast<const int64_t*>(off), sigma);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ---------------------------------------------------------------------------------
// HBM stream-read probe (measurement only): every lane reads 16-byte chunks of `buf`
// with UNROLL independent loads in flight per iteration, folds them with xor, and
// writes one word per thread (so the loads cannot be dropped).
// ---------------------------------------------------------------------------------
namespace {
template <int UNROLL>
__global__ void __launch_bounds__(256) read_probe(const uint4* __restrict__ buf, int64_t n16, uint32_t* out) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}
}  // namespace

namespace {
// The same probe with each workgroup (512 threads) streaming one contiguous share of the
// buffer, 8 loads in flight per lane, with the non-temporal hint: the shape and cache
// policy under which MI355X reads fastest (the per-lane xor keeps the loads live).
__global__ void __launch_bounds__(512) read_probe_stream(const uint4* __restrict__ buf, int64_t n16, int64_t per,
                                                         uint32_t* out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t lo = int64_t(blockIdx.x) * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  int64_t i = lo + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 7 * 512 < hi; i += 8 * 512) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(buf + i + u * 512));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < hi; i += 512) acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(buf + i));
  out[int64_t(blockIdx.x) * 512 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
}  // namespace

// buf: device, n16 chunks of 16 bytes; out: device uint32 [blocks * 512].
extern "C" int pkvgen_read_probe_stream(const void* buf, int64_t n16, int blocks, void* out, void* stream) {
  if (!buf || !out || n16 <= 0 || blocks <= 0) return -1;
  const int64_t per = (n16 + blocks - 1) / blocks;
  hipLaunchKernelGGL(read_probe_stream, dim3(blocks), dim3(512), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), n16, per, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// buf: device, n16 chunks of 16 bytes; out: device uint32 [blocks * 256].
extern "C" int pkvgen_read_probe(const void* buf, int64_t n16, int blocks, int unroll, void* out, void* stream) {
  if (!buf || !out || n16 <= 0 || blocks <= 0) return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint4* b = static_cast<const uint4*>(buf);
  uint32_t* o = static_cast<uint32_t*>(out);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(read_probe<1>, dim3(blocks), dim3(256), 0, st, b, n16, o); break;
    case 2: hipLaunchKernelGGL(read_probe<2>, dim3(blocks), dim3(256), 0, st, b, n16, o); break;
    case 4: hipLaunchKernelGGL(read_probe<4>, dim3(blocks), dim3(256), 0, st, b, n16, o); break;
    case 8: hipLaunchKernelGGL(read_probe<8>, dim3(blocks), dim3(256), 0, st, b, n16, o); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
