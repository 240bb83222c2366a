// paged_attention_prefill_varlen: one launch over a mixed continuous-batching step --
// prefill chunks (several new tokens of a sequence, with or without cached prefix) and
// decode rows (one new token) -- over the paged KV cache.
//
// "Continuous Batching", "5. Technical explanation" (mixed batching): the step's forward
// pass holds prefill tokens of some requests next to one decode token of others, and a
// varlen kernel handles the ragged shape, the requests delimited by cu_seqlens ("6. Under
// the hood"). What each query row computes is the page-walk attention of "Project 17:
// Production Serving: Continuous Batching and PagedAttention", "Step 6": new row i of a
// sequence with q new tokens and seq_len L sits at position L - q + i and attends keys
// 0 .. L - q + i (bottom-right causal alignment, the K/V of the step already written).
//
// gfx950 design (one kernel, 8-wave workgroups, a host work list, longest item first):
//  * prefill item = (sequence, KV head g, block of 128/G new tokens): the 128 query rows
//    (token, head) -- GQA packed, all G heads of g share each K/V tile -- are split over
//    the 8 waves, 16 rows (one 16-column MFMA block) each. K/V tiles of 32 keys are
//    staged in LDS by the whole workgroup with coalesced 16-byte loads (each 16 lanes
//    read one head row), double buffered; K fragments are read with ds_read_b128 as
//    the A operand of v_mfma_f32_16x16x32_bf16; the softmax runs over the whole tile and
//    P.V uses the same instruction, its V^T operand assembled from two
//    ds_read_b64_tr_b16. Tiles past the block's last position are never loaded; on the
//    diagonal, scores are masked per row.
//  * decode item = (sequence with one new token, KV head): the 8 waves stream contiguous
//    block ranges of the context with the decode kernel's per-wave loop (mfma_common.h)
//    and merge their partial softmax states by log-sum-exp through LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "mfma_common.h"
#include "pkv.h"
#include "pkv_internal.h"

namespace {

using pkv::bf16x8_t;
using pkv::f32x4_t;
using pkv::lds_s16x4_t;
using pkv::pack_bf16x2_rne;
using pkv::s16x4_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKindPrefill = 0;
constexpr int kKindDecode = 1;
constexpr int kRowsPerItem = 128;   // query rows (token, head) of a prefill item
constexpr int kTileKeys = 32;       // keys per LDS tile
constexpr int kWaves = 8;           // waves per workgroup: 16 rows each / one KV head each
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 4;           // K/V tiles in flight per workgroup (register ring)

struct VarlenArgs {
  const uint16_t* q;      // [total_q][Hq][D] bf16
  uint16_t* out;          // [total_q][Hq][D] bf16
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  float* lse_out;         // [total_q][Hq], nullable
  const int4* work;       // (seq, kind << 24 | head or head group, first new token, keys to visit)
  int table_width;
  int num_seqs;
  int total_q;
  int num_kv_heads;
  int group;
  int num_blocks;
  int len_clamp;
  float zscale_h[pkv::kHeadScales];   // per KV head: softmax scale * k_scale * log2(e)
  float vscale_h[pkv::kHeadScales];   // per KV head: v_scale
};

template <int CDT, int D>
struct Smem {
  static constexpr int RS = D * 2 + 32;                       // bytes per bf16 key row (padded)
  static constexpr int kTile = kTileKeys * RS;                // one K or V tile
  static constexpr int kPrefill = 4 * kTile;                  // K, V x double buffer
  static constexpr int kDecodeTiles = kWaves * 16 * RS;       // the waves' V tiles
  static constexpr int kDecodeMerge = (kWaves / 2) * (D / 4 + 2) * 64 * 4;   // merge states
  static constexpr int kDecode = kDecodeTiles > kDecodeMerge ? kDecodeTiles : kDecodeMerge;
  static constexpr int kBytes = kPrefill > kDecode ? kPrefill : kDecode;
};

// Decode item (one new token of sequence s, KV head g): the 8 waves take contiguous
// ranges of the context's blocks, stream them with the decode kernel's per-wave loop,
// then merge their (m, l, o) states in three LDS rounds (8 -> 4 -> 2 -> 1 waves).
template <int CDT, int D, int BS>
__device__ __forceinline__ void run_decode_item(const VarlenArgs& a, uint8_t* smem, int s, int g, int key_end) {
  constexpr int MT = D / 16;
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;
  constexpr int RS = D * 2 + 32;
  constexpr int NS = MT * 4 + 2;                 // floats of one lane's state
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int row = a.cu_q[s + 1] - 1;             // the sequence's one new token
  const int nblk = (key_end + BS - 1) / BS;
  const int per = (nblk + kWaves - 1) / kWaves;  // blocks per wave
  const int b0 = min(nblk, w * per), b1 = min(nblk, (w + 1) * per);
  pkv::DecodeWaveIn in;
  in.q = a.q + (int64_t(row) * Hq + int64_t(g) * G) * D;
  in.G = G;
  in.kc = a.kc;
  in.vc = a.vc;
  in.row_bytes = int64_t(Hkv) * D * EB;
  in.head_off = int64_t(g) * D * EB;
  in.bt_row = a.block_tables + int64_t(s) * a.table_width;
  in.num_blocks = a.num_blocks;
  in.tok_begin = b0 * BS;
  in.tok_end = min(key_end, b1 * BS);
  in.zscale = a.zscale_h[g & (pkv::kHeadScales - 1)];
  float m, lsum;
  f32x4_t o[MT];
  pkv::decode_wave<CDT, D, BS>(in, smem + w * 16 * RS, m, lsum, o);

  // tree merge; the state of wave x lives at st + x*NS*64, one float per (field, lane)
  __syncthreads();                               // the V tiles are no longer needed
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int half = kWaves / 2; half >= 1; half /= 2) {
    if (w >= half && w < 2 * half) {
      float* dst = st + (w - half) * NS * 64 + lane;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * mt + r) * 64] = o[mt][r];
      dst[(4 * MT) * 64] = m;
      dst[(4 * MT + 1) * 64] = lsum;
    }
    __syncthreads();
    if (w < half) {
      const float* src = st + w * NS * 64 + lane;
      const float mo = src[(4 * MT) * 64];
      const float lo = src[(4 * MT + 1) * 64];
      const float mn = fmaxf(m, mo);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float ca = pkv::fast_exp2(m - mref);
      const float cb = pkv::fast_exp2(mo - mref);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[mt][r] = o[mt][r] * ca + src[(4 * mt + r) * 64] * cb;
      lsum = lsum * ca + lo * cb;
      m = mn;
    }
    __syncthreads();
  }
  if (w != 0 || hl >= G) return;
  const int hq = g * G + hl;
  const float inv = lsum > 0.f ? a.vscale_h[g & (pkv::kHeadScales - 1)] / lsum : 0.f;
  uint16_t* orow = a.out + (int64_t(row) * Hq + hq) * D + 4 * grp;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t lo = pack_bf16x2_rne(o[mt][0] * inv, o[mt][1] * inv);
    const uint32_t hi = pack_bf16x2_rne(o[mt][2] * inv, o[mt][3] * inv);
    *reinterpret_cast<uint2*>(orow + 16 * mt) = make_uint2(lo, hi);
  }
  if (a.lse_out && grp == 0)
    a.lse_out[int64_t(row) * Hq + hq] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
}

template <int CDT, int D, int BS>
__device__ __forceinline__ void run_prefill_item(const VarlenArgs& a, uint8_t* smem, int s, int g, int q0,
                                                 int key_end) {
  constexpr int KS = D / 32;
  constexpr int MT = D / 16;
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;
  constexpr int RS = Smem<CDT, D>::RS;
  constexpr int TILE = Smem<CDT, D>::kTile;
  constexpr int CPK = D * EB / 16;                      // 16-byte chunks per key head row
  constexpr int CHUNKS = kTileKeys * CPK;               // per plane per tile
  constexpr int LPT = (CHUNKS + kThreads - 1) / kThreads;   // chunk loads per thread per plane
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int row0 = a.cu_q[s];
  const int qs = a.cu_q[s + 1] - row0;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_clamp ? a.len_clamp : L);
  if (key_end > L) key_end = L;
  const int pos0 = L - qs;                              // position of new token 0
  const int QB = kRowsPerItem / G;                      // new tokens of this item
  const int ntok = min(QB, qs - q0);

  // this wave's 16 rows: r = 16*w + hl -> token r / G, head r % G
  const int r_row = 16 * w + hl;
  const int tok = r_row / G;
  const bool row_ok = tok < ntok;
  const int pos = pos0 + q0 + tok;
  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = a.q + (int64_t(row0 + q0 + tok) * Hq + int64_t(g) * G + r_row % G) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // last position among this wave's valid rows (wave-uniform)
  const int last_tok = min(ntok - 1, (16 * w + 15) / G);
  const int wave_last_pos = last_tok >= (16 * w) / G ? pos0 + q0 + last_tok : -1;

  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt_row = a.block_tables + int64_t(s) * a.table_width;
  const int64_t row_bytes = int64_t(Hkv) * D * EB;
  const int64_t head_off = int64_t(g) * D * EB;
  const int ntiles = (key_end + kTileKeys - 1) / kTileKeys;

  // tile t is staged in registers kst[t % kDepth] (kDepth tiles in flight), then
  // committed to the LDS buffer t % 2 one iteration before it is consumed
  uint4 kst[kDepth][LPT], vst[kDepth][LPT];
  // block ids of a tile are wave-uniform scalar loads (constant address space); K/V loads
  // are unconditional (clamped to block 0, zeroed after) so the ring's waits stay partial
  const __attribute__((address_space(4))) int32_t* btc =
      (const __attribute__((address_space(4))) int32_t*)(uintptr_t)(bt_row);
  auto stage = [&](int t, uint4 (&ks)[LPT], uint4 (&vs)[LPT]) {
    const int key0 = t * kTileKeys;
    const int blk0 = btc[key0 / BS];
    const int blk1 = BS >= kTileKeys ? blk0 : (key0 + 16 < key_end ? btc[(key0 + 16) / BS] : -1);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = min(tid + kThreads * i, CHUNKS - 1);
      const int kt = c / CPK;                              // key within the tile
      const int key = key0 + kt;
      const int blk = (BS >= kTileKeys || kt < 16) ? blk0 : blk1;
      const bool ok = tid + kThreads * i < CHUNKS && key < key_end && blk >= 0 && blk < a.num_blocks;
      int64_t off = ok ? (int64_t(blk) * BS + key % BS) * row_bytes + head_off + 16 * (c % CPK) : 0;
      asm volatile("" : "+v"(off));                        // keep the load unconditional
      const uint4 kv = *reinterpret_cast<const uint4*>(a.kc + off);
      const uint4 vv = *reinterpret_cast<const uint4*>(a.vc + off);
      ks[i] = ok ? kv : make_uint4(0, 0, 0, 0);
      vs[i] = ok ? vv : make_uint4(0, 0, 0, 0);
    }
  };
  auto commit = [&](int buf, const uint4 (&kst)[LPT], const uint4 (&vst)[LPT]) {
    uint8_t* kt = smem + buf * 2 * TILE;
    uint8_t* vt = kt + TILE;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + kThreads * i;
      if (c >= CHUNKS) continue;
      const int key = c / CPK;
      const int ci = c % CPK;
      if constexpr (CDT == PKV_BF16) {
        *reinterpret_cast<uint4*>(kt + key * RS + 16 * ci) = kst[i];
        *reinterpret_cast<uint4*>(vt + key * RS + 16 * ci) = vst[i];
      } else {
        *reinterpret_cast<uint4*>(kt + key * RS + 32 * ci) = pkv::fp8x8_to_bf16x8(kst[i].x, kst[i].y);
        *reinterpret_cast<uint4*>(kt + key * RS + 32 * ci + 16) = pkv::fp8x8_to_bf16x8(kst[i].z, kst[i].w);
        *reinterpret_cast<uint4*>(vt + key * RS + 32 * ci) = pkv::fp8x8_to_bf16x8(vst[i].x, vst[i].y);
        *reinterpret_cast<uint4*>(vt + key * RS + 32 * ci + 16) = pkv::fp8x8_to_bf16x8(vst[i].z, vst[i].w);
      }
    }
  };
  // One 32-key tile: scores for keys key0 + 16*sb + 4*grp + r (sb = 0, 1), softmax over
  // the tile, then P.V on v_mfma_f32_16x16x32_bf16 whose k index 8*grp + j runs over keys
  // 4*grp + j (j < 4) and 16 + 4*grp + (j - 4) (j >= 4): the lane's own 8 weights.
  auto compute = [&](int t, int buf) {
    const int key0 = t * kTileKeys;
    if (key0 > wave_last_pos) return;                        // wave-uniform: all masked
    const uint8_t* kt = smem + buf * 2 * TILE;
    const uint8_t* vt = kt + TILE;
    float z[8];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(kt + (16 * sb + hl) * RS + 2 * (32 * kk + 8 * grp));
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], sc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 16 * sb + 4 * grp + r;
        z[4 * sb + r] = (row_ok && key <= pos && key < key_end) ? sc[r] * a.zscale_h[g & (pkv::kHeadScales - 1)] : -INFINITY;
      }
    }
    float mt_ = z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt_ = fmaxf(mt_, z[j]);
    mt_ = pkv::lane_groups_max(mt_);
    const float mn = fmaxf(m, mt_);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = pkv::fast_exp2(m - mref);
    uint32_t pw[4];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pw[j] = pack_bf16x2_rne(pkv::fast_exp2(z[2 * j] - mref), pkv::fast_exp2(z[2 * j + 1] - mref));
      ps += pkv::bf16_lo(pw[j]) + pkv::bf16_hi(pw[j]);
    }
    lsum = lsum * alpha + ps;
    m = mn;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    const uint8_t* vsrc = vt + (4 * grp + (hl >> 2)) * RS + (4 * (hl & 3)) * 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vsrc + 32 * mt));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vsrc + 16 * RS + 32 * mt));
      const bf16x8_t vf = __builtin_bit_cast(
          bf16x8_t, make_uint4(__builtin_bit_cast(uint2, v0).x, __builtin_bit_cast(uint2, v0).y,
                               __builtin_bit_cast(uint2, v1).x, __builtin_bit_cast(uint2, v1).y));
      f32x4_t acc = o[mt];
      acc[0] *= alpha;
      acc[1] *= alpha;
      acc[2] *= alpha;
      acc[3] *= alpha;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc, 0, 0, 0);
    }
  };

  if (ntiles > 0) {
    // the ring is static: tile t + kDepth is always staged (tiles past the end read
    // clamped addresses and are zeroed), so every wait is a known partial count
#pragma unroll
    for (int u = 0; u < kDepth; ++u) stage(u, kst[u], vst[u]);
    commit(0, kst[0], vst[0]);
    __syncthreads();
    for (int t0 = 0; t0 < ntiles; t0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int t = t0 + u;
        stage(t + kDepth, kst[u], vst[u]);                 // slot of tile t, already committed
        if (t < ntiles) compute(t, t & 1);
        commit((t + 1) & 1, kst[(u + 1) % kDepth], vst[(u + 1) % kDepth]);
        __syncthreads();
      }
    }
  }

  float l = lsum;
  l = pkv::lane_groups_sum(l);
  if (!row_ok) return;
  const int row = row0 + q0 + tok;
  const int hq = g * G + r_row % G;
  const float inv = l > 0.f ? a.vscale_h[g & (pkv::kHeadScales - 1)] / l : 0.f;
  uint16_t* orow = a.out + (int64_t(row) * Hq + hq) * D + 4 * grp;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t lo = pack_bf16x2_rne(o[mt][0] * inv, o[mt][1] * inv);
    const uint32_t hi = pack_bf16x2_rne(o[mt][2] * inv, o[mt][3] * inv);
    *reinterpret_cast<uint2*>(orow + 16 * mt) = make_uint2(lo, hi);
  }
  if (a.lse_out && grp == 0) a.lse_out[int64_t(row) * Hq + hq] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <int CDT, int D, int BS>
__global__ void __launch_bounds__(kThreads) varlen_kernel(VarlenArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<CDT, D>::kBytes];
  const int4 it = a.work[blockIdx.x];
  const int s = it.x;
  const int kind = it.y >> 24;
  const int h = it.y & 0xffffff;
  if (s < 0 || s >= a.num_seqs) return;                   // malformed item: skip (uniform)
  const int row0 = a.cu_q[s];
  const int qs = a.cu_q[s + 1] - row0;
  if (qs <= 0 || row0 < 0 || row0 + qs > a.total_q) return;   // malformed offsets: skip
  if (kind == kKindDecode) {
    if (h >= a.num_kv_heads) return;
    run_decode_item<CDT, D, BS>(a, smem, s, h, max(0, min(it.w, a.len_clamp)));
  } else {
    if (h >= a.num_kv_heads || it.z < 0 || it.z >= qs) return;
    run_prefill_item<CDT, D, BS>(a, smem, s, h, it.z, max(0, min(it.w, a.len_clamp)));
  }
}

using VarlenFn = void (*)(VarlenArgs);

template <int CDT, int D>
VarlenFn pick_bs(int BS) {
  switch (BS) {
    case 16: return varlen_kernel<CDT, D, 16>;
    case 32: return varlen_kernel<CDT, D, 32>;
    default: return nullptr;
  }
}

template <int CDT>
VarlenFn pick_d(int D, int BS) {
  switch (D) {
    case 64: return pick_bs<CDT, 64>(BS);
    case 128: return pick_bs<CDT, 128>(BS);
    default: return nullptr;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" int pkv_build_varlen_work(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                                     int32_t num_kv_heads, int32_t group, int32_t* items, int32_t capacity,
                                     int32_t* count) {
  using pkv::fail;
  if (num_seqs < 0 || num_kv_heads <= 0 || group <= 0 || !count || (num_seqs > 0 && (!q_lens || !seq_lens)))
    return fail(PKV_ERR_INVALID, "build_varlen_work: bad arguments");
  if (group > 16 || kRowsPerItem % group != 0)
    return fail(PKV_ERR_UNSUPPORTED, "build_varlen_work: group %d not in {1,2,4,8,16}", group);
  struct Item {
    int32_t s, kh, q0, keys, prefill;
  };
  std::vector<Item> v;
  const int32_t QB = kRowsPerItem / group;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q = q_lens[s], L = seq_lens[s];
    if (q < 0 || L < 0 || q > L) return fail(PKV_ERR_INVALID, "build_varlen_work: sequence %d q_len %d seq_len %d", s, q, L);
    if (q == 0) continue;
    if (q == 1) {
      for (int32_t g = 0; g < num_kv_heads; ++g) v.push_back({s, (kKindDecode << 24) | g, 0, L, 0});
      continue;
    }
    for (int32_t q0 = 0; q0 < q; q0 += QB) {
      const int32_t keys = std::min(L, L - q + std::min(q, q0 + QB));
      for (int32_t g = 0; g < num_kv_heads; ++g) v.push_back({s, (kKindPrefill << 24) | g, q0, keys, 1});
    }
  }
  // longest first: prefill items cost ~ keys x 128 rows of MFMA work, decode items
  // ~ keys of streaming; order by keys, prefill before decode at equal keys
  std::stable_sort(v.begin(), v.end(), [](const Item& x, const Item& y) {
    if (x.keys != y.keys) return x.keys > y.keys;
    return x.prefill > y.prefill;
  });
  *count = int32_t(v.size());
  if (int64_t(v.size()) > capacity || (!v.empty() && !items))
    return fail(PKV_ERR_INVALID, "build_varlen_work: %zu items, capacity %d", v.size(), capacity);
  for (size_t i = 0; i < v.size(); ++i) {
    items[4 * i + 0] = v[i].s;
    items[4 * i + 1] = v[i].kh;
    items[4 * i + 2] = v[i].q0;
    items[4 * i + 3] = v[i].keys;
  }
  return PKV_OK;
}

extern "C" int pkv_paged_attention_prefill_varlen(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                                  const void* v_cache, int32_t cache_dtype,
                                                  const int32_t* block_tables, const int32_t* seq_lens,
                                                  const int32_t* cu_seqlens_q, int32_t table_width, int32_t num_seqs,
                                                  int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                                  int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                                  const float* k_head_scales, const float* v_head_scales,
                                                  const int32_t* work_items, int32_t num_work, float* lse_out,
                                                  void* stream) {
  using pkv::fail;
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || table_width < 0 || num_blocks < 0 ||
      max_seq_len < 0 || num_work < 0)
    return fail(PKV_ERR_INVALID, "prefill_varlen: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "prefill_varlen: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (q_dtype != PKV_BF16 || (cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3) || G > 16 ||
      kRowsPerItem % G != 0)
    return fail(PKV_ERR_UNSUPPORTED, "prefill_varlen: unsupported (q dtype %d, cache dtype %d, group %d)", q_dtype,
                cache_dtype, G);
  VarlenFn fn = cache_dtype == PKV_BF16 ? pick_d<PKV_BF16>(head_dim, block_size)
                                        : pick_d<PKV_FP8_E4M3>(head_dim, block_size);
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "prefill_varlen: head_dim %d / block_size %d not supported", head_dim,
                block_size);
  if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PKV_ERR_INVALID, "prefill_varlen: scales must be > 0");
  if (num_work == 0 || num_seqs == 0 || total_q == 0) return PKV_OK;
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "prefill_varlen: the cache has no blocks");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !cu_seqlens_q || !work_items)
    return fail(PKV_ERR_INVALID, "prefill_varlen: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(work_items))
    return fail(PKV_ERR_INVALID, "prefill_varlen: q, out, cache planes and work list must be 16-byte aligned");
  VarlenArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.cu_q = cu_seqlens_q;
  a.lse_out = lse_out;
  a.work = reinterpret_cast<const int4*>(work_items);
  a.table_width = table_width;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_kv_heads = num_kv_heads;
  a.group = G;
  a.num_blocks = num_blocks;
  const int64_t tcap = int64_t(table_width) * block_size;
  a.len_clamp = int(tcap < max_seq_len ? tcap : max_seq_len);
  {
    const int rc = pkv::head_scales("attention", num_kv_heads, scale, k_scale, v_scale, k_head_scales,
                                    v_head_scales, a.zscale_h, a.vscale_h);
    if (rc != PKV_OK) return rc;
  }
  hipLaunchKernelGGL(fn, dim3(num_work), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill_varlen: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}
