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
// gfx950 design (one kernel, 4-wave workgroups, a host work list, longest item first):
//  * prefill item = (sequence, KV head g, block of 128/G new tokens): the 128 query rows
//    (token, head) -- GQA packed, all G heads of g share each K/V tile -- are split over
//    the 4 waves, 32 rows (two 16-column MFMA blocks) each. K/V tiles of 32 keys are
//    staged in LDS by the whole workgroup with coalesced 16-byte loads (each 16 lanes
//    read one head row), double buffered; K fragments are read with ds_read_b128 as
//    the A operand of v_mfma_f32_16x16x32_bf16, V^T fragments with ds_read_b64_tr_b16
//    for v_mfma_f32_16x16x16_bf16. Tiles past the block's last position are never
//    loaded; on the diagonal, scores are masked per row.
//  * decode item = (sequence with one new token, 4 KV heads): each wave streams one KV
//    head's context with the decode kernel's per-wave loop (mfma_common.h).
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
  float zscale;
  float v_scale;
};

template <int CDT, int D>
struct Smem {
  static constexpr int RS = D * 2 + 32;                       // bytes per bf16 key row (padded)
  static constexpr int kTile = kTileKeys * RS;                // one K or V tile
  static constexpr int kPrefill = 4 * kTile;                  // K, V x double buffer
  static constexpr int kDecode = 4 * 16 * RS;                 // 4 waves' V tiles
  static constexpr int kBytes = kPrefill > kDecode ? kPrefill : kDecode;
};

template <int CDT, int D, int BS>
__device__ __forceinline__ void run_decode_item(const VarlenArgs& a, uint8_t* smem, int s, int hg, int key_end) {
  constexpr int MT = D / 16;
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;
  constexpr int RS = D * 2 + 32;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = hg * 4 + w;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  if (g >= Hkv) return;                      // no workgroup barrier on this path
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int row = a.cu_q[s + 1] - 1;         // the sequence's one new token
  pkv::DecodeWaveIn in;
  in.q = a.q + (int64_t(row) * Hq + int64_t(g) * G) * D;
  in.G = G;
  in.kc = a.kc;
  in.vc = a.vc;
  in.row_bytes = int64_t(Hkv) * D * EB;
  in.head_off = int64_t(g) * D * EB;
  in.bt_row = a.block_tables + int64_t(s) * a.table_width;
  in.num_blocks = a.num_blocks;
  in.tok_begin = 0;
  in.tok_end = key_end;
  in.zscale = a.zscale;
  float m, lsum;
  f32x4_t o[MT];
  pkv::decode_wave<CDT, D, BS>(in, smem + w * 16 * RS, m, lsum, o);
  if (hl < G) {
    const int hq = g * G + hl;
    const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;
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
  constexpr int LPT = (CHUNKS + 255) / 256;             // chunk loads per thread per plane
  constexpr int NB = 2;                                 // 16-row MFMA blocks per wave
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

  // rows of this wave: r = 32*w + 16*nb + hl -> token r / G, head r % G
  int tok_of[NB];
  bool row_ok[NB];
  bf16x8_t qf[NB][KS];
  int wave_last_pos = -1;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 32 * w + 16 * nb + hl;
    tok_of[nb] = r / G;
    row_ok[nb] = tok_of[nb] < ntok;
    const uint16_t* qrow =
        a.q + (int64_t(row0 + q0 + tok_of[nb]) * Hq + int64_t(g) * G + r % G) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok[nb]) v = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qf[nb][kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  {
    // last position among this wave's valid rows (wave-uniform)
    const int last_tok = min(ntok - 1, (32 * w + 31) / G);
    wave_last_pos = last_tok >= (32 * w) / G ? pos0 + q0 + last_tok : -1;
  }

  float m[NB], lsum[NB];
  f32x4_t o[NB][MT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = -INFINITY;
    lsum[nb] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt_row = a.block_tables + int64_t(s) * a.table_width;
  const int64_t row_bytes = int64_t(Hkv) * D * EB;
  const int64_t head_off = int64_t(g) * D * EB;
  const int ntiles = (key_end + kTileKeys - 1) / kTileKeys;

  uint4 kst[LPT], vst[LPT];
  auto stage = [&](int t) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + 256 * i;
      const int key = t * kTileKeys + c / CPK;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (c < CHUNKS && key < key_end) {
        const int blk = bt_row[key / BS];
        if (blk >= 0 && blk < a.num_blocks) {
          const int64_t off = (int64_t(blk) * BS + key % BS) * row_bytes + head_off + 16 * (c % CPK);
          kv = *reinterpret_cast<const uint4*>(a.kc + off);
          vv = *reinterpret_cast<const uint4*>(a.vc + off);
        }
      }
      kst[i] = kv;
      vst[i] = vv;
    }
  };
  auto commit = [&](int buf) {
    uint8_t* kt = smem + buf * 2 * TILE;
    uint8_t* vt = kt + TILE;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + 256 * i;
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
  auto compute = [&](int t, int buf) {
    const uint8_t* kt = smem + buf * 2 * TILE;
    const uint8_t* vt = kt + TILE;
#pragma unroll
    for (int sb = 0; sb < kTileKeys / 16; ++sb) {
      const int key0 = t * kTileKeys + 16 * sb;
      if (key0 > wave_last_pos || key0 >= key_end) continue;     // wave-uniform: all masked
      bf16x8_t kf[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8_t*>(kt + (16 * sb + hl) * RS + 2 * (32 * kk + 8 * grp));
      s16x4_t vf[MT];
      const uint8_t* vsrc = vt + (16 * sb + 4 * grp + (hl >> 2)) * RS + (4 * (hl & 3)) * 2;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) vf[mt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vsrc + 32 * mt));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[nb][kk], sc, 0, 0, 0);
        const int pos = pos0 + q0 + tok_of[nb];
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 4 * grp + r;
          z[r] = (row_ok[nb] && key <= pos && key < key_end) ? sc[r] * a.zscale : -INFINITY;
        }
        float mt_ = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mt_ = fmaxf(mt_, __shfl_xor(mt_, 16));
        mt_ = fmaxf(mt_, __shfl_xor(mt_, 32));
        const float mn = fmaxf(m[nb], mt_);
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = pkv::fast_exp2(m[nb] - mref);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = pkv::fast_exp2(z[r] - mref);
        const uint32_t p01 = pack_bf16x2_rne(pr[0], pr[1]);
        const uint32_t p23 = pack_bf16x2_rne(pr[2], pr[3]);
        lsum[nb] = lsum[nb] * alpha + (pkv::bf16_lo(p01) + pkv::bf16_hi(p01)) + (pkv::bf16_lo(p23) + pkv::bf16_hi(p23));
        m[nb] = mn;
        const s16x4_t pf = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4_t acc = o[nb][mt];
          acc[0] *= alpha;
          acc[1] *= alpha;
          acc[2] *= alpha;
          acc[3] *= alpha;
          o[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[mt], pf, acc, 0, 0, 0);
        }
      }
    }
  };

  if (ntiles > 0) {
    stage(0);
    commit(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) stage(t + 1);
      compute(t, t & 1);
      if (t + 1 < ntiles) commit((t + 1) & 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = lsum[nb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!row_ok[nb]) continue;
    const int r = 32 * w + 16 * nb + hl;
    const int row = row0 + q0 + tok_of[nb];
    const int hq = g * G + r % G;
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    uint16_t* orow = a.out + (int64_t(row) * Hq + hq) * D + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t lo = pack_bf16x2_rne(o[nb][mt][0] * inv, o[nb][mt][1] * inv);
      const uint32_t hi = pack_bf16x2_rne(o[nb][mt][2] * inv, o[nb][mt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * mt) = make_uint2(lo, hi);
    }
    if (a.lse_out && grp == 0)
      a.lse_out[int64_t(row) * Hq + hq] = l > 0.f ? (m[nb] + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int CDT, int D, int BS>
__global__ void __launch_bounds__(256) varlen_kernel(VarlenArgs a) {
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
    if (h * 4 >= a.num_kv_heads) return;
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
      for (int32_t hg = 0; hg * 4 < num_kv_heads; ++hg) v.push_back({s, (kKindDecode << 24) | hg, 0, L, 0});
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
  a.zscale = float(double(scale) * double(k_scale) * 1.4426950408889634);
  a.v_scale = v_scale;
  hipLaunchKernelGGL(fn, dim3(num_work), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefill_varlen: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}
