// paged_attention_decode: one query token per sequence over a paged KV cache.
//
// What is computed follows "Project 17: Production Serving: Continuous Batching and
// PagedAttention", "Step 6: Implement attention over paged storage": walk the
// sequence's page table, score every cached key against the query (scaled), softmax
// over the scores, and sum the cached values with those weights -- per query head,
// with query head h reading KV head h / G.
//
// How it is computed on gfx950 (the page's two-pass loop is replaced):
//  * Work item = (sequence s, KV head g, context partition p). A workgroup of NW
//    wave64s owns one item; its blocks are dealt round-robin to the waves.
//  * GQA packing: the G query heads of KV head g are held in registers together, so
//    each K/V element loaded from HBM serves all G heads.
//  * Gather: a block id comes from the block table (wave-uniform, scalar load); each
//    lane then loads 16 bytes (8 bytes for E4M3) of one token's [head_dim] row. A
//    token row is LPT lanes wide, so one load instruction covers TPL = 64/LPT tokens.
//  * Scores: per-lane partial dot products, summed over the LPT lanes of a token with
//    DPP row operations (no LDS).
//  * Online softmax per row group (the lanes sharing a token slot): running max m,
//    running sum l and a [G][EPL] accumulator, rescaled once per 16-token tile. Row
//    groups, then waves, are merged by log-sum-exp at the end (shuffles, then LDS).
//  * Split context: with partition_size > 0 a sequence longer than one partition
//    writes per-partition (normalised output, log-sum-exp) partials and a second
//    kernel merges them; a sequence that fits in one partition writes its output
//    directly.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "pkv.h"
#include "pkv_internal.h"
#include "mfma_common.h"
#include "decode_split.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxPartitions = 65535;

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Cache element traits: bytes per lane per load, elements per lane per load.
template <int CDT>
struct Cache;
template <>
struct Cache<PKV_F32> {
  static constexpr int EPL = 4;
  using Vec = uint4;
};
template <>
struct Cache<PKV_BF16> {
  static constexpr int EPL = 8;
  using Vec = uint4;
};
template <>
struct Cache<PKV_FP8_E4M3> {
  static constexpr int EPL = 8;
  using Vec = uint2;
};

template <int CDT>
__device__ __forceinline__ void unpack(const typename Cache<CDT>::Vec& x, float (&f)[Cache<CDT>::EPL]) {
  if constexpr (CDT == PKV_F32) {
    f[0] = __uint_as_float(x.x);
    f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z);
    f[3] = __uint_as_float(x.w);
  } else if constexpr (CDT == PKV_BF16) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = pkv::bf16_lo(w[j]);
      f[2 * j + 1] = pkv::bf16_hi(w[j]);
    }
  } else {
    const uint32_t w[2] = {x.x, x.y};
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = pkv::fp8_to_f32(w[j >> 2] >> (8 * (j & 3)));
  }
}

template <int CDT>
__device__ __forceinline__ typename Cache<CDT>::Vec zero_vec() {
  if constexpr (CDT == PKV_FP8_E4M3)
    return make_uint2(0, 0);
  else
    return make_uint4(0, 0, 0, 0);
}

using namespace pkv::split;

// The (sequence, partition) of this workgroup and its token range; false = nothing to do.
__device__ __forceinline__ bool locate_item(const DecodeArgs& a, int& s, int& p, int& nparts, int& tok_begin,
                                            int& tok_end) {
  if (a.work) {
    const int4 it = a.work[blockIdx.y];
    s = it.x;
    p = it.y;
    nparts = it.z;
    // malformed item (bad index, or split without a workspace): skip
    if (s < 0 || s >= a.num_seqs || p < 0 || p >= a.pmax || nparts < 1 || p >= nparts ||
        (nparts > 1 && !a.ws_o))
      return false;
    tok_end = it.w < 0 ? 0 : (it.w > a.len_clamp ? a.len_clamp : it.w);
    tok_begin = a.part_tokens > 0 ? p * a.part_tokens : 0;
    if (tok_begin > tok_end) tok_begin = tok_end;
    return true;
  }
  s = blockIdx.z;
  p = blockIdx.y;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_clamp ? a.len_clamp : L);
  tok_begin = 0;
  tok_end = L;
  nparts = 1;
  if (a.part_tokens > 0) {
    nparts = (L + a.part_tokens - 1) / a.part_tokens;
    if (nparts < 1) nparts = 1;
    if (p >= nparts) return false;
    tok_begin = p * a.part_tokens;
    tok_end = min(L, tok_begin + a.part_tokens);
  }
  return true;
}

template <int QDT, int CDT, int D, int G, int BS, int NW>
__global__ void __launch_bounds__(NW * 64) decode_kernel(DecodeArgs a) {
  using Vec = typename Cache<CDT>::Vec;
  constexpr int EPL = Cache<CDT>::EPL;
  constexpr int LPT = D / EPL;                 // lanes per token row
  constexpr int TPL = 64 / LPT;                // tokens per load instruction
  constexpr int TILE = BS < 16 ? BS : 16;      // tokens per softmax update
  constexpr int NLT = TILE / TPL;              // loads per tile (each of K and V)
  constexpr int SUB = BS / TILE;               // tiles per block
  constexpr bool DOT2 = (QDT == PKV_BF16 && CDT == PKV_BF16);
  static_assert(NLT >= 1 && TILE % TPL == 0, "tile too small for this row width");

  const int g = blockIdx.x;
  const float zscale_g = a.zscale_h[g & (pkv::kHeadScales - 1)];
  const float vscale_g = a.vscale_h[g & (pkv::kHeadScales - 1)];
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane / LPT;
  const int c = lane % LPT;
  int s, p, nparts, tok_begin, tok_end;
  if (!locate_item(a, s, p, nparts, tok_begin, tok_end)) return;
  const int blk_begin = tok_begin / BS;
  const int blk_end = (tok_end + BS - 1) / BS;

  // ---- queries of the G packed heads, this lane's EPL-wide slice of head_dim
  constexpr int QW = DOT2 ? EPL / 2 : EPL;     // words (bf16 pairs) or floats per head
  float qf[DOT2 ? 1 : G][DOT2 ? 1 : EPL];
  uint32_t qp[DOT2 ? G : 1][DOT2 ? QW : 1];
  {
    const int64_t qbase = (int64_t(s) * Hq + int64_t(g) * G) * D + c * EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (QDT == PKV_F32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qbase + h * D);
        qf[h][0] = v.x;
        qf[h][1] = v.y;
        qf[h][2] = v.z;
        qf[h][3] = v.w;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qbase + h * D);
        if constexpr (DOT2) {
          qp[h][0] = v.x;
          qp[h][1] = v.y;
          qp[h][2] = v.z;
          qp[h][3] = v.w;
        } else {
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            qf[h][2 * j] = pkv::bf16_lo(wv[j]);
            qf[h][2 * j + 1] = pkv::bf16_hi(wv[j]);
          }
        }
      }
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const Vec* kc = static_cast<const Vec*>(a.k_cache);
  const Vec* vc = static_cast<const Vec*>(a.v_cache);
  const int64_t row_vecs = int64_t(Hkv) * LPT;          // Vec units per token row
  const int64_t lane_off = int64_t(g) * LPT + c;        // this lane's Vec within the row
  const int32_t* bt_row = a.block_tables + int64_t(s) * a.table_width;

  // tiles owned by this wave: block j = blk_begin + w + NW*(n / SUB), sub-tile n % SUB
  const int my_blocks = blk_end - blk_begin > w ? (blk_end - blk_begin - w + NW - 1) / NW : 0;
  const int ntiles = my_blocks * SUB;

  Vec kb[2][NLT], vb[2][NLT];
  int tok0[2];
  bool okb[2];

  auto issue = [&](int n, Vec (&kr)[NLT], Vec (&vr)[NLT], int& t0, bool& ok) {
    const int j = blk_begin + w + NW * (n / SUB);
    const int sub = n % SUB;
    const int blk = __builtin_amdgcn_readfirstlane(bt_row[j]);
    ok = blk >= 0 && blk < a.num_blocks;
    t0 = j * BS + sub * TILE;
    const int64_t base = (int64_t(ok ? blk : 0) * BS + sub * TILE + r) * row_vecs + lane_off;
#pragma unroll
    for (int i = 0; i < NLT; ++i) {
      if (ok) {
        kr[i] = kc[base + int64_t(i) * TPL * row_vecs];
        vr[i] = vc[base + int64_t(i) * TPL * row_vecs];
      } else {
        kr[i] = zero_vec<CDT>();
        vr[i] = zero_vec<CDT>();
      }
    }
  };

  auto consume = [&](const Vec (&kr)[NLT], const Vec (&vr)[NLT], int t0, bool ok) {
    float z[NLT][G];
    bool valid[NLT];
#pragma unroll
    for (int i = 0; i < NLT; ++i) {
      const int t = t0 + i * TPL + r;
      valid[i] = ok && t < tok_end;
      float part[G];
      if constexpr (DOT2) {
        const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float sacc = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) sacc = dot2_bf16(qp[h][j], kw[j], sacc);
          part[h] = sacc;
        }
      } else {
        float kf[EPL];
        unpack<CDT>(kr[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float sacc = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) sacc = fmaf(qf[h][e], kf[e], sacc);
          part[h] = sacc;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float zz = pkv::group_sum<LPT>(part[h]) * zscale_g;
        z[i][h] = valid[i] ? zz : -INFINITY;
      }
    }
    // online softmax update, once per tile
    float pw[NLT][G];
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mt = z[0][h];
#pragma unroll
      for (int i = 1; i < NLT; ++i) mt = fmaxf(mt, z[i][h]);
      const float mn = fmaxf(m[h], mt);
      const float mref = mn == -INFINITY ? 0.f : mn;
      alpha[h] = pkv::fast_exp2(m[h] - mref);
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < NLT; ++i) {
        pw[i][h] = pkv::fast_exp2(z[i][h] - mref);
        ls += pw[i][h];
      }
      l[h] = l[h] * alpha[h] + ls;
      m[h] = mn;
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
#pragma unroll
    for (int i = 0; i < NLT; ++i) {
      float vf[EPL];
      unpack<CDT>(vr[i], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[e] = valid[i] ? vf[e] : 0.f;   // masked slots may hold NaN
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw[i][h], vf[e], acc[h][e]);
    }
  };

  if (ntiles > 0) {
    issue(0, kb[0], vb[0], tok0[0], okb[0]);
    int n = 0;
    for (; n + 1 < ntiles; n += 2) {
      issue(n + 1, kb[1], vb[1], tok0[1], okb[1]);
      consume(kb[0], vb[0], tok0[0], okb[0]);
      if (n + 2 < ntiles) issue(n + 2, kb[0], vb[0], tok0[0], okb[0]);
      consume(kb[1], vb[1], tok0[1], okb[1]);
    }
    if (n < ntiles) consume(kb[0], vb[0], tok0[0], okb[0]);
  }

  // ---- merge the TPL row groups of the wave (lanes with equal c)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float wa = pkv::fast_exp2(m[h] - mref);
      const float wb = pkv::fast_exp2(mo - mref);
      l[h] = l[h] * wa + lo * wb;
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * wa + ao * wb;
      }
    }
  }

  // ---- merge the NW waves through LDS
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ float sm_acc[NW][G][D];
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) {
        sm_m[w][h] = m[h];
        sm_l[w][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_acc[w][h][c * EPL + e] = acc[h][e];
    }
  }
  __syncthreads();

  const bool single = nparts == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int e = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < NW; ++x) M = fmaxf(M, sm_m[x][h]);
    const float mref = M == -INFINITY ? 0.f : M;
    float S = 0.f, A = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const float wx = pkv::fast_exp2(sm_m[x][h] - mref);
      S += sm_l[x][h] * wx;
      A += sm_acc[x][h][e] * wx;
    }
    const float o = S > 0.f ? A / S * vscale_g : 0.f;
    const float lse2 = S > 0.f ? M + log2f(S) : -INFINITY;
    const int hq = g * G + h;
    if (single) {
      const int64_t oi = (int64_t(s) * Hq + hq) * D + e;
      if constexpr (QDT == PKV_F32)
        static_cast<float*>(a.out)[oi] = o;
      else
        static_cast<uint16_t*>(a.out)[oi] = uint16_t(pkv::f32_to_bf16(o));
      if (a.lse_out && e == 0) a.lse_out[int64_t(s) * Hq + hq] = lse2 * kLn2;
    } else {
      const int64_t pi = (int64_t(s) * Hq + hq) * a.pmax + p;
      a.ws_o[pi * D + e] = o;
      if (e == 0) a.ws_lse[pi] = lse2;
    }
  }
}

constexpr int kMergeFast = 4;      // pieces merged with all loads in flight at once

// Log-sum-exp merge of the partition partials. A workgroup of 4 waves takes HW query
// heads of one sequence; D/4 lanes own one head, 4 consecutive head_dim elements each
// (16-byte loads): M = max_k lse_k, out = sum_k 2^(lse_k - M) o_k / sum_k 2^(lse_k - M).
template <int QDT, int D>
__global__ void __launch_bounds__(256) merge_kernel(DecodeArgs a, int num_q_heads) {
  constexpr int LPH = D / 4;                  // lanes per head
  constexpr int HW = 256 / LPH;               // heads per workgroup
  const int s = blockIdx.y;
  const int hq = blockIdx.x * HW + threadIdx.x / LPH;
  const int e = 4 * (threadIdx.x % LPH);
  if (hq >= num_q_heads) return;
  const int orow_idx = s;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_clamp ? a.len_clamp : L);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;                    // written directly by the partition pass
  const int64_t base = (int64_t(s) * num_q_heads + hq) * a.pmax;
  auto piece = [&](int k) -> int64_t { return base + k; };
  float M = -INFINITY, S = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  if (nparts <= kMergeFast) {
    // few pieces (the usual case): every load issued at once, one memory round trip;
    // slots past nparts re-read piece 0 and are dropped
    float lse[kMergeFast];
    float4 ov[kMergeFast];
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k) {
      const int64_t pi = piece(k < nparts ? k : 0);
      lse[k] = a.ws_lse[pi];
      ov[k] = *reinterpret_cast<const float4*>(a.ws_o + pi * D + e);
    }
    __builtin_amdgcn_sched_barrier(0);                    // all loads issued before any use
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k) M = k < nparts ? fmaxf(M, lse[k]) : M;
    const float mref = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int k = 0; k < kMergeFast; ++k) {
      const float wk = k < nparts ? pkv::fast_exp2(lse[k] - mref) : 0.f;   // 0 for an empty piece
      S += wk;
      A.x = fmaf(wk, ov[k].x, A.x);
      A.y = fmaf(wk, ov[k].y, A.y);
      A.z = fmaf(wk, ov[k].z, A.z);
      A.w = fmaf(wk, ov[k].w, A.w);
    }
  } else {
    // pass 1: the maximum log-sum-exp; pass 2: independent weighted loads (unrolled)
#pragma unroll 8
    for (int k = 0; k < nparts; ++k) M = fmaxf(M, a.ws_lse[piece(k)]);
    const float mref = M == -INFINITY ? 0.f : M;
#pragma unroll 4
    for (int k = 0; k < nparts; ++k) {
      const int64_t pi = piece(k);
      const float wk = pkv::fast_exp2(a.ws_lse[pi] - mref);   // 0 for an empty partition
      const float4 ok = *reinterpret_cast<const float4*>(a.ws_o + pi * D + e);
      S += wk;
      A.x = fmaf(wk, ok.x, A.x);
      A.y = fmaf(wk, ok.y, A.y);
      A.z = fmaf(wk, ok.z, A.z);
      A.w = fmaf(wk, ok.w, A.w);
    }
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  const float r[4] = {A.x * inv, A.y * inv, A.z * inv, A.w * inv};
  const int64_t oi = (int64_t(orow_idx) * num_q_heads + hq) * D + e;
  if constexpr (QDT == PKV_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oi) = make_float4(r[0], r[1], r[2], r[3]);
  } else {
    const uint32_t lo = pkv::f32_to_bf16(r[0]) | (pkv::f32_to_bf16(r[1]) << 16);
    const uint32_t hi = pkv::f32_to_bf16(r[2]) | (pkv::f32_to_bf16(r[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + oi) = make_uint2(lo, hi);
  }
  if (a.lse_out && e == 0)
    a.lse_out[int64_t(orow_idx) * num_q_heads + hq] = (S > 0.f ? M + log2f(S) : -INFINITY) * kLn2;
}

// Log-sum-exp merge of the sequences a balanced split cut across slots: workgroup (s, y)
// takes plan row s when its pieces span np >= 2 slots f .. f + np - 1 (one scalar load of
// the plan's (first slot, pieces) pair; the other rows leave at once), and 256 of its
// Hq x D / 4 float4 output chunks, one per thread: M = max_k lse_k, out = sum_k
// 2^(lse_k - M) o_k / sum_k 2^(lse_k - M) over its pieces (the partials o_k are
// normalised). The output row's lookups are issued before the partial loads, and pieces
// are loaded KB at a time (8, or 32 when some sequence spans more than 8 slots), so a
// sequence's pieces usually take one memory round trip after the plan's.
template <int D, int KB>
__global__ void __launch_bounds__(256) split_merge_kernel(DecodeArgs a, int num_q_heads) {
  constexpr int CH = D / 4;
  typedef __attribute__((address_space(4))) const int32_t* cptr;
  const int s = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  const int B = a.num_seqs;
  if (s >= B || c >= num_q_heads * CH || !a.ws_o) return;
  const LayerPtrs lp = layer_ptrs(a);
  const cptr plan = (cptr)(uintptr_t)(a.plan);
  const cptr seq_slots = plan + (B + 1) + 2 * a.num_slots + 1;
  const int f = seq_slots[2 * s], np = seq_slots[2 * s + 1];
  if (np < 2 || f < 0 || f + np > a.num_slots) return;
  int b, row;
  split_row(a, s, b, row);
  const int hq = c / CH, d0 = 4 * (c % CH);
  float M = -INFINITY, S = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < np; k0 += KB) {
    float lse[KB];
    float4 ov[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int kk = k0 + k < np ? k0 + k : k0;
      const int64_t pi = split_partial(f + kk, kk, num_q_heads, hq);
      lse[k] = lp.ws_lse[pi];
      ov[k] = *reinterpret_cast<const float4*>(lp.ws_o + pi * D + d0);
    }
    // every load above is issued before any use below (left alone, the scheduler folds
    // each value into the maximum as it arrives: one memory round trip per piece)
    __builtin_amdgcn_sched_barrier(0);
    float Mb = M;
#pragma unroll
    for (int k = 0; k < KB; ++k) Mb = k0 + k < np ? fmaxf(Mb, lse[k]) : Mb;
    const float mref = Mb == -INFINITY ? 0.f : Mb;
    const float r = M == -INFINITY ? 0.f : pkv::fast_exp2(M - mref);
    S *= r;
    A.x *= r;
    A.y *= r;
    A.z *= r;
    A.w *= r;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float wk = k0 + k < np ? pkv::fast_exp2(lse[k] - mref) : 0.f;
      S += wk;
      A.x = fmaf(wk, ov[k].x, A.x);
      A.y = fmaf(wk, ov[k].y, A.y);
      A.z = fmaf(wk, ov[k].z, A.z);
      A.w = fmaf(wk, ov[k].w, A.w);
    }
    M = Mb;
  }
  if (row < 0) return;
  const float inv = S > 0.f ? 1.f / S : 0.f;
  const uint32_t lo = pkv::f32_to_bf16(A.x * inv) | (pkv::f32_to_bf16(A.y * inv) << 16);
  const uint32_t hi = pkv::f32_to_bf16(A.z * inv) | (pkv::f32_to_bf16(A.w * inv) << 16);
  *reinterpret_cast<uint2*>(lp.out + (int64_t(row) * num_q_heads + hq) * D + d0) = make_uint2(lo, hi);
  if (lp.lse && d0 == 0)
    lp.lse[int64_t(row) * num_q_heads + hq] = (S > 0.f ? M + log2f(S) : -INFINITY) * kLn2;
}

// ---------------------------------------------------------------------------------
// MFMA decode (bf16 queries; bf16 or E4M3 cache).
//
// One wave owns 16-token tiles. Lane l works for query head slot hl = l % 16 (slots
// >= G are zero padding) and lane group grp = l / 16.
//  * K tile -> registers: in load i, lane l reads 16 bytes of token hl's head row at
//    byte 64*i + 16*grp, so each load instruction covers 64 contiguous bytes of each of
//    16 token rows. Those registers are directly the A operand of
//    v_mfma_f32_16x16x32_bf16 (A[token][k]); the packed queries are the B operand with
//    the same head_dim permutation. Result: lane l holds the scores of head hl for
//    tokens 4*grp .. 4*grp+3.
//  * Online softmax is lane-local per head (tile max over the 4 lane groups by two
//    shuffles). exp2 of the scores, rounded to bf16, is already the B operand of
//    v_mfma_f32_16x16x16_bf16 for P^T (tokens 4*grp+j, head hl).
//  * V tile -> LDS ([token][head_dim], padded rows), read back with ds_read_b64_tr_b16
//    as V^T fragments (d = 16*mt + hl, tokens 4*grp+j): the A operand. The output
//    O^T accumulates in lane l for head hl, d = 16*mt + 4*grp + r: per-head rescaling
//    stays lane-local.
// ---------------------------------------------------------------------------------

using pkv::bf16x8_t;
using pkv::f32x4_t;
using pkv::pack_bf16x2_rne;

template <int CDT, int D, int BS, int HPW>
// Three waves per SIMD: the largest occupancy this kernel reaches without spilling
// (measured register use: 153 VGPRs at this bound, 128 + 66 spilled at four).
__global__ void __launch_bounds__(HPW * 64, 3) decode_mfma_kernel(DecodeArgs a) {
  constexpr int MT = D / 16;
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;
  constexpr int RS = D * 2 + 32;
  // the HPW waves of a workgroup take HPW consecutive KV heads of the same work item,
  // so together they stream whole token rows of every block
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = blockIdx.x * HPW + w;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  int s, p, nparts, tok_begin, tok_end;
  if (!locate_item(a, s, p, nparts, tok_begin, tok_end)) return;

  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[HPW][16 * RS];
  pkv::DecodeWaveIn in;
  in.q = static_cast<const uint16_t*>(a.q) + (int64_t(s) * Hq + int64_t(g) * G) * D;
  in.G = G;
  in.kc = static_cast<const uint8_t*>(a.k_cache);
  in.vc = static_cast<const uint8_t*>(a.v_cache);
  in.row_bytes = int64_t(Hkv) * D * EB;
  in.head_off = int64_t(g) * D * EB;
  in.bt_row = a.block_tables + int64_t(s) * a.table_width;
  in.num_blocks = a.num_blocks;
  in.tok_begin = tok_begin;
  in.tok_end = tok_end;
  in.zscale = a.zscale_h[__builtin_amdgcn_readfirstlane(g) & (pkv::kHeadScales - 1)];
  float m, lsum;
  f32x4_t o[MT];
  pkv::decode_wave<CDT, D, BS>(in, vt_lds[w], m, lsum, o);


  if (hl < G) {
    const int hq = g * G + hl;
    const float inv = lsum > 0.f ? a.vscale_h[__builtin_amdgcn_readfirstlane(g) & (pkv::kHeadScales - 1)] / lsum : 0.f;
    const float lse2 = lsum > 0.f ? m + log2f(lsum) : -INFINITY;
    if (nparts == 1) {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + (int64_t(s) * Hq + hq) * D + 4 * grp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t lo = pack_bf16x2_rne(o[mt][0] * inv, o[mt][1] * inv);
        const uint32_t hi = pack_bf16x2_rne(o[mt][2] * inv, o[mt][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * mt) = make_uint2(lo, hi);
      }
      if (a.lse_out && grp == 0) a.lse_out[int64_t(s) * Hq + hq] = lse2 * kLn2;
    } else {
      const int64_t pi = (int64_t(s) * Hq + hq) * a.pmax + p;
      float* orow = a.ws_o + pi * D + 4 * grp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<float4*>(orow + 16 * mt) =
            make_float4(o[mt][0] * inv, o[mt][1] * inv, o[mt][2] * inv, o[mt][3] * inv);
      if (grp == 0) a.ws_lse[pi] = lse2;
    }
  }
}

// The balanced-split decode pass: one workgroup per (KV-head group, slot, layer).
template <int CDT, int D, int BS, int HPW, int NS = kSplitRing, int TPS = 1>
__global__ void __launch_bounds__(HPW * 64, 2) decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[split_lds_bytes<CDT, D, HPW, TPS>()];
  decode_split_body<CDT, D, BS, HPW, NS, TPS>(a, lds, blockIdx.x, blockIdx.y, blockIdx.z);
}

constexpr int kWaves = 4;

thread_local hipEvent_t g_profile_event = nullptr;

using DecodeFn = void (*)(DecodeArgs);
using MergeFn = void (*)(DecodeArgs, int);

template <int QDT, int CDT, int D, int BS>
DecodeFn pick_g(int G) {
  switch (G) {
    case 1: return decode_kernel<QDT, CDT, D, 1, BS, kWaves>;
    case 2: return decode_kernel<QDT, CDT, D, 2, BS, kWaves>;
    case 4: return decode_kernel<QDT, CDT, D, 4, BS, kWaves>;
    case 8: return decode_kernel<QDT, CDT, D, 8, BS, kWaves>;
    default: return nullptr;
  }
}

template <int QDT, int CDT, int D>
DecodeFn pick_bs(int G, int BS) {
  switch (BS) {
    case 16: return pick_g<QDT, CDT, D, 16>(G);
    case 32: return pick_g<QDT, CDT, D, 32>(G);
    default: return nullptr;
  }
}

template <int QDT, int CDT>
DecodeFn pick_d(int D, int G, int BS) {
  switch (D) {
    case 64: return pick_bs<QDT, CDT, 64>(G, BS);
    case 128: return pick_bs<QDT, CDT, 128>(G, BS);
    default: return nullptr;
  }
}

template <int CDT, int D, int HPW>
DecodeFn pick_mfma_bs(int BS) {
  switch (BS) {
    case 16: return decode_mfma_kernel<CDT, D, 16, HPW>;
    case 32: return decode_mfma_kernel<CDT, D, 32, HPW>;
    default: return nullptr;
  }
}

template <int CDT, int HPW>
DecodeFn pick_mfma(int D, int BS) {
  switch (D) {
    case 64: return pick_mfma_bs<CDT, 64, HPW>(BS);
    case 128: return pick_mfma_bs<CDT, 128, HPW>(BS);
    default: return nullptr;
  }
}

template <int CDT, int D, int HPW>
DecodeFn pick_split_bs(int BS) {
  switch (BS) {
    case 16: return decode_split_kernel<CDT, D, 16, HPW, kSplitRing, split_tps(CDT, D)>;
    case 32: return decode_split_kernel<CDT, D, 32, HPW, kSplitRing, split_tps(CDT, D)>;
    default: return nullptr;
  }
}

template <int CDT, int HPW>
DecodeFn pick_split(int D, int BS) {
  switch (D) {
    case 64: return pick_split_bs<CDT, 64, HPW>(BS);
    case 128: return pick_split_bs<CDT, 128, HPW>(BS);
    default: return nullptr;
  }
}

template <int CDT>
DecodeFn pick_split_hpw(int D, int BS, int hpw) {
  switch (hpw) {
    case 1: return pick_split<CDT, 1>(D, BS);
    case 2: return pick_split<CDT, 2>(D, BS);
    case 4: return pick_split<CDT, 4>(D, BS);
    case 8: return pick_split<CDT, 8>(D, BS);
    default: return nullptr;
  }
}

// Resident workgroups of `fn` per CU times the CU count (cached per device and kernel).
int resident_slots(DecodeFn fn, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), threads, 0) !=
      hipSuccess)
    return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

template <int CDT>
DecodeFn pick_mfma_hpw(int D, int BS, int hpw) {
  switch (hpw) {
    case 1: return pick_mfma<CDT, 1>(D, BS);
    case 2: return pick_mfma<CDT, 2>(D, BS);
    case 4: return pick_mfma<CDT, 4>(D, BS);
    case 8: return pick_mfma<CDT, 8>(D, BS);
    default: return nullptr;
  }
}

// KV heads per workgroup for the MFMA kernel: the largest of 8, 4, 2, 1 dividing Hkv
// (measured on the 256-sequence batch: 8 heads 5.23 TB/s, 4 heads 5.20, 2 heads 4.13,
// 1 head 3.73 with the earlier load layout; whole token rows per workgroup stream best).
int mfma_heads_per_wg(int Hkv) {
  for (int h : {8, 4, 2})
    if (Hkv % h == 0) return h;
  return 1;
}

// fp32 -> the VALU kernel (fp32 products, four waves per work item); bf16 queries ->
// the MFMA kernel (one wave per KV head, *waves heads per workgroup).
DecodeFn pick_decode(int qdt, int cdt, int D, int G, int BS, int Hkv, int* waves) {
  if (qdt == PKV_F32 && cdt == PKV_F32) {
    *waves = kWaves;
    return pick_d<PKV_F32, PKV_F32>(D, G, BS);
  }
  if (qdt != PKV_BF16 || (cdt != PKV_BF16 && cdt != PKV_FP8_E4M3) || G < 1 || G > 16) return nullptr;
  *waves = mfma_heads_per_wg(Hkv);
  return cdt == PKV_BF16 ? pick_mfma_hpw<PKV_BF16>(D, BS, *waves) : pick_mfma_hpw<PKV_FP8_E4M3>(D, BS, *waves);
}

MergeFn pick_merge(int qdt, int D) {
  if (qdt == PKV_F32) return D == 64 ? merge_kernel<PKV_F32, 64> : merge_kernel<PKV_F32, 128>;
  return D == 64 ? merge_kernel<PKV_BF16, 64> : merge_kernel<PKV_BF16, 128>;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int64_t partitions_for(int32_t max_seq_len, int32_t partition_size) {
  if (partition_size <= 0 || max_seq_len <= 0) return 1;
  return (int64_t(max_seq_len) + partition_size - 1) / partition_size;
}

}  // namespace

extern "C" void pkv_decode_set_profile_event(void* hip_event) {
  g_profile_event = static_cast<hipEvent_t>(hip_event);
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                             int32_t max_seq_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || partition_size <= 0) return 0;
  const int64_t pmax = partitions_for(max_seq_len, partition_size);
  if (pmax <= 1) return 0;
  return size_t(num_seqs) * num_q_heads * pmax * (head_dim + 1) * sizeof(float);
}

extern "C" int pkv_paged_attention_decode(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                          const void* v_cache, int32_t cache_dtype, const int32_t* block_tables,
                                          const int32_t* seq_lens, int32_t table_width, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                                          float scale, float k_scale, float v_scale,
                                          const float* k_head_scales, const float* v_head_scales,
                                          int32_t partition_size, void* workspace, size_t workspace_bytes, float* lse_out,
                                          const int32_t* work_items, int32_t num_work, void* stream) {
  using pkv::fail;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || table_width < 0 || num_blocks < 0 ||
      max_seq_len < 0 || partition_size < 0)
    return fail(PKV_ERR_INVALID, "decode: bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "decode: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  if (num_seqs > 65535) return fail(PKV_ERR_INVALID, "decode: at most 65535 sequences per launch");
  const int G = num_q_heads / num_kv_heads;
  int waves = kWaves;
  DecodeFn fn = pick_decode(q_dtype, cache_dtype, head_dim, G, block_size, num_kv_heads, &waves);
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED,
                "decode: unsupported (q dtype %d, cache dtype %d, head_dim %d, group %d, block_size %d)", q_dtype,
                cache_dtype, head_dim, G, block_size);
  if (partition_size > 0 && partition_size % block_size != 0)
    return fail(PKV_ERR_INVALID, "decode: partition_size %d not a multiple of block_size %d", partition_size,
                block_size);
  if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PKV_ERR_INVALID, "decode: scales must be > 0");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return fail(PKV_ERR_INVALID, "decode: NULL pointer");
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "decode: the cache has no blocks");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID, "decode: q, out and cache planes must be 16-byte aligned");
  int64_t pmax = partitions_for(max_seq_len, partition_size);
  if (pmax > kMaxPartitions)
    return fail(PKV_ERR_INVALID, "decode: %lld partitions exceed %d", (long long)pmax, kMaxPartitions);
  const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_INVALID, "decode: workspace of %zu bytes needed, %zu given", need, workspace_bytes);

  DecodeArgs a{};
  a.q = q;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.lse_out = lse_out;
  a.table_width = table_width;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  const int64_t tcap = int64_t(table_width) * block_size;
  a.len_clamp = int(tcap < max_seq_len ? tcap : max_seq_len);
  a.part_tokens = need > 0 ? partition_size : 0;
  a.pmax = need > 0 ? int(pmax) : 1;
  if (need > 0) {
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = a.ws_o + size_t(num_seqs) * num_q_heads * pmax * head_dim;
  }
  {
    const int rc = pkv::head_scales("attention", num_kv_heads, scale, k_scale, v_scale, k_head_scales,
                                    v_head_scales, a.zscale_h, a.vscale_h);
    if (rc != PKV_OK) return rc;
  }
  a.group = G;
  a.num_seqs = num_seqs;
  const bool mfma = q_dtype == PKV_BF16;
  const int head_groups = mfma ? num_kv_heads / waves : num_kv_heads;
  dim3 grid(head_groups, a.pmax, num_seqs);
  if (work_items) {
    if (num_work <= 0 || num_work > 2147483647 / 4)
      return fail(PKV_ERR_INVALID, "decode: num_work %d out of range", num_work);
    if ((reinterpret_cast<uintptr_t>(work_items) & 15) != 0)
      return fail(PKV_ERR_INVALID, "decode: work_items must be 16-byte aligned");
    a.work = reinterpret_cast<const int4*>(work_items);
    a.num_work = num_work;
    grid = dim3(head_groups, num_work, 1);
    if (num_work > 65535 * 32) return fail(PKV_ERR_INVALID, "decode: too many work items");
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(fn, grid, dim3(waves * 64), 0, st, a);
  if (g_profile_event) (void)hipEventRecord(g_profile_event, st);
  if (need > 0) {
    MergeFn mf = pick_merge(q_dtype, head_dim);
    const int heads_per_wg = 256 / (head_dim / 4);
    hipLaunchKernelGGL(mf, dim3((num_q_heads + heads_per_wg - 1) / heads_per_wg, num_seqs), dim3(256), 0, st, a,
                       num_q_heads);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int pkv_decode_split_slots(int32_t cache_dtype, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t* slots) {
  using pkv::fail;
  if (!slots || num_kv_heads <= 0) return fail(PKV_ERR_INVALID, "decode_split_slots: bad arguments");
  const int hpw = mfma_heads_per_wg(num_kv_heads);
  DecodeFn fn = cache_dtype == PKV_BF16       ? pick_split_hpw<PKV_BF16>(head_dim, block_size, hpw)
                : cache_dtype == PKV_FP8_E4M3 ? pick_split_hpw<PKV_FP8_E4M3>(head_dim, block_size, hpw)
                                              : nullptr;
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "decode_split_slots: unsupported (cache dtype %d, head_dim %d, block_size %d)",
                cache_dtype, head_dim, block_size);
  const int resident = resident_slots(fn, hpw * 64);
  if (resident <= 0) return fail(PKV_ERR_HIP, "decode_split_slots: occupancy query failed");
  *slots = std::max(1, resident / (num_kv_heads / hpw));
  return PKV_OK;
}

extern "C" size_t pkv_decode_split_workspace_bytes(int32_t num_slots, int32_t num_q_heads, int32_t head_dim,
                                                   int32_t max_pieces) {
  if (num_slots <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_pieces <= 1) return 0;
  // partials [S][2][Hq][D] and their log-sum-exps [S][2][Hq], float; rounded up to 256
  // bytes so that the layers of a layer-batched call sit at multiples of it
  const size_t b = size_t(2) * num_slots * num_q_heads * (head_dim + 1) * sizeof(float);
  return (b + 255) / 256 * 256;
}

extern "C" int pkv_paged_attention_decode_split(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                                const void* v_cache, int32_t cache_dtype,
                                                const int32_t* block_tables, const int32_t* seq_lens,
                                                int32_t table_width, int32_t num_seqs, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale,
                                                float v_scale, const float* k_head_scales,
                                                const float* v_head_scales, const int32_t* rows, int32_t num_rows,
                                                const int32_t* cu_seqlens_q, int32_t total_q,
                                                const int32_t* plan, int32_t num_slots,
                                                int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
                                                size_t workspace_bytes, float* lse_out, void* stream) {
  return pkv::decode_split(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, table_width,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                           k_scale, v_scale, k_head_scales, v_head_scales, rows, num_rows, cu_seqlens_q, total_q,
                           plan, num_slots, tiles_per_slot, max_pieces, workspace, workspace_bytes, lse_out,
                           pkv::Layers{}, stream);
}

extern "C" int pkv_paged_attention_decode_split_layers(
    void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache, int32_t cache_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_seq_len, float scale, float k_scale, float v_scale, const float* k_head_scales,
    const float* v_head_scales, const int32_t* rows, int32_t num_rows, const int32_t* cu_seqlens_q, int32_t total_q,
    const int32_t* plan, int32_t num_slots, int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
    size_t workspace_bytes, float* lse_out, const pkv_layers* layers, void* stream) {
  pkv::Layers ls;
  const int rc = pkv::layers_from("decode_split_layers", layers, true,
                                  pkv::kLayerIn | pkv::kLayerOut | pkv::kLayerCache | (lse_out ? pkv::kLayerLse : 0u),
                                  &ls);
  if (rc != PKV_OK) return rc;
  return pkv::decode_split(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, table_width,
                           num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale,
                           k_scale, v_scale, k_head_scales, v_head_scales, rows, num_rows, cu_seqlens_q, total_q,
                           plan, num_slots, tiles_per_slot, max_pieces, workspace, workspace_bytes, lse_out, ls,
                           stream);
}

int pkv::split::split_prepare(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                      int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale,
                      float v_scale, const float* k_head_scales, const float* v_head_scales, const int32_t* rows,
                      int32_t num_rows, const int32_t* cu_seqlens_q, int32_t total_q, const int32_t* plan,
                      int32_t num_slots, int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
                      size_t workspace_bytes, float* lse_out, const Layers& layers, SplitLaunch* L) {
  using pkv::fail;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || table_width < 0 || num_blocks < 0 ||
      max_seq_len < 0)
    return fail(PKV_ERR_INVALID, "decode_split: bad sizes");
  if (layers.n < 1 || layers.n > 65535) return fail(PKV_ERR_INVALID, "decode_split: bad layer count %d", layers.n);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "decode_split: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  if (num_seqs > 65535) return fail(PKV_ERR_INVALID, "decode_split: at most 65535 sequences per launch");
  const int G = num_q_heads / num_kv_heads;
  if (q_dtype != PKV_BF16 || G > 16)
    return fail(PKV_ERR_UNSUPPORTED, "decode_split: needs bf16 queries and at most 16 query heads per KV head");
  const int hpw = mfma_heads_per_wg(num_kv_heads);
  DecodeFn fn = cache_dtype == PKV_BF16       ? pick_split_hpw<PKV_BF16>(head_dim, block_size, hpw)
                : cache_dtype == PKV_FP8_E4M3 ? pick_split_hpw<PKV_FP8_E4M3>(head_dim, block_size, hpw)
                                              : nullptr;
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "decode_split: unsupported (cache dtype %d, head_dim %d, block_size %d)",
                cache_dtype, head_dim, block_size);
  if (num_slots < 1 || num_slots > 65535 || tiles_per_slot < 1 || max_pieces < 0 || max_pieces > kMaxPartitions)
    return fail(PKV_ERR_INVALID, "decode_split: bad plan sizes (slots %d, tiles per slot %d, pieces %d)", num_slots,
                tiles_per_slot, max_pieces);
  if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PKV_ERR_INVALID, "decode_split: scales must be > 0");
  if (rows ? num_rows < 0 : num_rows != num_seqs)
    return fail(PKV_ERR_INVALID, "decode_split: num_rows %d (rows %s) with %d sequences", num_rows,
                rows ? "given" : "NULL", num_seqs);
  if (cu_seqlens_q ? total_q < 0 : total_q != num_seqs)
    return fail(PKV_ERR_INVALID, "decode_split: total_q %d (cu_seqlens_q %s) with %d sequences", total_q,
                cu_seqlens_q ? "given" : "NULL", num_seqs);
  L->empty = true;
  if (num_rows == 0 || num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !plan)
    return fail(PKV_ERR_INVALID, "decode_split: NULL pointer");
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "decode_split: the cache has no blocks");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID, "decode_split: q, out and cache planes must be 16-byte aligned");
  const size_t need = pkv_decode_split_workspace_bytes(num_slots, num_q_heads, head_dim, max_pieces);
  if (need > 0 && (!workspace || workspace_bytes / size_t(layers.n) < need))
    return fail(PKV_ERR_INVALID, "decode_split: workspace of %d x %zu bytes needed, %zu given", layers.n, need,
                workspace_bytes);

  DecodeArgs a{};
  a.q = q;
  a.out = out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.lse_out = lse_out;
  a.table_width = table_width;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  const int64_t tcap = int64_t(table_width) * block_size;
  a.len_clamp = int(tcap < max_seq_len ? tcap : max_seq_len);
  a.pmax = 1;
  a.num_slots = num_slots;
  if (need > 0) {
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = a.ws_o + size_t(2) * num_slots * num_q_heads * head_dim;
  }
  {
    const int rc = pkv::head_scales("attention", num_kv_heads, scale, k_scale, v_scale, k_head_scales,
                                    v_head_scales, a.zscale_h, a.vscale_h);
    if (rc != PKV_OK) return rc;
  }
  a.group = G;
  a.num_seqs = num_rows;                      // the plan's rows
  a.plan = plan;
  a.rows = rows;
  a.cu_q = cu_seqlens_q;
  a.num_batch = num_seqs;
  a.total_q = total_q;
  a.ls_in = layers.in;
  a.ls_out = layers.out;
  a.ls_cache = layers.cache;
  a.ls_lse = layers.lse;
  a.ls_ws = int64_t(need / sizeof(float));
  L->args = a;
  L->pass = reinterpret_cast<const void*>(fn);
  L->hpw = hpw;
  L->hgroups = num_kv_heads / hpw;
  L->num_slots = num_slots;
  L->layers = layers.n;
  L->num_rows = num_rows;
  L->num_q_heads = num_q_heads;
  L->head_dim = head_dim;
  L->max_pieces = max_pieces;
  L->need = need;
  L->empty = false;
  return PKV_OK;
}

int pkv::split::split_launch_merge(const SplitLaunch& L, hipStream_t st) {
  if (L.empty || L.need == 0) return PKV_OK;
  const int chunks = L.num_q_heads * (L.head_dim / 4);
  auto mk = L.max_pieces <= 8 ? (L.head_dim == 64 ? split_merge_kernel<64, 8> : split_merge_kernel<128, 8>)
                              : (L.head_dim == 64 ? split_merge_kernel<64, 32> : split_merge_kernel<128, 32>);
  hipLaunchKernelGGL(mk, dim3(L.num_rows, (chunks + 255) / 256, L.layers), dim3(256), 0, st, L.args, L.num_q_heads);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "decode_split: merge launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int pkv::decode_split(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                      int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale,
                      float v_scale, const float* k_head_scales, const float* v_head_scales, const int32_t* rows,
                      int32_t num_rows, const int32_t* cu_seqlens_q, int32_t total_q, const int32_t* plan,
                      int32_t num_slots, int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
                      size_t workspace_bytes, float* lse_out, const Layers& layers, void* stream) {
  pkv::split::SplitLaunch L;
  int rc = pkv::split::split_prepare(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens,
                                     table_width, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     num_blocks, max_seq_len, scale, k_scale, v_scale, k_head_scales, v_head_scales,
                                     rows, num_rows, cu_seqlens_q, total_q, plan, num_slots, tiles_per_slot,
                                     max_pieces, workspace, workspace_bytes, lse_out, layers, &L);
  if (rc != PKV_OK || L.empty) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the pass (which also writes zeros for rows without context), then the merge of the
  // sequences it cut across slots (none when no sequence spans two slots); the layers of
  // a layer-batched call are the grid's third dimension
  hipLaunchKernelGGL(reinterpret_cast<DecodeFn>(const_cast<void*>(L.pass)), dim3(L.hgroups, L.num_slots, L.layers),
                     dim3(L.hpw * 64), 0, st, L.args);
  if (g_profile_event) (void)hipEventRecord(g_profile_event, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "decode_split: launch failed: %s", hipGetErrorString(e));
  return pkv::split::split_launch_merge(L, st);
}
