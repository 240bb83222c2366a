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

struct DecodeArgs {
  const void* q;
  void* out;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  // partials: fixed partitions [B][Hq][pmax][D] and [B][Hq][pmax] (log2 domain);
  // balanced split [num_slots][2][Hq][D] and [num_slots][2][Hq] (see decode_split_kernel)
  float* ws_o;
  float* ws_lse;
  float* lse_out;    // [B][Hq] natural log, nullable
  int table_width;
  int num_kv_heads;
  int num_blocks;
  int len_clamp;     // min(max_seq_len, table_width * block_size)
  int part_tokens;   // 0 = whole context in one item
  int pmax;
  float zscale_h[pkv::kHeadScales];   // per KV head: softmax scale * k_scale * log2(e)
  float vscale_h[pkv::kHeadScales];   // per KV head: v_scale
  int group;         // query heads per KV head
  int num_seqs;
  int num_work;      // items in `work`
  const int4* work;  // (seq, partition, partitions, end token) per item, or null: grid over all
  const int32_t* plan;   // balanced split: tile offsets [B + 1], then first sequence per slot
  const int32_t* rows;   // balanced split: batch sequence of each plan row (null: row = sequence)
  const int32_t* cu_q;   // balanced split: the batch's cu_seqlens_q (null: one query row per sequence)
  int num_batch;         // batch sequences (rows of block_tables / seq_lens)
  int total_q;           // query / output rows
  int num_slots;         // balanced split: workgroup slots of the launch
  // balanced split over several layers (blockIdx.z): bytes between layers of q, out and
  // the cache planes, floats between layers of lse_out and of the partials
  int64_t ls_in, ls_out, ls_cache, ls_lse, ls_ws;
};

// The tensors of layer blockIdx.z of a layer-batched balanced-split launch.
struct LayerPtrs {
  const uint16_t* q;
  uint16_t* out;
  const uint8_t* kc;
  const uint8_t* vc;
  float* lse;
  float* ws_o;
  float* ws_lse;
};
__device__ __forceinline__ LayerPtrs layer_ptrs(const DecodeArgs& a) {
  const int64_t l = blockIdx.z;
  LayerPtrs p;
  p.q = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.q) + l * a.ls_in);
  p.out = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.out) + l * a.ls_out);
  p.kc = static_cast<const uint8_t*>(a.k_cache) + l * a.ls_cache;
  p.vc = static_cast<const uint8_t*>(a.v_cache) + l * a.ls_cache;
  p.lse = a.lse_out ? a.lse_out + l * a.ls_lse : nullptr;
  p.ws_o = a.ws_o ? a.ws_o + l * a.ls_ws : nullptr;
  p.ws_lse = a.ws_lse ? a.ws_lse + l * a.ls_ws : nullptr;
  return p;
}

// Partial of one piece of the balanced split, as an index into [num_slots][2][Hq]: a
// sequence spanning slots first..first+np-1 leaves its piece p in slot first + p. Only the
// first and the last piece of a slot can belong to such a sequence, and when both do they
// are the same piece, so the slot keeps two entries: [1] for piece 0 (a sequence that
// starts in the slot and runs past its end) and [0] for the others (a sequence that
// began in an earlier slot). The bound is 2 * slots * heads, whatever the batch.
__device__ __forceinline__ int64_t split_partial(int slot, int piece, int num_q_heads, int hq) {
  return (int64_t(2 * slot + (piece == 0 ? 1 : 0))) * num_q_heads + hq;
}

// Batch sequence and query/output row of plan row s of a balanced split (the decode row
// of a sequence is its last new token); -1 in *row for an index outside the batch.
__device__ __forceinline__ void split_row(const DecodeArgs& a, int s, int& b, int& row) {
  typedef __attribute__((address_space(4))) const int32_t* cptr;
  b = a.rows ? ((cptr)(uintptr_t)(a.rows))[s] : s;
  row = -1;
  if (b < 0 || b >= a.num_batch) return;
  const int r = a.cu_q ? ((cptr)(uintptr_t)(a.cu_q))[b + 1] - 1 : b;
  if (r >= 0 && r < a.total_q) row = r;
}

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

// ---------------------------------------------------------------------------------
// Tiles in each wave's load ring of the balanced-split kernel: while one is consumed,
// NS - 1 are in flight.
constexpr int kSplitRing = 2;
// Tiles folded per softmax step of the balanced-split kernel: two for E4M3 caches, whose
// 16-token tiles carry half the bytes of bf16 ones through the same per-tile work.
constexpr int split_tps(int cdt) { return cdt == PKV_FP8_E4M3 ? 2 : 1; }

// Balanced split decode (bf16 queries; bf16 or E4M3 cache). The context of every
// sequence is cut into 16-token tiles and the tiles of all sequences are laid end to
// end; workgroup slot j streams global tiles [j*C, (j+1)*C), so every slot moves the
// same number of bytes and all finish together, whatever the length mix. The part of
// one sequence inside a slot's range is a piece: a sequence held by one slot is written
// directly, the pieces of a longer one go to the workspace (piece index = slot - first
// slot of the sequence) for the log-sum-exp merge. One wave per KV head (8 heads per
// workgroup stream whole token rows together); the load pipeline runs across piece
// boundaries (the next piece's queries and first tile are in flight while the last
// tile of the current one is consumed). Per-tile work is that of decode_wave.
// ---------------------------------------------------------------------------------
template <int CDT, int D, int BS, int HPW, int NS = kSplitRing, int TPS = 1>
__global__ void __launch_bounds__(HPW * 64, 2) decode_split_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;
  constexpr int MT = D / 16;
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;
  constexpr int NV = (D / 4) * EB / 16;
  constexpr int SUB = BS / 16;
  constexpr int RS = D * 2 + 32;            // LDS row stride of the bf16 V tile
  constexpr int RSK = D * 2 + 16;           // LDS row stride of the bf16 K tile
  // Load shape: HB bytes of this KV head per token row. One load instruction covers LPR
  // lanes x 16 bytes of each of RPI rows: whole 128-byte lines when HB >= 128, so the
  // non-temporal hint never leaves the other half of a line to a later instruction (with
  // half lines per instruction it made the stream slower, with whole lines faster).
  constexpr int HB = D * EB;
  constexpr int LPR = HB >= 128 ? 8 : HB / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int HPR = HB / (16 * LPR);      // loads per group of RPI rows
  constexpr bool kStream = LPR == 8;
  static_assert(NV == (16 / RPI) * HPR, "load shape must cover the tile");
  static_assert(TPS == 1 || TPS == 2, "one or two tiles per step");
  typedef __attribute__((address_space(4))) const int32_t* cptr_i32;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = blockIdx.x * HPW + w;
  const float zscale_g = a.zscale_h[__builtin_amdgcn_readfirstlane(g) & (pkv::kHeadScales - 1)];
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int hl_q = hl < G ? hl : hl % G;
  const int slot = blockIdx.y;
  const LayerPtrs lp = layer_ptrs(a);
  const uint8_t* kc = lp.kc;
  const uint8_t* vc = lp.vc;
  const int64_t row_bytes = int64_t(Hkv) * D * EB;
  const int lrow = lane / LPR;               // row of this lane in each load
  const int lchunk = lane % LPR;             // 16-byte chunk of the head slice
  const int64_t lane_off = int64_t(lrow) * row_bytes + int64_t(g) * HB + 16 * lchunk;
  const int64_t group_step = int64_t(RPI) * row_bytes;

  // per wave: TPS K tiles (16 rows, stride RSK), then TPS V tiles (16 rows, stride RS)
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[HPW][TPS * 16 * (RSK + RS)];
  uint8_t* my_kt = kv_lds[w];
  uint8_t* my_vt = kv_lds[w] + TPS * 16 * RSK;

  // ---- issue cursor: the piece whose tiles are being loaded. Slot j owns global tiles
  // [slot_lo[j], slot_lo[j + 1]) of the sequences' tiles laid end to end; a piece is the
  // part of one sequence inside that range.
  const int B = a.num_seqs;
  const cptr_i32 plan = (cptr_i32)(uintptr_t)(a.plan);
  const cptr_i32 lens = (cptr_i32)(uintptr_t)(a.seq_lens);
  const cptr_i32 slot_lo = plan + B + 1 + a.num_slots;
  const cptr_i32 seq_slots = slot_lo + a.num_slots + 1;          // [B][2]: first slot, pieces
  const int total = plan[B];
  const int lo0 = min(max(slot_lo[slot], 0), total);
  int t = lo0;                                                   // global tile cursor
  const int hi = min(max(slot_lo[slot + 1], lo0), total);
  int cs = plan[B + 1 + slot];                                   // current sequence
  cs = cs < 0 ? 0 : (cs > B ? B : cs);
  int cu_cur = plan[cs];
  int cu_next = cs < B ? plan[cs + 1] : 0x7fffffff;
  int i_row = 0, i_p = 0, i_np = 1, i_te = 0, i_t0 = 0, i_nt = 0, i_n = 0;
  bool i_valid = false;
  cptr_i32 i_bt = nullptr;
  // Queries: a piece's rows are loaded into qtmp when the piece is entered and moved into
  // stage (ordinal mod 2) at the start of the next live issue step, by which time only the
  // loads issued after them are still in flight. Two stages suffice: a step's tiles belong
  // to one piece, and when a piece's queries move in only the other ring slot's step is
  // issued and not consumed, so the piece two ordinals back has been fully consumed. Named
  // register arrays, selected by bit tests: an indexed array would be placed in scratch.
  uint4 qtmp[KS];
  bf16x8_t qs0[KS], qs1[KS];
  int q_stage = 0;                           // stage of the piece being issued
  bool q_pending = false;

  // enters the piece that starts at tile t and loads its queries; false when none is left
  auto enter = [&]() -> bool {
    if (t >= hi) return false;
    while (cs < B && cu_next <= t) {          // skip finished and empty sequences
      ++cs;
      cu_cur = cu_next;
      cu_next = cs < B ? plan[cs + 1] : 0x7fffffff;
    }
    if (cs >= B) return false;
    const int pe = hi < cu_next ? hi : cu_next;
    const int tb = t - cu_cur;               // first tile of the piece within the sequence
    const int nt = pe - t;
    t = pe;
    int b, row;
    split_row(a, cs, b, row);                 // scalar loads: no vector wait at piece entry
    if (row < 0) b = 0;
    int L = lens[b];
    L = L < 0 ? 0 : (L > a.len_clamp ? a.len_clamp : L);
    const int first = seq_slots[2 * cs];
    const int np = seq_slots[2 * cs + 1];
    const int p = slot - first;
    // a piece of an inconsistent plan is streamed masked and not written
    const bool valid = row >= 0 && tb >= 0 && cu_cur >= 0 && p >= 0 && p < np &&
                       (np == 1 || a.ws_o != nullptr);
    i_row = row;
    i_p = p;
    i_np = np;
    i_valid = valid;
    i_t0 = valid ? tb : 0;
    i_te = valid ? min(16 * (tb + nt), L) : 0;
    i_nt = nt;
    i_n = 0;
    i_bt = (cptr_i32)(uintptr_t)(a.block_tables + int64_t(b) * a.table_width);
    // lanes past the group read a duplicate head of it: their columns are never written
    const uint16_t* qrow = lp.q + (int64_t(row < 0 ? 0 : row) * Hq + int64_t(g) * G + hl_q) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      qtmp[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * grp);
    }
    q_pending = true;
    return true;
  };

  // Ring state: NS slots of TPS consecutive tiles of one piece each (the step being
  // consumed and the one in flight); per-tile metadata at index slot * TPS + tile. A step
  // never spans two pieces: when its first tile ends a piece, its second is issued dead.
  static_assert(NS == 2, "ring of 2 steps");
  uint4 kb[NS][TPS * NV], vb[NS][TPS * NV];
  int sl_t0[NS * TPS], sl_row[NS * TPS], sl_p[NS * TPS], sl_np[NS * TPS], sl_te[NS * TPS], sl_par[NS * TPS];
  bool sl_ok[NS * TPS], sl_first[NS * TPS], sl_last[NS * TPS], sl_valid[NS * TPS];

  bool more = enter();
  // issue the next tile of the stream as tile e of the ring (a dead, masked tile when
  // !take); false when the stream is exhausted
  auto issue_tile = [&](int e, uint4* kr, uint4* vr, bool take) -> bool {
    if (q_pending && take) {
      q_pending = false;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8_t v = __builtin_bit_cast(bf16x8_t, qtmp[kk]);
        if (q_stage & 1) qs1[kk] = v;
        else qs0[kk] = v;
      }
    }
    // Every call issues the same loads (row 0 of block 0 once the stream is exhausted),
    // so each consume waits on a fixed count and never drains the tile behind it.
    const bool live = more && take;
    const int ti = i_t0 + i_n;               // tile within the sequence
    const int tok_lo = 16 * ti;
    const bool any = live && tok_lo < i_te;
    const int blk = any ? i_bt[ti / SUB] : -1;
    const bool ok = any && blk >= 0 && blk < a.num_blocks;
    const int64_t off = (int64_t(ok ? blk : 0) * BS + (ti % SUB) * 16) * row_bytes + lane_off;
    sl_t0[e] = tok_lo;
    sl_ok[e] = ok;
    sl_row[e] = i_row;
    sl_p[e] = i_p;
    sl_np[e] = i_np;
    sl_te[e] = i_te;
    sl_valid[e] = live && i_valid;
    sl_first[e] = live && i_n == 0;
    sl_last[e] = live && i_n == i_nt - 1;
    sl_par[e] = q_stage;
    // the next piece's queries go out before this tile's rows
    if (live && ++i_n == i_nt) {
      q_stage ^= 1;
      more = enter();
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t o = off + (i / HPR) * group_step + (i % HPR) * (16 * LPR);
      if constexpr (kStream) {
        kr[i] = pkv::load_b128_stream(kc + o);
        vr[i] = pkv::load_b128_stream(vc + o);
      } else {
        kr[i] = *reinterpret_cast<const uint4*>(kc + o);
        vr[i] = *reinterpret_cast<const uint4*>(vc + o);
      }
    }
    return live;
  };
  // issue the next step (TPS tiles) into ring slot k; false when its first tile is past the stream
  auto issue = [&](int k) -> bool {
    const bool l0 = issue_tile(k * TPS, kb[k], vb[k], true);
    if constexpr (TPS == 2) issue_tile(k * TPS + 1, kb[k] + NV, vb[k] + NV, !sl_last[k * TPS]);
    return l0;
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4_t o[MT];

  auto qsel = [&](int e, bf16x8_t (&qf)[KS]) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = (sl_par[e] & 1) ? qs1[kk] : qs0[kk];
  };
  // K and V rows of tile e -> LDS tile u as bf16 [token][head_dim] (E4M3 widened on the
  // way). V rows past the end are zeroed by masking, not by a branch: every lane waits for
  // its rows on the main path, so no later wait is made conservative by a skipped one (a
  // stale slot may hold NaN, and 0 x NaN would reach the output). K rows past the end only
  // give scores that are masked.
  auto stage_tile = [&](int e, int u, const uint4* kr, const uint4* vr) {
    uint8_t* kt = my_kt + u * (16 * RSK);
    uint8_t* vt = my_vt + u * (16 * RS);
    const int t0 = sl_t0[e];
    const int tok_end = sl_te[e];
    const bool ok = sl_ok[e];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = (i / HPR) * RPI + lrow;
      const int c = (i % HPR) * LPR + lchunk;
      const uint32_t keep = (ok && (t0 + r < tok_end)) ? 0xffffffffu : 0u;
      const uint4 kv = kr[i];
      uint4 v = vr[i];
      asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
      v.x &= keep;
      v.y &= keep;
      v.z &= keep;
      v.w &= keep;
      if constexpr (CDT == PKV_BF16) {
        *reinterpret_cast<uint4*>(kt + r * RSK + 16 * c) = kv;
        *reinterpret_cast<uint4*>(vt + r * RS + 16 * c) = v;
      } else {
        // A lane's 16 codes widen to 32 bytes, two 16-byte stores. An LDS store serves 8
        // lanes at a time over 8 bank groups of 16 bytes (16-byte position mod 8). With
        // 8 lanes per row (head_dim 128) they hold one row's chunks, 32 bytes apart, so the
        // lanes of the upper four chunks store their halves in the opposite order; with 4
        // (head_dim 64) they hold two rows, which the K stride already puts on opposite
        // parities and the V stride does not, so odd V rows swap. Each store then meets 8
        // distinct groups instead of 4 twice.
        const bool swap_k = LPR == 8 && (lchunk & 4) != 0;
        const bool swap_v = LPR == 8 ? (lchunk & 4) != 0 : (lrow & 1) != 0;
        const uint32_t k0 = swap_k ? 16u : 0u, v0 = swap_v ? 16u : 0u;
        *reinterpret_cast<uint4*>(kt + r * RSK + 32 * c + k0) =
            pkv::fp8x8_to_bf16x8(swap_k ? kv.z : kv.x, swap_k ? kv.w : kv.y);
        *reinterpret_cast<uint4*>(kt + r * RSK + 32 * c + (16u - k0)) =
            pkv::fp8x8_to_bf16x8(swap_k ? kv.x : kv.z, swap_k ? kv.y : kv.w);
        *reinterpret_cast<uint4*>(vt + r * RS + 32 * c + v0) =
            pkv::fp8x8_to_bf16x8(swap_v ? v.z : v.x, swap_v ? v.w : v.y);
        *reinterpret_cast<uint4*>(vt + r * RS + 32 * c + (16u - v0)) =
            pkv::fp8x8_to_bf16x8(swap_v ? v.x : v.z, swap_v ? v.y : v.w);
      }
    }
  };
  auto reset_if_first = [&](int e) {
    if (sl_first[e]) {
      m = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  // S = K.Q^T of LDS tile u: the A operand is K in its MFMA layout (token hl, head_dim
  // 32kk + 8grp ..), read back from the K tile; the B operand is the packed queries in the
  // same order. Scores of tile e come out as lane l: head hl, tokens 4grp + r, masked.
  auto scores = [&](int e, int u, const bf16x8_t (&qf)[KS], float (&z)[4]) {
    const uint8_t* kt = my_kt + u * (16 * RSK);
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 kf = *reinterpret_cast<const uint4*>(kt + hl * RSK + 64 * kk + 16 * grp);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[kk], sc, 0, 0, 0);
    }
    const int t0 = sl_t0[e];
    const int tok_end = sl_te[e];
    const bool ok = sl_ok[e];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * grp + r;
      z[r] = (ok && t < tok_end) ? sc[r] * zscale_g : -INFINITY;
    }
  };
  // the piece's last tile was folded in: write its output (or partial)
  auto finish = [&](int e) {
    if (!sl_last[e]) return;
    float l = lsum;
    l = pkv::lane_groups_sum(l);
    if (!sl_valid[e] || hl >= G) return;
    const int hq = g * G + hl;
    const float inv = l > 0.f ? a.vscale_h[__builtin_amdgcn_readfirstlane(g) & (pkv::kHeadScales - 1)] / l : 0.f;
    const float lse2 = l > 0.f ? m + log2f(l) : -INFINITY;
    if (sl_np[e] == 1) {
      const int row = sl_row[e];
      uint16_t* orow = lp.out + (int64_t(row) * Hq + hq) * D + 4 * grp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t lo = pack_bf16x2_rne(o[mt][0] * inv, o[mt][1] * inv);
        const uint32_t hi = pack_bf16x2_rne(o[mt][2] * inv, o[mt][3] * inv);
        pkv::store_b64_untracked(orow + 16 * mt, lo, hi);
      }
      if (lp.lse && grp == 0)
        pkv::store_b32_untracked(lp.lse + int64_t(row) * Hq + hq, __float_as_uint(lse2 * kLn2));
    } else {
      const int64_t pi = split_partial(slot, sl_p[e], Hq, hq);
      float* orow = lp.ws_o + pi * D + 4 * grp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        pkv::store_b128_untracked(orow + 16 * mt, o[mt][0] * inv, o[mt][1] * inv, o[mt][2] * inv, o[mt][3] * inv);
      if (grp == 0) pkv::store_b32_untracked(lp.ws_lse + pi, __float_as_uint(lse2));
    }
  };
  // one 16-token tile (ring tile e, LDS tile u) folded into the running state
  auto step1 = [&](int e, int u) {
    bf16x8_t qf[KS];
    qsel(e, qf);
    reset_if_first(e);
    float z[4];
    scores(e, u, qf, z);
    float mt_ = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt_ = pkv::lane_groups_max(mt_);
    const float mn = fmaxf(m, mt_);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = pkv::fast_exp2(m - mref);
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = pkv::fast_exp2(z[r] - mref);
    const uint32_t p01 = pack_bf16x2_rne(pr[0], pr[1]);
    const uint32_t p23 = pack_bf16x2_rne(pr[2], pr[3]);
    lsum = lsum * alpha + (pkv::bf16_lo(p01) + pkv::bf16_hi(p01)) + (pkv::bf16_lo(p23) + pkv::bf16_hi(p23));
    m = mn;
    const pkv::s16x4_t pf = __builtin_bit_cast(pkv::s16x4_t, make_uint2(p01, p23));
    __builtin_amdgcn_wave_barrier();
    const uint8_t* src = my_vt + u * (16 * RS) + (4 * grp + (hl >> 2)) * RS + (4 * (hl & 3)) * 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const pkv::s16x4_t vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pkv::lds_s16x4_t*)(src + 32 * mt));
      f32x4_t acc = o[mt];
      acc[0] *= alpha;
      acc[1] *= alpha;
      acc[2] *= alpha;
      acc[3] *= alpha;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, acc, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
    finish(e);
  };
  // two consecutive tiles of one piece (ring tiles e, e + 1 in LDS tiles 0, 1; the second
  // may be dead) in one softmax step: one maximum and one rescale for 32 keys, and P.V on
  // 16x16x32 MFMAs whose 32 contraction slots of a lane are its own 4 + 4 rounded weights
  // (tokens 4grp + r of each tile) against the two tiles' transposed V reads at the same keys
  auto step2 = [&](int e) {
    bf16x8_t qf[KS];
    qsel(e, qf);
    reset_if_first(e);
    float z0[4], z1[4];
    scores(e, 0, qf, z0);
    scores(e + 1, 1, qf, z1);
    const float z[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
    float mt_ = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
    mt_ = pkv::lane_groups_max(mt_);
    const float mn = fmaxf(m, mt_);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = pkv::fast_exp2(m - mref);
    float pr[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pr[r] = pkv::fast_exp2(z[r] - mref);
    uint32_t pw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pw[j] = pack_bf16x2_rne(pr[2 * j], pr[2 * j + 1]);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) ps += pkv::bf16_lo(pw[j]) + pkv::bf16_hi(pw[j]);
    lsum = lsum * alpha + ps;
    m = mn;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    __builtin_amdgcn_wave_barrier();
    const uint8_t* src = my_vt + (4 * grp + (hl >> 2)) * RS + (4 * (hl & 3)) * 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const pkv::s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pkv::lds_s16x4_t*)(src + 32 * mt));
      const pkv::s16x4_t v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((pkv::lds_s16x4_t*)(src + 16 * RS + 32 * mt));
      const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      f32x4_t acc = o[mt];
      acc[0] *= alpha;
      acc[1] *= alpha;
      acc[2] *= alpha;
      acc[3] *= alpha;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
    finish(e);
    finish(e + 1);
  };
  // consume ring slot k: stage its tiles in LDS, then fold them in (a dead tile changes
  // nothing: its scores are masked and its V rows zeroed)
  auto consume = [&](int k) {
#pragma unroll
    for (int u = 0; u < TPS; ++u) stage_tile(k * TPS + u, u, kb[k] + u * NV, vb[k] + u * NV);
    __builtin_amdgcn_wave_barrier();
    if constexpr (TPS == 1) step1(k, 0);
    else step2(2 * k);
  };

  // rows without context (no piece anywhere): zero output, log-sum-exp -inf; plan row s
  // belongs to slot s mod num_slots
  for (int s0 = slot; s0 < B; s0 += a.num_slots) {
    if (seq_slots[2 * s0 + 1] != 0) continue;
    int b, row;
    split_row(a, s0, b, row);
    if (row < 0 || hl >= G) continue;
    uint16_t* orow = lp.out + (int64_t(row) * Hq + g * G + hl) * D + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) pkv::store_b64_untracked(orow + 16 * mt, 0u, 0u);
    if (lp.lse && grp == 0)
      pkv::store_b32_untracked(lp.lse + int64_t(row) * Hq + g * G + hl, __float_as_uint(-INFINITY));
  }
  if (!more) return;
  // One exit, at the bottom: a tile issued after the stream ran out is masked to nothing
  // (no row is valid, so it changes neither the running sums nor the outputs). An exit
  // between the two halves would join the loop's back edge in the control-flow graph
  // with a slot still in flight, and every wait at the top would become a full drain.
#pragma unroll
  for (int k = 0; k + 1 < NS; ++k) issue(k);
  bool live = true;
  do {
    // issue into the slot consumed last, then consume the oldest; after the sweep the
    // slots issued at k >= 1 are outstanding, and the first of them decides whether any is live
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int ik = (k + NS - 1) % NS;
      const bool l = issue(ik);
      if (k == 1) live = l;
      consume(k);
    }
    // The waves of the workgroup stream the same tiles (one KV head each) and stay in
    // step here. Left alone, the older wave on each SIMD wins issue and runs ahead: the
    // waves of one slot ended up to a quarter of the pass apart, and the last stretch ran
    // with half of the loads in flight. No memory wait is attached to the barrier.
    __builtin_amdgcn_s_barrier();
  } while (live);
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
    case 16: return decode_split_kernel<CDT, D, 16, HPW, kSplitRing, split_tps(CDT)>;
    case 32: return decode_split_kernel<CDT, D, 32, HPW, kSplitRing, split_tps(CDT)>;
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

int pkv::decode_split(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                      int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale,
                      float v_scale, const float* k_head_scales, const float* v_head_scales, const int32_t* rows,
                      int32_t num_rows, const int32_t* cu_seqlens_q, int32_t total_q, const int32_t* plan,
                      int32_t num_slots, int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
                      size_t workspace_bytes, float* lse_out, const Layers& layers, void* stream) {
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
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the pass (which also writes zeros for rows without context), then the merge of the
  // sequences it cut across slots (none when no sequence spans two slots); the layers of
  // a layer-batched call are the grid's third dimension
  hipLaunchKernelGGL(fn, dim3(num_kv_heads / hpw, num_slots, layers.n), dim3(hpw * 64), 0, st, a);
  if (g_profile_event) (void)hipEventRecord(g_profile_event, st);
  if (need > 0) {
    const int chunks = num_q_heads * (head_dim / 4);
    auto mk = max_pieces <= 8 ? (head_dim == 64 ? split_merge_kernel<64, 8> : split_merge_kernel<128, 8>)
                              : (head_dim == 64 ? split_merge_kernel<64, 32> : split_merge_kernel<128, 32>);
    hipLaunchKernelGGL(mk, dim3(num_rows, (chunks + 255) / 256, layers.n), dim3(256), 0, st, a, num_q_heads);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "decode_split: launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}
