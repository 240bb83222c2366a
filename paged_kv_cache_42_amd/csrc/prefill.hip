// paged_attention_prefill_chunks: the prefill chunks of a continuous-batching step (a
// sequence's new tokens, with or without a cached prefix) over the paged KV cache.
//
// What a query row computes is the page-walk attention of "Project 17: Production
// Serving: Continuous Batching and PagedAttention", "Step 6": new row i of a sequence
// with q new tokens and seq_len L sits at position L - q + i and attends keys
// 0 .. L - q + i (bottom-right causal alignment; the step's K/V already written). The
// rows are those of the mixed batch of "Continuous Batching", "5. Technical
// explanation", delimited by cu_seqlens ("6. Under the hood").
//
// gfx950 design (the MFMA-bound part of a mixed step; decode rows go to the split decode):
//  * item = (sequence, KV head g, block of 128/G new tokens): 128 GQA-packed query rows
//    (token, head), all G heads of g sharing each K/V tile. A workgroup of 8 waves takes
//    an item (one workgroup per compute unit): its two groups of 4 waves take the first
//    and the second half of the item's key tiles, 32 rows per wave as two 16-row MFMA
//    blocks, so every K and V fragment read from LDS feeds two MFMAs; at the end group 1
//    hands its softmax states to group 0 through LDS, which merges them.
//  * S^T = K.Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS as the A operand, the packed
//    queries as B): lane l holds row l%16 of its block for keys 4(l/16)+r of each
//    16-key group. Online softmax per row (two shuffles for the tile maximum); masks only
//    on tiles that reach a row's diagonal or the end of the keys.
//  * O^T += V^T.P^T on v_mfma_f32_16x16x32_bf16 per 32 keys: the lane's own 8 rounded
//    weights (two 16-key groups) are its B fragment, V^T comes straight from two
//    ds_read_b64_tr_b16 at the same keys. The softmax reference maximum is lazy: it moves
//    (and the accumulators are rescaled) only when a row's maximum grows by more than 2^8.
//  * Two kernels share that arithmetic. chunk_pp_kernel (bf16 cache, head_dim 128):
//    the groups run in opposite phases (matrix / softmax), tiles reach LDS by direct
//    global-to-LDS loads into swizzled, unpadded rows. chunk_kernel (E4M3 caches, head_dim
//    64): both groups compute each tile in step, tiles of 64 keys staged per group in two
//    LDS buffers (rows padded by 32 bytes) with coalesced 16-byte loads, the next tile held
//    in registers while the current one is computed; E4M3 rows are widened to bf16 on the
//    way in. Block ids are scalar loads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "decode_split.h"
#include "mfma_common.h"
#include "pkv.h"
#include "pkv_internal.h"

namespace {

using pkv::bf16x8_t;
using pkv::f32x4_t;
using pkv::lds_s16x4_t;
using pkv::pack_bf16x2_rne;
using pkv::s16x4_t;

using pkv::bf16x2_t;
constexpr float kLn2 = 0.6931471805599453f;
constexpr bf16x2_t kOnes = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
constexpr float kLazy = 8.f;       // log2 headroom of the lazy softmax maximum
constexpr int kRows = 128;         // query rows (token, head) of an item
constexpr int kKeys = 64;          // keys per LDS tile
constexpr int kWaves = 4;          // waves of a group, 32 rows each
constexpr int kGroups = 2;         // groups of a workgroup, each over half of the item's key tiles
constexpr int kGroupThreads = 64 * kWaves;
constexpr int kThreads = kGroupThreads * kGroups;

struct ChunkArgs {
  const uint16_t* q;      // [total_q][Hq][D] bf16
  uint16_t* out;          // [total_q][Hq][D] bf16
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  float* lse_out;         // [total_q][Hq], nullable
  const int4* work;       // [n][2] int4: (seq, KV head, first new token, first key) (key end, slot, 0, 0)
  float* ws_o;            // partials [slot][kRows][D] (normalised), then
  float* ws_lse;          //   their log2-sum-exps [slot][kRows]
  int num_slots;          // partials the workspace holds
  int table_width;
  int num_seqs;
  int total_q;
  int num_kv_heads;
  int group;
  int num_blocks;
  int len_clamp;
  float zscale_h[pkv::kHeadScales];   // per KV head: softmax scale * k_scale * log2(e)
  float vscale_h[pkv::kHeadScales];   // per KV head: v_scale
  // several layers (blockIdx.z): bytes between layers of q, out and the cache planes,
  // floats between layers of lse_out and of the partials
  int64_t ls_in, ls_out, ls_cache, ls_lse, ls_ws;
};

// The tensors of layer blockIdx.z of a layer-batched launch.
struct ChunkLayer {
  const uint16_t* q;
  uint16_t* out;
  const uint8_t* kc;
  const uint8_t* vc;
  float* lse;
  float* ws_o;
  float* ws_lse;
};
__device__ __forceinline__ ChunkLayer chunk_layer(const ChunkArgs& a, int64_t l) {
  ChunkLayer p;
  p.q = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.q) + l * a.ls_in);
  p.out = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(a.out) + l * a.ls_out);
  p.kc = a.kc + l * a.ls_cache;
  p.vc = a.vc + l * a.ls_cache;
  p.lse = a.lse_out ? a.lse_out + l * a.ls_lse : nullptr;
  p.ws_o = a.ws_o ? a.ws_o + l * a.ls_ws : nullptr;
  p.ws_lse = a.ws_lse ? a.ws_lse + l * a.ls_ws : nullptr;
  return p;
}
__device__ __forceinline__ ChunkLayer chunk_layer(const ChunkArgs& a) { return chunk_layer(a, blockIdx.z); }

template <int D>
struct Lds {
  static constexpr int RS = D * 2 + 32;          // bytes per bf16 key row (padded)
  static constexpr int kTile = kKeys * RS;       // one K or V tile
  static constexpr int kGroupBytes = 4 * kTile;  // K, V x double buffer, per group
  static constexpr int kBytes = kGroups * kGroupBytes;
  // the hand-over of a group's row states at the end: o [waves][2][D/16][64] float4, then
  // m and the lane sums [waves][2][64] float each
  static constexpr int kXchg = kWaves * 2 * (D / 16) * 64 * 16 + 2 * kWaves * 2 * 64 * 4;
  static_assert(kXchg <= kBytes, "exchange fits in the tile buffers");
};

// This wave's 32 query rows of an item (block rb holds rows 32w + 16rb + l % 16 -> token
// r / G, head r % G) as the B operands of S^T = K.Q^T, zero past the item's tokens, and
// their positions in the sequence.
template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* q, int row0, int q0, int ntok, int Hq, int g, int G,
                                          int pos0, int w, int hl, int grp, int (&pos)[2], bool (&row_ok)[2],
                                          bf16x8_t (&qf)[2][D / 32]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * w + 16 * rb + hl;
    const int tok = r / G;
    row_ok[rb] = tok < ntok;
    pos[rb] = pos0 + q0 + tok;
    const uint16_t* qrow = q + (int64_t(row0 + q0 + min(tok, ntok - 1)) * Hq + int64_t(g) * G + r % G) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      if (!row_ok[rb]) v = make_uint4(0, 0, 0, 0);
      qf[rb][kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
}

// The weights of one 64-key tile for a wave's 32 rows (two 16-row blocks; lane l holds
// row 16rb + l % 16 for keys key0 + 16kb + 4(l / 16) + r in sc[rb][kb][r]): masks where
// the tile reaches a row's diagonal or the end of the keys (`full` false; the mask is
// added to the raw score, 0 or -inf, since a select around the scaled score was compiled
// into per-lane branches), the lazy reference maximum, the exponentials rounded to bf16
// (two per word, the P^T fragments of P.V) and the row sums of those same rounded values.
// Lazy maximum: a row's reference moves only when the tile holds a score above it by
// more than kLazy (log2 units), so weights stay below 2^kLazy; the sum and the output
// share the reference, so the result is the same. Each lane first checks its own 16
// scores per row block; only when some lane of the wave sees such a score (the first
// tile, then rarely) is the row maximum reduced across lanes and the state rescaled.
template <int MT>
__device__ __forceinline__ void tile_weights(f32x4_t (&sc)[2][4], int key0, bool full, const int (&pos)[2],
                                             int key_end, int grp, float zscale, float (&m)[2], float (&lsum)[2],
                                             f32x4_t (&o)[2][MT], uint32_t (&pw)[2][4][2]) {
  if (!full) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 16 * kb + 4 * grp + r;
          sc[rb][kb][r] += ((key <= pos[rb]) & (key < key_end)) ? 0.f : -INFINITY;
        }
  }
  float lm[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    // the scale is positive: the maximum of the raw scores, scaled once; a linear chain,
    // so pairs fold into three-operand v_max3 (a tree did not)
    float mx = sc[rb][0][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[rb][e / 4][e % 4]);
    lm[rb] = mx * zscale;
  }
  if (__any((lm[0] > m[0] + kLazy) | (lm[1] > m[1] + kLazy))) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = lm[rb];
      mx = pkv::lane_groups_max(mx);
      const bool up = mx > m[rb] + kLazy;                  // false while the row has no key
      const float mn = up ? mx : m[rb];
      const float alpha = up ? pkv::fast_exp2(m[rb] - mn) : 1.f;
      m[rb] = mn;
      lsum[rb] *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        o[rb][mt][0] *= alpha;
        o[rb][mt][1] *= alpha;
        o[rb][mt][2] *= alpha;
        o[rb][mt][3] *= alpha;
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float mref = m[rb] == -INFINITY ? 0.f : m[rb];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t p01 = pack_bf16x2_rne(pkv::fast_exp2(fmaf(sc[rb][kb][0], zscale, -mref)),
                                           pkv::fast_exp2(fmaf(sc[rb][kb][1], zscale, -mref)));
      const uint32_t p23 = pack_bf16x2_rne(pkv::fast_exp2(fmaf(sc[rb][kb][2], zscale, -mref)),
                                           pkv::fast_exp2(fmaf(sc[rb][kb][3], zscale, -mref)));
      // the sum uses the same bf16-rounded weights that enter P.V (two per dot2)
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p01), kOnes, ps, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p23), kOnes, ps, false);
      pw[rb][kb][0] = p01;
      pw[rb][kb][1] = p23;
    }
    lsum[rb] += ps;
  }
}

// End of an item: group 1 hands its row states (reference maximum, lane sums,
// accumulators) to group 0 through LDS (`smem`, free of tiles by then), which merges them
// by log-sum-exp: with M = max(m0, m1), o = o0 2^(m0 - M) + o1 2^(m1 - M), l likewise
// (either group may have had no key). Group 0 then writes its rows: the bf16 output and
// natural-log LSE, or for a split item the normalised partial and its log2-sum-exp.
template <int D>
__device__ __forceinline__ void chunk_finish(const ChunkArgs& a, const ChunkLayer& lp, uint8_t* smem, int gi, int w,
                                             int lane, int g, int G, int Hq, int row0, int q0, int slot,
                                             const bool (&row_ok)[2], float (&m)[2], float (&lsum)[2],
                                             f32x4_t (&o)[2][D / 16]) {
  constexpr int MT = D / 16;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  {
    f32x4_t* xo = reinterpret_cast<f32x4_t*>(smem);
    float* xm = reinterpret_cast<float*>(smem + kWaves * 2 * MT * 64 * 16);
    float* xl = xm + kWaves * 2 * 64;
    if (gi == 1) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xo[((w * 2 + rb) * MT + mt) * 64 + lane] = o[rb][mt];
        xm[(w * 2 + rb) * 64 + lane] = m[rb];
        xl[(w * 2 + rb) * 64 + lane] = lsum[rb];
      }
    }
    __syncthreads();
    if (gi == 1) return;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float m1 = xm[(w * 2 + rb) * 64 + lane];
      const float l1 = xl[(w * 2 + rb) * 64 + lane];
      const float M = fmaxf(m[rb], m1);
      const float mref = M == -INFINITY ? 0.f : M;
      const float c0 = pkv::fast_exp2(m[rb] - mref), c1 = pkv::fast_exp2(m1 - mref);
      lsum[rb] = lsum[rb] * c0 + l1 * c1;
      m[rb] = M;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4_t o1 = xo[((w * 2 + rb) * MT + mt) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[rb][mt][e] = fmaf(o[rb][mt][e], c0, o1[e] * c1);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float l = lsum[rb];
    l = pkv::lane_groups_sum(l);
    if (!row_ok[rb]) continue;
    const int r = 32 * w + 16 * rb + hl;
    const float inv = l > 0.f ? a.vscale_h[g & (pkv::kHeadScales - 1)] / l : 0.f;
    if (slot >= 0) {                                       // partial of a split item
      float* prow = lp.ws_o + (int64_t(slot) * kRows + r) * D + 4 * grp;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        pkv::store_b128_untracked(prow + 16 * mt, o[rb][mt][0] * inv, o[rb][mt][1] * inv, o[rb][mt][2] * inv,
                                  o[rb][mt][3] * inv);
      if (grp == 0)
        pkv::store_b32_untracked(lp.ws_lse + int64_t(slot) * kRows + r,
                                 __float_as_uint(l > 0.f ? m[rb] + log2f(l) : -INFINITY));
      continue;
    }
    const int row = row0 + q0 + r / G;
    const int hq = g * G + r % G;
    uint16_t* orow = lp.out + (int64_t(row) * Hq + hq) * D + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t lo = pack_bf16x2_rne(o[rb][mt][0] * inv, o[rb][mt][1] * inv);
      const uint32_t hi = pack_bf16x2_rne(o[rb][mt][2] * inv, o[rb][mt][3] * inv);
      pkv::store_b64_untracked(orow + 16 * mt, lo, hi);
    }
    if (lp.lse && grp == 0)
      pkv::store_b32_untracked(lp.lse + int64_t(row) * Hq + hq,
                               __float_as_uint(l > 0.f ? (m[rb] + log2f(l)) * kLn2 : -INFINITY));
  }
}

// One item of the chunk kernel: work record `item`, on layer `layer`; smem:
// Lds<D>::kBytes bytes of LDS, 16-byte aligned. Called by the chunk kernel and by the
// mixed-step kernel.
template <int CDT, int D, int BS>
__device__ __forceinline__ void chunk_body(const ChunkArgs& a, uint8_t* smem, int item, int layer) {
  constexpr int KS = D / 32;
  constexpr int MT = D / 16;
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;
  constexpr int RS = Lds<D>::RS;
  constexpr int TILE = Lds<D>::kTile;
  constexpr int CPK = D * EB / 16;                       // 16-byte chunks per key head row
  constexpr int LPT = kKeys * CPK / kGroupThreads;       // chunk loads per thread per plane
  static_assert(kKeys * CPK % kGroupThreads == 0 && LPT >= 1, "tile / workgroup shape");
  static_assert(LPT <= 32, "mask word");
  typedef __attribute__((address_space(4))) const int32_t* cptr_i32;

  // ---- item (uniform): rows of (seq, KV head, block of new tokens) over keys
  // [key_lo, key_end); slot >= 0: write a partial for the merge. A malformed item exits
  // before any barrier.
  const int4 it = a.work[2 * item];
  const int4 it2 = a.work[2 * item + 1];
  const int s = it.x;
  const int g = it.y;
  const int q0 = it.z;
  const int slot = it2.y;
  if (s < 0 || s >= a.num_seqs || g < 0 || g >= a.num_kv_heads || slot >= a.num_slots) return;
  const float zscale_g = a.zscale_h[g & (pkv::kHeadScales - 1)];
  const int row0 = a.cu_q[s];
  const int qs = a.cu_q[s + 1] - row0;
  if (qs <= 0 || row0 < 0 || row0 + qs > a.total_q || q0 < 0 || q0 >= qs) return;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_clamp ? a.len_clamp : L);
  if (qs > L) return;
  const int key_end = max(0, min(it2.x, L));
  const int key_lo = it.w;
  if (key_lo < 0 || key_lo % kKeys != 0) return;
  const ChunkLayer lp = chunk_layer(a, layer);

  // the two groups take the first and the second half of the item's key tiles; each
  // has its own LDS buffers, and group 1 hands its row states to group 0 at the end
  // (group and wave indices go through readfirstlane so that the compiler sees them, and
  // everything derived from them, as wave-uniform: scalar loads and branches)
  const int gi = __builtin_amdgcn_readfirstlane(threadIdx.x / kGroupThreads);
  const int tid = threadIdx.x % kGroupThreads;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave within the group
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int pos0 = L - qs;                               // position of new token 0
  const int ntok = min(kRows / G, qs - q0);

  // ---- this wave's rows: block rb holds rows 32w + 16rb + hl -> token r / G, head r % G
  int pos[2];
  bool row_ok[2];
  bf16x8_t qf[2][KS];
  load_rows<D>(lp.q, row0, q0, ntok, Hq, g, G, pos0, w, hl, grp, pos, row_ok, qf);
  // positions of the wave's first and last valid rows (uniform); -1: no valid row
  const int tok_first = (32 * w) / G;
  const int tok_last = min(ntok - 1, (32 * w + 31) / G);
  const int wave_first = pos0 + q0 + tok_first;
  const int wave_last = tok_first < ntok ? pos0 + q0 + tok_last : -1;

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4_t o[2][MT];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[rb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const cptr_i32 btc = (cptr_i32)(uintptr_t)(a.block_tables + int64_t(s) * a.table_width);
  const int64_t row_bytes = int64_t(Hkv) * D * EB;
  const int64_t head_off = int64_t(g) * D * EB;
  const int t_lo = key_lo / kKeys;                      // the item's tiles [t_lo, t_hi)
  const int t_hi = (key_end + kKeys - 1) / kKeys;
  const int n_half = (max(t_hi - t_lo, 0) + 1) / 2;     // group 0: the first n_half tiles
  const int my_t0 = gi == 0 ? t_lo : t_lo + n_half;
  const int my_n = gi == 0 ? n_half : max(t_hi - t_lo - n_half, 0);
  const int my_key_end = gi == 0 ? min(key_end, (t_lo + n_half) * kKeys) : key_end;

  // Per-thread parts of the chunk addresses (the same in every tile): chunk i of this
  // thread is 16 bytes of key kti0 + KPL i of the tile. The 64 chunks of one wave's load
  // cover 64 / CPK consecutive keys, aligned, so they never straddle a block: the block is
  // wave-uniform, and the address is a scalar block base (plus the key's compile-time
  // offset in the block) and one 32-bit lane offset; the LDS offset of load i is loff0
  // plus a constant.
  constexpr int KPL = kGroupThreads / CPK;               // keys per load of the group
  static_assert(BS % (64 / CPK) == 0, "a wave's chunks of one load stay in one block");
  static_assert(KPL % BS == 0 || BS % KPL == 0, "loads and blocks nest");
  const int kti0 = tid / CPK;
  const int jw0 = KPL % BS == 0 ? __builtin_amdgcn_readfirstlane(kti0 / BS) : 0;
  const uint32_t voff0 = uint32_t((kti0 % BS) * row_bytes + head_off + 16 * (tid % CPK));
  const uint32_t loff0 = uint32_t(kti0 * RS + (CDT == PKV_BF16 ? 16 : 32) * (tid % CPK));
  const int64_t block_bytes = int64_t(BS) * row_bytes;

  // Stage tile t into registers: every load is issued (from block 0 when the block is
  // past the end or invalid), so the loads stay unconditional. The blocks are those that
  // hold this wave's chunks, one scalar load each. `keep` marks the real rows; all-ones
  // (uniform) when every row the wave loads is in the context and its blocks are valid.
  auto stage = [&](int t, uint4 (&ks)[LPT], uint4 (&vs)[LPT], uint32_t& keep) {
    const int key0 = t * kKeys;
    int blk[LPT];
    bool all_ok = key0 + kKeys <= my_key_end;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int bi = key0 / BS + jw0 + KPL * i / BS;
      blk[i] = bi * BS < my_key_end ? btc[bi] : -1;
      all_ok = all_ok && blk[i] >= 0 && blk[i] < a.num_blocks;
    }
    keep = all_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const bool bok = blk[i] >= 0 && blk[i] < a.num_blocks;
      if (!all_ok) {                                      // uniform: the tail tile, or a bad block id
        const bool ok = (key0 + kti0 + KPL * i < my_key_end) & bok;
        keep |= ok ? (1u << i) : 0u;
      }
      const int64_t base = int64_t(bok ? blk[i] : 0) * block_bytes + int64_t((KPL * i) % BS) * row_bytes;
      ks[i] = *reinterpret_cast<const uint4*>(lp.kc + base + voff0);
      vs[i] = *reinterpret_cast<const uint4*>(lp.vc + base + voff0);
    }
  };
  uint8_t* const gsmem = smem + gi * Lds<D>::kGroupBytes;
  auto commit = [&](int buf, const uint4 (&ks)[LPT], const uint4 (&vs)[LPT], uint32_t keep) {
    uint8_t* kt = gsmem + buf * 2 * TILE;
    uint8_t* vt = kt + TILE;
    const bool plain = keep == 0xffffffffu;                // uniform
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      uint4 k = ks[i], v = vs[i];
      if (!plain) {
        const uint32_t mk = (keep >> i) & 1u ? 0xffffffffu : 0u;
        k = make_uint4(k.x & mk, k.y & mk, k.z & mk, k.w & mk);
        v = make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk);
      }
      const uint32_t lo = loff0 + KPL * i * RS;
      if constexpr (CDT == PKV_BF16) {
        *reinterpret_cast<uint4*>(kt + lo) = k;
        *reinterpret_cast<uint4*>(vt + lo) = v;
      } else {
        *reinterpret_cast<uint4*>(kt + lo) = pkv::fp8x8_to_bf16x8(k.x, k.y);
        *reinterpret_cast<uint4*>(kt + lo + 16) = pkv::fp8x8_to_bf16x8(k.z, k.w);
        *reinterpret_cast<uint4*>(vt + lo) = pkv::fp8x8_to_bf16x8(v.x, v.y);
        *reinterpret_cast<uint4*>(vt + lo + 16) = pkv::fp8x8_to_bf16x8(v.z, v.w);
      }
    }
  };

  // One 64-key tile from LDS buffer `buf`.
  auto compute = [&](int t, int buf) {
    const int key0 = t * kKeys;
    if (key0 > wave_last) return;                          // uniform: every key is past every row
    const uint8_t* kt = gsmem + buf * 2 * TILE;
    const uint8_t* vt = kt + TILE;
    // S^T blocks: sc[rb][kb] -> keys key0 + 16kb + 4grp + r of row block rb
    // the K fragments of 16-key group kb + 1 are read while group kb is on the MFMAs
    f32x4_t sc[2][4];
    bf16x8_t kf[2][KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      kf[0][kk] = *reinterpret_cast<const bf16x8_t*>(kt + hl * RS + 2 * (32 * kk + 8 * grp));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb + 1 < 4) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          kf[(kb + 1) & 1][kk] =
              *reinterpret_cast<const bf16x8_t*>(kt + (16 * (kb + 1) + hl) * RS + 2 * (32 * kk + 8 * grp));
      }
      sc[0][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      sc[1][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        sc[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb & 1][kk], qf[0][kk], sc[0][kb], 0, 0, 0);
        sc[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb & 1][kk], qf[1][kk], sc[1][kb], 0, 0, 0);
      }
    }
    // keep that order through the scheduler (left alone, it pulls every read down to
    // just before its MFMA and the wave waits out the LDS latency each time)
    __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);          // LDS reads, group 0
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);   // reads of group kb + 1
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);   // MFMAs of group kb
    }
    // masks only where the tile reaches a row's diagonal or the end of the keys (uniform)
    const bool full = key0 + kKeys - 1 <= wave_first && key0 + kKeys <= key_end;
    uint32_t pw[2][4][2];                                  // [rb][kb]: rounded weights, 2 per word
    tile_weights<MT>(sc, key0, full, pos, key_end, grp, zscale_g, m, lsum, o, pw);
    // O^T[d][row] += V^T[d][key] . P^T[key][row] per 32 keys on the 16x16x32 MFMA. The
    // contraction slots of lane l are 8(l/16) .. +7; they take keys 32j + 4(l/16) + r and
    // 32j + 16 + 4(l/16) + r (r < 4) - the lane's own weights of 16-key groups 2j and 2j+1 -
    // and the A operand takes V^T at the same keys: two ds_read_b64_tr_b16 (rows
    // 16kb + 4(l/16) + (l%16)/4) per fragment, each fragment feeding both row blocks.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint8_t* vsrc = vt + (32 * j + 4 * grp + (hl >> 2)) * RS + (4 * (hl & 3)) * 2;
      const bf16x8_t pb0 = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0][2 * j][0], pw[0][2 * j][1],
                                                                     pw[0][2 * j + 1][0], pw[0][2 * j + 1][1]));
      const bf16x8_t pb1 = __builtin_bit_cast(bf16x8_t, make_uint4(pw[1][2 * j][0], pw[1][2 * j][1],
                                                                     pw[1][2 * j + 1][0], pw[1][2 * j + 1][1]));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vsrc + 32 * mt));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vsrc + 16 * RS + 32 * mt));
        const uint2 u0 = __builtin_bit_cast(uint2, v0), u1 = __builtin_bit_cast(uint2, v1);
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
        o[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb0, o[0][mt], 0, 0, 0);
        o[1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb1, o[1][mt], 0, 0, 0);
      }
    }
    // V reads run four fragments ahead of their MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
    for (int f = 0; f < 2 * MT; ++f) {
      if (f + 4 < 2 * MT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
    }
  };

  if (n_half > 0) {
    // Per group: two LDS buffers, one register stage: tile i + 1 is loaded into registers
    // while tile i is computed, then written to the buffer tile i - 1 used (free once every
    // wave has passed the barrier after i - 1). Tiles past the group's end are staged
    // clamped and masked. Both groups run n_half steps (group 1 may have one tile fewer),
    // so they meet at the same workgroup barriers.
    uint4 kr[LPT], vr[LPT];
    uint32_t keep;
    stage(my_t0, kr, vr, keep);
    commit(0, kr, vr, keep);
    stage(my_t0 + 1, kr, vr, keep);
    __syncthreads();
    for (int i = 0; i < n_half; i += 2) {
      if (i < my_n) compute(my_t0 + i, 0);
      commit(1, kr, vr, keep);
      stage(my_t0 + i + 2, kr, vr, keep);
      __syncthreads();
      if (i + 1 < my_n) compute(my_t0 + i + 1, 1);
      commit(0, kr, vr, keep);
      stage(my_t0 + i + 3, kr, vr, keep);
      __syncthreads();
    }
  }
  chunk_finish<D>(a, lp, smem, gi, w, lane, g, G, Hq, row0, q0, slot, row_ok, m, lsum, o);
}

// ---------------------------------------------------------------------------------
// bf16 cache, head_dim 128: the same items, rows and arithmetic as chunk_kernel, with
// the two groups run in opposite phases. A group's step alternates a matrix phase
// (P.V of tile t - 1 and S^T = K.Q^T of tile t on the MFMAs) and a softmax phase (the
// weights of tile t on the vector ALUs); group 1 runs one phase behind group 0, so on
// every SIMD one wave issues MFMAs while the other runs its softmax, and a workgroup
// barrier ends each phase. Tiles reach LDS by direct loads (global_load_lds_dwordx4: a
// wave's 64 lanes fill 1 KB of LDS, no registers in between), issued at the start of a
// softmax phase into buffers the group has finished with, three phases before their
// first use. LDS rows are 256 bytes, unpadded; 16-byte chunk c of key row r sits at
// chunk position c ^ swz_k(r) in K tiles and c ^ swz_v(r) in V tiles, so the K-fragment
// reads and the transposing V reads fall on distinct banks. Rows
// past the item's keys or in blocks outside the pool are zeroed after their load lands.
// ---------------------------------------------------------------------------------
// Chunk positions of the two planes: a K-fragment read takes one chunk of 16 rows, and
// ds_read_b128 serves 8 lanes at a time, so 8 consecutive rows must land on 8 distinct
// chunk positions of an aligned group of 8 (r mod 16 does; 2(r mod 8) + (r / 8) mod 2 cost
// ~590 bank-conflict cycles per wave). A transposing V read takes 32 bytes (a chunk pair)
// of 8 rows per half wave: 2(r mod 8) + (r / 8) mod 2 gives them distinct pairs.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// s_waitcnt vmcnt(N), no other counter
template <int CDT, int D, int BS>
__global__ void __launch_bounds__(kThreads, 1) chunk_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Lds<D>::kBytes];
  chunk_body<CDT, D, BS>(a, smem, blockIdx.x, blockIdx.z);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS of the opposite-phase chunk kernel: per group K0, K1, V0, V1 tiles of 64 keys x 256 B
constexpr int kPpLds = 2 * 4 * kKeys * 2 * 128;

// One item of the opposite-phase chunk kernel (bf16 cache, head_dim 128): work record
// `item`, on layer blockIdx.z; smem: kPpLds bytes of LDS, 16-byte aligned. Called by the
// chunk kernel and by the mixed-step kernel.
template <int BS>
__device__ __forceinline__ void chunk_pp_body(const ChunkArgs& a, uint8_t* smem, int item, int layer) {
  constexpr int D = 128;
  constexpr int KS = D / 32;
  constexpr int MT = D / 16;
  constexpr int RW = 2 * D;                              // LDS bytes per key row
  constexpr int TILE = kKeys * RW;
  constexpr int GB = 4 * TILE;                           // per group: K0, K1, V0, V1
  static_assert(Lds<D>::kXchg <= 2 * GB, "exchange fits in the tile buffers");
  static_assert(BS == 16 || BS == 32, "a wave's 4 rows of one load stay in one block");
  static_assert(2 * GB == kPpLds, "LDS layout");
  typedef __attribute__((address_space(4))) const int32_t* cptr_i32;
  typedef __attribute__((address_space(3))) uint8_t* lds_u8;

  const int4 it = a.work[2 * item];
  const int4 it2 = a.work[2 * item + 1];
  const int s = it.x;
  const int g = it.y;
  const int q0 = it.z;
  const int slot = it2.y;
  if (s < 0 || s >= a.num_seqs || g < 0 || g >= a.num_kv_heads || slot >= a.num_slots) return;
  const float zscale_g = a.zscale_h[g & (pkv::kHeadScales - 1)];
  const int row0 = a.cu_q[s];
  const int qs = a.cu_q[s + 1] - row0;
  if (qs <= 0 || row0 < 0 || row0 + qs > a.total_q || q0 < 0 || q0 >= qs) return;
  int L = a.seq_lens[s];
  L = L < 0 ? 0 : (L > a.len_clamp ? a.len_clamp : L);
  if (qs > L) return;
  const int key_end = max(0, min(it2.x, L));
  const int key_lo = it.w;
  if (key_lo < 0 || key_lo % kKeys != 0) return;
  const ChunkLayer lp = chunk_layer(a, layer);

  const int gi = __builtin_amdgcn_readfirstlane(threadIdx.x / kGroupThreads);
  const int tid = threadIdx.x % kGroupThreads;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int pos0 = L - qs;
  const int ntok = min(kRows / G, qs - q0);

  int pos[2];
  bool row_ok[2];
  bf16x8_t qf[2][KS];
  load_rows<D>(lp.q, row0, q0, ntok, Hq, g, G, pos0, w, hl, grp, pos, row_ok, qf);
  const int tok_first = (32 * w) / G;
  const int tok_last = min(ntok - 1, (32 * w + 31) / G);
  const int wave_first = pos0 + q0 + tok_first;
  const int wave_last = tok_first < ntok ? pos0 + q0 + tok_last : -1;

  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4_t o[2][MT];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[rb][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const cptr_i32 btc = (cptr_i32)(uintptr_t)(a.block_tables + int64_t(s) * a.table_width);
  const int64_t row_bytes = int64_t(Hkv) * D * 2;
  const int64_t head_off = int64_t(g) * D * 2;
  const int64_t block_bytes = int64_t(BS) * row_bytes;
  const int t_lo = key_lo / kKeys;
  const int t_hi = (key_end + kKeys - 1) / kKeys;
  const int n_half = (max(t_hi - t_lo, 0) + 1) / 2;
  const int my_t0 = gi == 0 ? t_lo : t_lo + n_half;
  const int my_n = gi == 0 ? n_half : max(t_hi - t_lo - n_half, 0);
  const int my_key_end = gi == 0 ? min(key_end, (t_lo + n_half) * kKeys) : key_end;

  // ---- direct loads: load i of wave w fills rows 16i + 4w .. +3 of a tile; lane l
  // writes row 16i + 4w + l/16, chunk position l % 16, so it loads data chunk
  // (l % 16) ^ swz(row) of that key's head row (swz_k or swz_v by plane)
  uint8_t* const gs = smem + gi * GB;
  const uint32_t gs_lds = uint32_t(uintptr_t((lds_u8)gs));
  const int drow = 4 * w + (lane >> 4);
  const uint32_t dvoff_k = uint32_t(drow * row_bytes + head_off + 16 * ((lane & 15) ^ swz_k(drow)));
  const uint32_t dvoff_v = uint32_t(drow * row_bytes + head_off + 16 * ((lane & 15) ^ swz_v(drow)));
  // The block ids of tile u's four loads (-1 past the keys; the table is read in bounds,
  // clamped to the last block that holds a key).
  const int last_bi = max(my_key_end - 1, 0) / BS;
  auto ids = [&](int u, int (&b)[4]) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = btc[min((u * kKeys + 16 * i) / BS, last_bi)];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (u * kKeys + 16 * i) / BS <= last_bi ? v[i] : -1;
  };
  // Issue one plane's four loads of a tile into LDS buffer `buf` (load i: the block of
  // id blk[i], rows 16i + 4w .. +3; block 0 where the id is past the keys or outside the
  // pool). M0 holds the LDS address; an SALU write of M0 needs one wait state before a
  // load reads it. Returns the mask of loads whose block is in the pool.
  auto dma = [&](const uint8_t* plane, const int (&blk)[4], uint32_t buf, uint32_t voff) -> int {
    int vm = 0;
    const uint8_t* base[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = uint32_t(blk[i]) < uint32_t(a.num_blocks);
      vm |= ok ? (1 << i) : 0;
      base[i] = plane + uint64_t(ok ? uint32_t(blk[i]) : 0u) * uint32_t(block_bytes) +
                (BS == 32 && (i & 1) ? 16 * row_bytes : 0);
    }
    const uint32_t m0 = gs_lds + buf + 4 * w * RW;
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %4\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %5\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(m0), "v"(voff), "s"(base[0]), "s"(base[1]), "s"(base[2]), "s"(base[3])
        : "memory");
    return vm;
  };
  auto bad = [&](int u, int vm) { return vm != 15 || u * kKeys + kKeys > my_key_end; };
  // zero this lane's rows of tile u that are past the keys or whose block was not loaded
  auto fix = [&](int u, uint32_t buf, int vm) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = ((vm >> i) & 1) && u * kKeys + 16 * i + drow < my_key_end;
      if (!ok) *reinterpret_cast<uint4*>(gs + buf + (16 * i + 4 * w) * RW + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
  };
  auto kbuf = [&](int t) -> uint32_t { return uint32_t((t & 1) * TILE); };
  auto vbuf = [&](int t) -> uint32_t { return uint32_t(2 * TILE + (t & 1) * TILE); };

  // per-lane LDS offsets: K fragment kk of row 16kb + hl sits at chunk (4kk + grp) ^ swz_k(hl);
  // V^T read of row 32j + 16h + 4grp + hl/4, data chunk 2mt + (hl/2)%2
  const int kswz = grp ^ swz_k(hl);
  const int vrow = 4 * grp + (hl >> 2);
  const int vswz = ((hl >> 1) & 1) ^ swz_v(vrow);

  f32x4_t sc[2][4];
  uint32_t pw[2][4][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pw[rb][kb][0] = 0u;
      pw[rb][kb][1] = 0u;
    }

  // matrix phase of step t: O^T += V^T(t - 1).P^T(t - 1) (weights of step t - 1, zero at
  // t = 0 over the loaded V(0)), and S^T(t) = K(t).Q^T (discarded past the last tile)
  auto gemm = [&](int t) {
    const uint8_t* kt = gs + kbuf(t);
    const uint8_t* vt = gs + vbuf(t > 0 ? t - 1 : 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8_t pb0 = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0][2 * j][0], pw[0][2 * j][1],
                                                                     pw[0][2 * j + 1][0], pw[0][2 * j + 1][1]));
      const bf16x8_t pb1 = __builtin_bit_cast(bf16x8_t, make_uint4(pw[1][2 * j][0], pw[1][2 * j][1],
                                                                     pw[1][2 * j + 1][0], pw[1][2 * j + 1][1]));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int coff = 16 * ((2 * mt) ^ vswz) + 8 * (hl & 1);
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vt + (32 * j + vrow) * RW + coff));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vt + (32 * j + 16 + vrow) * RW + coff));
        const uint2 u0 = __builtin_bit_cast(uint2, v0), u1 = __builtin_bit_cast(uint2, v1);
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
        o[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb0, o[0][mt], 0, 0, 0);
        o[1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb1, o[1][mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8_t kf[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8_t*>(kt + (16 * kb + hl) * RW + 16 * ((4 * kk) ^ kswz));
      sc[0][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      sc[1][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        sc[0][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[0][kk], sc[0][kb], 0, 0, 0);
        sc[1][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[1][kk], sc[1][kb], 0, 0, 0);
      }
    }
    // order for the scheduler: V reads four fragments ahead of their MFMAs, the K reads
    // of 16-key group 0 over the last P.V fragments, those of group kb + 1 before the
    // MFMAs of group kb (left alone, it hoists every read and runs out of registers)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int f = 0; f < 2 * MT; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (f + 4 < 2 * MT)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
    }
  };

  // softmax phase of step t: the rounded weights of tile t (zero when every key of the
  // tile is past every row of the wave); lazy reference maximum as in chunk_kernel
  auto softmax = [&](int t) {
    const int key0 = t * kKeys;
    if (key0 > wave_last) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          pw[rb][kb][0] = 0u;
          pw[rb][kb][1] = 0u;
        }
      return;
    }
    const bool full = key0 + kKeys - 1 <= wave_first && key0 + kKeys <= key_end;
    tile_weights<MT>(sc, key0, full, pos, key_end, grp, zscale_g, m, lsum, o, pw);
  };

  // ---- the loop: step t = matrix phase t, barrier, softmax phase t, barrier, the same
  // code in both groups; group 1 takes one extra barrier before it and group 0 one
  // after, so each phase of one group meets the opposite phase of the other. Loads: K(0),
  // V(0), K(1) before the loop; softmax phase t issues K(t + 2) and V(t + 1), then waits
  // for K(t + 1) and V(t) (the next matrix phase's) and zeroes their bad rows.
  const uint8_t* const kpl = lp.kc;
  const uint8_t* const vpl = lp.vc;
  int vmk1 = 15;                 // block mask of K tile t + 1 (issued, not yet checked)
  int vmv0 = 15;                 // of V tile t
  int bk[4], bv[4];              // block ids of the next K and V loads (tiles t + 2, t + 1)
  if (my_n > 0) {
    int b[4];
    ids(my_t0, b);
    const int k0 = dma(kpl, b, kbuf(0), dvoff_k);
    vmv0 = dma(vpl, b, vbuf(0), dvoff_v);
    if (my_n > 1) {
      ids(my_t0 + 1, b);
      vmk1 = dma(kpl, b, kbuf(1), dvoff_k);
      wait_vmcnt<4>();
    } else {
      wait_vmcnt<0>();
    }
    if (bad(my_t0, k0)) fix(my_t0, kbuf(0), k0);
    if (bad(my_t0, vmv0)) fix(my_t0, vbuf(0), vmv0);
  }
  __syncthreads();
  if (gi == 1) __syncthreads();
  for (int t = 0; t <= n_half; ++t) {
    if (my_n > 0 && t <= my_n) gemm(t);
    if (t + 2 < my_n) ids(my_t0 + t + 2, bk);
    if (t + 1 < my_n) ids(my_t0 + t + 1, bv);
    __syncthreads();
    if (t < my_n) {
      int vmk_new = 15, vmv_new = 15;
      if (t + 2 < my_n) vmk_new = dma(kpl, bk, kbuf(t + 2), dvoff_k);
      if (t + 1 < my_n) vmv_new = dma(vpl, bv, vbuf(t + 1), dvoff_v);
      __builtin_amdgcn_sched_barrier(0);                   // every load issued before the softmax
      softmax(my_t0 + t);
      if (t + 2 < my_n)
        wait_vmcnt<8>();
      else if (t + 1 < my_n)
        wait_vmcnt<4>();
      else
        wait_vmcnt<0>();
      // K(t + 1) and V(t) are in LDS now (both issued one softmax phase earlier)
      if (t + 1 < my_n && bad(my_t0 + t + 1, vmk1)) fix(my_t0 + t + 1, kbuf(t + 1), vmk1);
      if (bad(my_t0 + t, vmv0)) fix(my_t0 + t, vbuf(t), vmv0);
      vmk1 = vmk_new;
      vmv0 = vmv_new;
    }
    __syncthreads();
  }
  if (gi == 0) __syncthreads();
  chunk_finish<D>(a, lp, smem, gi, w, lane, g, G, Hq, row0, q0, slot, row_ok, m, lsum, o);
}

template <int BS>
__global__ void __launch_bounds__(kThreads, 1) chunk_pp_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPpLds];
  chunk_pp_body<BS>(a, smem, blockIdx.x, blockIdx.z);
}

// A mixed step in one launch: workgroups 0 .. layers x n_dec - 1 run the balanced-split
// decode pass over the step's decode rows (layer b / n_dec; slot r / hgroups and KV-head
// group r % hgroups of r = b mod n_dec, 8 KV heads per workgroup), the others chunk items
// of its prefill rows (item c / layers of layer c % layers, c counting from the first chunk
// workgroup: every layer's longest items first), one LDS array serving either. The decode
// workgroups come first, so they hold their units for the whole pass while chunk items
// flow through the rest: the memory-bound decode and the MFMA-bound chunks run side by
// side instead of one after the other.
template <int CDT, int D>
constexpr int mixed_lds_bytes() {
  constexpr int dec = pkv::split::split_lds_bytes<CDT, D, 8, pkv::split::split_tps(CDT, D)>();
  constexpr int chk = CDT == PKV_BF16 && D == 128 ? kPpLds : Lds<D>::kBytes;
  return dec > chk ? dec : chk;
}
template <int CDT, int D, int BS>
__global__ void __launch_bounds__(kThreads, 1) mixed_kernel(pkv::split::DecodeArgs da, ChunkArgs ca, int n_dec,
                                                             int hgroups, int layers) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[mixed_lds_bytes<CDT, D>()];
  const int b = blockIdx.x;
  if (b < n_dec * layers) {
    const int r = b % n_dec;
    pkv::split::decode_split_body<CDT, D, BS, 8, pkv::split::kSplitRing, pkv::split::split_tps(CDT, D)>(
        da, smem, r % hgroups, r / hgroups, b / n_dec);
  } else {
    const int c = b - n_dec * layers;
    if constexpr (CDT == PKV_BF16 && D == 128)
      chunk_pp_body<BS>(ca, smem, c / layers, c % layers);
    else
      chunk_body<CDT, D, BS>(ca, smem, c / layers, c % layers);
  }
}


// Log-sum-exp merge of the partials of split items. Merge record: (seq, KV head,
// first new token, first slot | pieces << 20). One thread per (row of the 128, four
// head_dim elements), blockIdx.y picking 256 of them, so every load of a thread is issued
// at once: M = max_k lse_k, out = sum_k 2^(lse_k - M) o_k / sum_k 2^(lse_k - M).
constexpr int kChunkMergeFast = 4;   // pieces merged with all loads in flight at once

template <int D>
__global__ void __launch_bounds__(256) chunk_merge_kernel(ChunkArgs a, const int4* merges) {
  const int4 mg = merges[blockIdx.x];
  const int s = mg.x, g = mg.y, q0 = mg.z;
  const int first = mg.w & 0xfffff, np = mg.w >> 20;
  if (s < 0 || s >= a.num_seqs || g < 0 || g >= a.num_kv_heads || np < 1 || first < 0 || first + np > a.num_slots)
    return;
  const ChunkLayer lp = chunk_layer(a);
  constexpr int LPR = D / 4;                               // threads per row
  const int task = blockIdx.y * 256 + threadIdx.x;
  const int r = task / LPR;
  const int e = 4 * (task % LPR);
  if (r >= kRows) return;
  float M = -INFINITY, S = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  if (np <= kChunkMergeFast) {
    float lse[kChunkMergeFast];
    float4 ov[kChunkMergeFast];
#pragma unroll
    for (int k = 0; k < kChunkMergeFast; ++k) {             // slots past np re-read piece 0
      const int64_t sl = first + (k < np ? k : 0);
      lse[k] = lp.ws_lse[sl * kRows + r];
      ov[k] = *reinterpret_cast<const float4*>(lp.ws_o + (sl * kRows + r) * D + e);
    }
    __builtin_amdgcn_sched_barrier(0);                    // all loads issued before any use
#pragma unroll
    for (int k = 0; k < kChunkMergeFast; ++k) M = k < np ? fmaxf(M, lse[k]) : M;
    const float mref = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int k = 0; k < kChunkMergeFast; ++k) {
      const float wk = k < np ? pkv::fast_exp2(lse[k] - mref) : 0.f;
      S += wk;
      A.x = fmaf(wk, ov[k].x, A.x);
      A.y = fmaf(wk, ov[k].y, A.y);
      A.z = fmaf(wk, ov[k].z, A.z);
      A.w = fmaf(wk, ov[k].w, A.w);
    }
  } else {
    for (int k = 0; k < np; ++k) M = fmaxf(M, lp.ws_lse[int64_t(first + k) * kRows + r]);
    const float mref = M == -INFINITY ? 0.f : M;
    for (int k = 0; k < np; ++k) {
      const float wk = pkv::fast_exp2(lp.ws_lse[int64_t(first + k) * kRows + r] - mref);
      const float4 ok = *reinterpret_cast<const float4*>(lp.ws_o + (int64_t(first + k) * kRows + r) * D + e);
      S += wk;
      A.x = fmaf(wk, ok.x, A.x);
      A.y = fmaf(wk, ok.y, A.y);
      A.z = fmaf(wk, ok.z, A.z);
      A.w = fmaf(wk, ok.w, A.w);
    }
  }
  // the row's place in the batch (rows of a block are in token order)
  const int row0 = a.cu_q[s];
  const int qs = a.cu_q[s + 1] - row0;
  if (qs <= 0 || row0 < 0 || row0 + qs > a.total_q || q0 < 0 || q0 >= qs) return;
  const int G = a.group;
  if (r / G >= min(kRows / G, qs - q0)) return;
  const int Hq = a.num_kv_heads * G;
  const float inv = S > 0.f ? 1.f / S : 0.f;
  const int row = row0 + q0 + r / G;
  const int hq = g * G + r % G;
  uint16_t* orow = lp.out + (int64_t(row) * Hq + hq) * D + e;
  *reinterpret_cast<uint2*>(orow) = make_uint2(pack_bf16x2_rne(A.x * inv, A.y * inv), pack_bf16x2_rne(A.z * inv, A.w * inv));
  if (lp.lse && e == 0) lp.lse[int64_t(row) * Hq + hq] = S > 0.f ? (M + log2f(S)) * kLn2 : -INFINITY;
}

using ChunkFn = void (*)(ChunkArgs);

template <int CDT, int D>
ChunkFn pick_bs(int BS) {
  switch (BS) {
    case 16: return chunk_kernel<CDT, D, 16>;
    case 32: return chunk_kernel<CDT, D, 32>;
    default: return nullptr;
  }
}

template <int CDT>
ChunkFn pick_d(int D, int BS) {
  switch (D) {
    case 64: return pick_bs<CDT, 64>(BS);
    case 128: return pick_bs<CDT, 128>(BS);
    default: return nullptr;
  }
}

using MergeFn = void (*)(ChunkArgs, const int4*);

MergeFn pick_merge(int D) {
  switch (D) {
    case 64: return chunk_merge_kernel<64>;
    case 128: return chunk_merge_kernel<128>;
    default: return nullptr;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

constexpr int kSlotBits = 20;                              // merge record: first slot | pieces << 20

}  // namespace

extern "C" int pkv_build_chunk_work(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                                    int32_t num_kv_heads, int32_t group, int32_t num_slots,
                                    int32_t min_piece_tiles, int32_t* items,
                                    int32_t capacity, int32_t* count, int32_t* merges, int32_t merge_capacity,
                                    int32_t* merge_count, int32_t* num_partials) {
  using pkv::fail;
  if (num_seqs < 0 || num_kv_heads <= 0 || group <= 0 || !count || !merge_count || !num_partials ||
      (num_seqs > 0 && (!q_lens || !seq_lens)))
    return fail(PKV_ERR_INVALID, "build_chunk_work: bad arguments");
  if (group > 16 || kRows % group != 0)
    return fail(PKV_ERR_UNSUPPORTED, "build_chunk_work: group %d not in {1,2,4,8,16}", group);
  struct Item {
    int32_t s, g, q0, key_lo, key_hi, slot, tiles;
  };
  std::vector<Item> v;
  std::vector<int32_t> m;
  const int32_t QB = kRows / group;
  // cap on a piece: the tiles of all blocks spread evenly over the slots, at least
  // min_piece_tiles (a smaller piece does not repay its partial and merge)
  int64_t total = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q = q_lens[s], L = seq_lens[s];
    if (q < 0 || L < 0 || q > L) return fail(PKV_ERR_INVALID, "build_chunk_work: sequence %d q_len %d seq_len %d", s, q, L);
    if (q < 2) continue;                                   // decode rows and idle sequences: not here
    for (int32_t q0 = 0; q0 < q; q0 += QB)
      total += (int64_t(std::min(L, L - q + std::min(q, q0 + QB))) + kKeys - 1) / kKeys * num_kv_heads;
  }
  const int64_t max_tiles = num_slots > 0 ? std::max<int64_t>({1, min_piece_tiles, (total + num_slots - 1) / num_slots})
                                          : int64_t(1) << 40;
  int64_t partials = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q = q_lens[s], L = seq_lens[s];
    if (q < 2) continue;
    for (int32_t q0 = 0; q0 < q; q0 += QB) {
      const int32_t keys = std::min(L, L - q + std::min(q, q0 + QB));   // through the block's last position
      const int32_t tiles = (keys + kKeys - 1) / kKeys;
      const int32_t np = tiles > max_tiles ? int32_t((tiles + max_tiles - 1) / max_tiles) : 1;
      for (int32_t g = 0; g < num_kv_heads; ++g) {
        if (np == 1) {
          v.push_back({s, g, q0, 0, keys, -1, tiles});
          continue;
        }
        if (partials + np >= (int64_t(1) << kSlotBits) || np >= (1 << (31 - kSlotBits)))
          return fail(PKV_ERR_INVALID, "build_chunk_work: too many partials (%lld)", (long long)(partials + np));
        m.insert(m.end(), {s, g, q0, int32_t(partials) | (np << kSlotBits)});
        for (int32_t k = 0; k < np; ++k) {                // balanced pieces of whole tiles
          const int32_t t0 = int32_t(int64_t(tiles) * k / np), t1 = int32_t(int64_t(tiles) * (k + 1) / np);
          v.push_back({s, g, q0, t0 * kKeys, std::min(keys, t1 * kKeys), int32_t(partials + k), t1 - t0});
        }
        partials += np;
      }
    }
  }
  // longest first: an item costs about its tiles x 128 rows of MFMA work
  std::stable_sort(v.begin(), v.end(), [](const Item& x, const Item& y) { return x.tiles > y.tiles; });
  *count = int32_t(v.size());
  *merge_count = int32_t(m.size() / 4);
  *num_partials = int32_t(partials);
  if (int64_t(v.size()) > capacity || (!v.empty() && !items))
    return fail(PKV_ERR_INVALID, "build_chunk_work: %zu items, capacity %d", v.size(), capacity);
  if (int64_t(m.size() / 4) > merge_capacity || (!m.empty() && !merges))
    return fail(PKV_ERR_INVALID, "build_chunk_work: %zu merges, capacity %d", m.size() / 4, merge_capacity);
  for (size_t i = 0; i < v.size(); ++i) {
    const int32_t rec[8] = {v[i].s, v[i].g, v[i].q0, v[i].key_lo, v[i].key_hi, v[i].slot, 0, 0};
    std::copy(rec, rec + 8, items + 8 * i);
  }
  std::copy(m.begin(), m.end(), merges);
  return PKV_OK;
}

extern "C" int pkv_chunk_slots(int32_t cache_dtype, int32_t head_dim, int32_t block_size, int32_t* slots) {
  using pkv::fail;
  if (!slots) return fail(PKV_ERR_INVALID, "chunk_slots: slots is NULL");
  ChunkFn fn = cache_dtype == PKV_BF16       ? pick_d<PKV_BF16>(head_dim, block_size)
               : cache_dtype == PKV_FP8_E4M3 ? pick_d<PKV_FP8_E4M3>(head_dim, block_size)
                                             : nullptr;
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "chunk_slots: unsupported (cache dtype %d, head_dim %d, block_size %d)",
                cache_dtype, head_dim, block_size);
  // One item per compute unit: a second workgroup on the unit shares its issue slots and
  // roughly halves the speed of both, so balancing over more slots than units only adds
  // pieces (measured on the 4 x 512-token chunk step: pieces of 17 tiles over 512 slots
  // ran slower than uncut items of up to 32 tiles).
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(PKV_ERR_HIP, "chunk_slots: device query failed");
  *slots = std::max(1, cus);
  return PKV_OK;
}

extern "C" int64_t pkv_chunk_workspace_bytes(int32_t num_partials, int32_t head_dim) {
  if (num_partials <= 0 || head_dim <= 0) return 0;
  return int64_t(num_partials) * kRows * (head_dim + 1) * 4;
}

namespace {
// A checked chunk launch (the chunk kernel and, for split blocks, the merge), built by
// chunk_prepare from the arguments of pkv_paged_attention_prefill_chunks; empty when there
// is nothing to launch.
struct ChunkLaunch {
  ChunkArgs a;
  ChunkFn fn;
  int num_work, num_merges, layers, head_dim;
  const int4* merges;
  bool empty;
};

int chunk_prepare(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                   int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens,
                   const int32_t* cu_seqlens_q, int32_t table_width, int32_t num_seqs, int32_t total_q,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t max_seq_len, float scale, float k_scale, float v_scale, const float* k_head_scales,
                   const float* v_head_scales, const int32_t* work_items, int32_t num_work, const int32_t* merges,
                   int32_t num_merges, int32_t num_partials, void* workspace, int64_t workspace_bytes,
                   float* lse_out, const pkv::Layers& layers, ChunkLaunch* L) {
  using pkv::fail;
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || table_width < 0 || num_blocks < 0 ||
      max_seq_len < 0 || num_work < 0 || num_merges < 0 || num_partials < 0 || num_partials >= (1 << kSlotBits))
    return fail(PKV_ERR_INVALID, "prefill_chunks: bad sizes");
  if (layers.n < 1 || layers.n > 65535) return fail(PKV_ERR_INVALID, "prefill_chunks: bad layer count %d", layers.n);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "prefill_chunks: num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const int G = num_q_heads / num_kv_heads;
  if (q_dtype != PKV_BF16 || (cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3) || G > 16 || kRows % G != 0)
    return fail(PKV_ERR_UNSUPPORTED, "prefill_chunks: unsupported (q dtype %d, cache dtype %d, group %d)", q_dtype,
                cache_dtype, G);
  ChunkFn fn = cache_dtype == PKV_BF16 ? pick_d<PKV_BF16>(head_dim, block_size)
                                       : pick_d<PKV_FP8_E4M3>(head_dim, block_size);
  if (!fn)
    return fail(PKV_ERR_UNSUPPORTED, "prefill_chunks: head_dim %d / block_size %d not supported", head_dim,
                block_size);
  if (cache_dtype == PKV_BF16 && head_dim == 128) fn = block_size == 16 ? chunk_pp_kernel<16> : chunk_pp_kernel<32>;
  if (!(scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PKV_ERR_INVALID, "prefill_chunks: scales must be > 0");
  L->empty = true;
  if (num_work == 0 || num_seqs == 0 || total_q == 0) return PKV_OK;
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "prefill_chunks: the cache has no blocks");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !cu_seqlens_q || !work_items)
    return fail(PKV_ERR_INVALID, "prefill_chunks: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(work_items))
    return fail(PKV_ERR_INVALID, "prefill_chunks: q, out, cache planes and work list must be 16-byte aligned");
  if (num_merges > 0 && num_partials == 0) return fail(PKV_ERR_INVALID, "prefill_chunks: merges without partials");
  if (num_partials > 0) {
    if (!merges || !workspace || !aligned16(merges) || !aligned16(workspace))
      return fail(PKV_ERR_INVALID, "prefill_chunks: split items need 16-byte aligned merges and workspace");
    const int64_t need = pkv_chunk_workspace_bytes(num_partials, head_dim);
    if (workspace_bytes / layers.n < need)
      return fail(PKV_ERR_INVALID, "prefill_chunks: workspace %lld bytes, %d x %lld needed",
                  (long long)workspace_bytes, layers.n, (long long)need);
  }
  ChunkArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.kc = static_cast<const uint8_t*>(k_cache);
  a.vc = static_cast<const uint8_t*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.cu_q = cu_seqlens_q;
  a.lse_out = lse_out;
  a.work = reinterpret_cast<const int4*>(work_items);
  a.num_slots = num_partials;
  if (num_partials > 0) {
    a.ws_o = static_cast<float*>(workspace);
    a.ws_lse = a.ws_o + int64_t(num_partials) * kRows * head_dim;
  }
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
  a.ls_in = layers.in;
  a.ls_out = layers.out;
  a.ls_cache = layers.cache;
  a.ls_lse = layers.lse;
  a.ls_ws = pkv_chunk_workspace_bytes(num_partials, head_dim) / 4;
  L->a = a;
  L->fn = fn;
  L->num_work = num_work;
  L->num_merges = num_merges;
  L->layers = layers.n;
  L->head_dim = head_dim;
  L->merges = reinterpret_cast<const int4*>(merges);
  L->empty = false;
  return PKV_OK;
}

int chunk_launch_merge(const ChunkLaunch& L, hipStream_t st) {
  if (L.empty || L.num_merges == 0) return PKV_OK;
  hipLaunchKernelGGL(pick_merge(L.head_dim), dim3(L.num_merges, kRows * (L.head_dim / 4) / 256, L.layers), dim3(256),
                     0, st, L.a, L.merges);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "prefill_chunks: merge launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

int prefill_chunks(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                   int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens,
                   const int32_t* cu_seqlens_q, int32_t table_width, int32_t num_seqs, int32_t total_q,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t max_seq_len, float scale, float k_scale, float v_scale, const float* k_head_scales,
                   const float* v_head_scales, const int32_t* work_items, int32_t num_work, const int32_t* merges,
                   int32_t num_merges, int32_t num_partials, void* workspace, int64_t workspace_bytes,
                   float* lse_out, const pkv::Layers& layers, void* stream) {
  ChunkLaunch L;
  const int rc = chunk_prepare(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, cu_seqlens_q,
                               table_width, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                               num_blocks, max_seq_len, scale, k_scale, v_scale, k_head_scales, v_head_scales,
                               work_items, num_work, merges, num_merges, num_partials, workspace, workspace_bytes,
                               lse_out, layers, &L);
  if (rc != PKV_OK || L.empty) return rc;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(L.fn, dim3(L.num_work, 1, L.layers), dim3(kThreads), 0, st, L.a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "prefill_chunks: launch failed: %s", hipGetErrorString(e));
  return chunk_launch_merge(L, st);
}
}  // namespace

extern "C" int pkv_paged_attention_prefill_chunks(void* out, const void* q, int32_t q_dtype, const void* k_cache,
                                                  const void* v_cache, int32_t cache_dtype,
                                                  const int32_t* block_tables, const int32_t* seq_lens,
                                                  const int32_t* cu_seqlens_q, int32_t table_width, int32_t num_seqs,
                                                  int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                                  int32_t max_seq_len, float scale, float k_scale, float v_scale,
                                                  const float* k_head_scales, const float* v_head_scales,
                                                  const int32_t* work_items, int32_t num_work,
                                                  const int32_t* merges, int32_t num_merges, int32_t num_partials,
                                                  void* workspace, int64_t workspace_bytes, float* lse_out,
                                                  void* stream) {
  return prefill_chunks(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, cu_seqlens_q,
                        table_width, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_seq_len, scale, k_scale, v_scale, k_head_scales, v_head_scales, work_items, num_work,
                        merges, num_merges, num_partials, workspace, workspace_bytes, lse_out, pkv::Layers{}, stream);
}

extern "C" int pkv_paged_attention_prefill_chunks_layers(
    void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache, int32_t cache_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t table_width,
    int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale, float v_scale,
    const float* k_head_scales, const float* v_head_scales, const int32_t* work_items, int32_t num_work,
    const int32_t* merges, int32_t num_merges, int32_t num_partials, void* workspace, int64_t workspace_bytes,
    float* lse_out, const pkv_layers* layers, void* stream) {
  pkv::Layers ls;
  const int rc = pkv::layers_from("prefill_chunks_layers", layers, true,
                                  pkv::kLayerIn | pkv::kLayerOut | pkv::kLayerCache | (lse_out ? pkv::kLayerLse : 0u),
                                  &ls);
  if (rc != PKV_OK) return rc;
  return prefill_chunks(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, cu_seqlens_q,
                        table_width, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        max_seq_len, scale, k_scale, v_scale, k_head_scales, v_head_scales, work_items, num_work,
                        merges, num_merges, num_partials, workspace, workspace_bytes, lse_out, ls, stream);
}

namespace {
// Per-unit costs that balance a one-launch mixed step, measured on MI355X with these
// kernels (a step of 64 decode rows with 256-3000 keys and 4 chunks of 512 new tokens, 8
// KV heads, the split decode over 64 slots and the chunk kernel alone, caches flushed):
// us per 16-token decode tile of one 8-KV-head workgroup, and us of a unit per 64-key tile
// of a 128-row chunk item. An E4M3 tile takes 0.83x a bf16 one for half the bytes, so a
// rate in bytes would misjudge it.
struct MixedRates {
  double tile_us, item_tile_us;
};
MixedRates mixed_rates(int cache_dtype, int head_dim) {
  if (head_dim == 128) return cache_dtype == PKV_BF16 ? MixedRates{1.55, 1.96} : MixedRates{1.29, 2.02};
  return cache_dtype == PKV_BF16 ? MixedRates{0.91, 1.31} : MixedRates{0.84, 1.35};
}
constexpr double kMixedReadBytesPerUs = 6.3e6;   // the decode's stream-read rate at full occupancy
// Beside chunk items the decode runs ~15% slower than alone (they share the memory
// system): on the config-2 step the rates alone pick 55 slots (98 us), while 60-128 slots
// take 86-89 us and fewer than 56 climb steeply, so the decode's work is scaled by this.
constexpr double kMixedDecodeContention = 1.15;

using MixedFn = void (*)(pkv::split::DecodeArgs, ChunkArgs, int, int, int);
template <int CDT, int D>
MixedFn pick_mixed_bs(int BS) {
  switch (BS) {
    case 16: return mixed_kernel<CDT, D, 16>;
    case 32: return mixed_kernel<CDT, D, 32>;
    default: return nullptr;
  }
}
template <int CDT>
MixedFn pick_mixed_d(int D, int BS) {
  switch (D) {
    case 64: return pick_mixed_bs<CDT, 64>(BS);
    case 128: return pick_mixed_bs<CDT, 128>(BS);
    default: return nullptr;
  }
}
// The mixed kernel of a shape (null where the step runs as two launches): decode
// workgroups of 8 KV heads, so num_kv_heads a multiple of 8.
MixedFn pick_mixed(int cache_dtype, int head_dim, int block_size, int num_kv_heads) {
  if (num_kv_heads % 8 != 0) return nullptr;
  if (cache_dtype == PKV_BF16) return pick_mixed_d<PKV_BF16>(head_dim, block_size);
  if (cache_dtype == PKV_FP8_E4M3) return pick_mixed_d<PKV_FP8_E4M3>(head_dim, block_size);
  return nullptr;
}
}  // namespace

extern "C" int pkv_mixed_decode_slots(int32_t num_seqs, const int32_t* q_lens, const int32_t* seq_lens,
                                      int32_t cache_dtype, int32_t num_kv_heads, int32_t group, int32_t head_dim,
                                      int32_t block_size, int32_t num_layers, int32_t* slots) {
  using pkv::fail;
  if (num_seqs < 0 || num_kv_heads <= 0 || group <= 0 || num_layers < 1 || !slots ||
      (num_seqs > 0 && (!q_lens || !seq_lens)))
    return fail(PKV_ERR_INVALID, "mixed_decode_slots: bad arguments");
  int full = 0;
  int rc = pkv_decode_split_slots(cache_dtype, num_kv_heads, head_dim, block_size, &full);
  if (rc != PKV_OK) return rc;
  const int per_layer = std::max(1, (full + num_layers - 1) / num_layers);   // the layers share the units
  *slots = per_layer;
  if (!pick_mixed(cache_dtype, head_dim, block_size, num_kv_heads) || group > 16 || kRows % group != 0)
    return PKV_OK;                                       // two launches: the decode takes the device
  int64_t dec_tiles = 0, chunk_tiles = 0;
  const int32_t QB = kRows / group;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q = q_lens[s], L = seq_lens[s];
    if (q < 0 || L < 0 || q > L) return fail(PKV_ERR_INVALID, "mixed_decode_slots: sequence %d q_len %d seq_len %d", s, q, L);
    if (q == 1) dec_tiles += (L + 15) / 16;
    if (q < 2) continue;
    for (int32_t q0 = 0; q0 < q; q0 += QB)
      chunk_tiles += (int64_t(std::min(L, L - q + std::min(q, q0 + QB))) + kKeys - 1) / kKeys * num_kv_heads;
  }
  if (dec_tiles == 0 || chunk_tiles == 0) return PKV_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(PKV_ERR_HIP, "mixed_decode_slots: device query failed");
  // Decode workgroups n (slots x KV-head groups x layers, so in steps of one slot per
  // layer) on n of the cus units: the decode ends after max(tiles x tile_us / n, bytes /
  // read rate), the chunk items on the other units after item_tiles x item_tile_us /
  // (cus - n). The best such n is kept only where it beats the decode at the layers' share
  // of the units followed by the chunk items on all of them by 5%: a step of a few long
  // prefills leaves the decode too little to hide, and slots come in whole steps per layer.
  const int hgroups = num_kv_heads / 8;
  const MixedRates r = mixed_rates(cache_dtype, head_dim);
  const double dec_work = double(dec_tiles) * hgroups * num_layers * r.tile_us * kMixedDecodeContention;
  const double dec_bytes = double(dec_tiles) * num_layers * 16.0 * num_kv_heads * head_dim *
                           (cache_dtype == PKV_BF16 ? 2 : 1) * 2;
  const double chk_work = double(chunk_tiles) * num_layers * r.item_tile_us;
  auto t_dec = [&](int n) { return std::max(dec_work / n, dec_bytes / kMixedReadBytesPerUs); };
  const int step = hgroups * num_layers;
  const int share = per_layer * step;
  const double t_seq = t_dec(share) + chk_work / cus;
  int best = share;
  double best_t = 1e300;
  for (int n = step; n < cus && n < share; n += step) {
    const double t = std::max(t_dec(n), chk_work / (cus - n));
    if (t < best_t) {
      best_t = t;
      best = n;
    }
  }
  if (best_t <= 0.95 * t_seq) *slots = best / step;
  return PKV_OK;
}

namespace {
int mixed_attention(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                    int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens,
                    const int32_t* cu_seqlens_q, int32_t table_width, int32_t num_seqs, int32_t total_q,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale, float v_scale,
                    const float* k_head_scales, const float* v_head_scales, const int32_t* decode_rows,
                    int32_t num_decode_rows, const int32_t* split_plan, int32_t split_slots, int32_t tiles_per_slot,
                    int32_t max_pieces, void* split_workspace, size_t split_workspace_bytes,
                    const int32_t* chunk_items, int32_t num_chunk_items, const int32_t* chunk_merges,
                    int32_t num_chunk_merges, int32_t num_chunk_partials, void* chunk_workspace,
                    int64_t chunk_workspace_bytes, float* lse_out, const pkv::Layers& layers, void* stream) {
  using pkv::fail;
  if (num_decode_rows < 0 || num_chunk_items < 0) return fail(PKV_ERR_INVALID, "mixed: bad sizes");
  pkv::split::SplitLaunch SL;
  SL.empty = true;
  if (num_decode_rows > 0) {
    const int rc = pkv::split::split_prepare(
        out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, table_width, num_seqs, num_q_heads,
        num_kv_heads, head_dim, block_size, num_blocks, max_seq_len, scale, k_scale, v_scale, k_head_scales,
        v_head_scales, decode_rows, num_decode_rows, cu_seqlens_q, total_q, split_plan, split_slots, tiles_per_slot,
        max_pieces, split_workspace, split_workspace_bytes, lse_out, layers, &SL);
    if (rc != PKV_OK) return rc;
  }
  ChunkLaunch CL;
  {
    const int rc = chunk_prepare(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens,
                                 cu_seqlens_q, table_width, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                 block_size, num_blocks, max_seq_len, scale, k_scale, v_scale, k_head_scales,
                                 v_head_scales, chunk_items, num_chunk_items, chunk_merges, num_chunk_merges,
                                 num_chunk_partials, chunk_workspace, chunk_workspace_bytes, lse_out, layers, &CL);
    if (rc != PKV_OK) return rc;
  }
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const MixedFn mfn = pick_mixed(cache_dtype, head_dim, block_size, num_kv_heads);
  if (mfn && !SL.empty && !CL.empty && SL.hpw == 8 && SL.hpw * 64 == kThreads) {
    const int n_dec = SL.hgroups * SL.num_slots;
    const int64_t grid = (int64_t(n_dec) + CL.num_work) * layers.n;
    if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "mixed: grid of %lld workgroups", (long long)grid);
    hipLaunchKernelGGL(mfn, dim3(uint32_t(grid), 1, 1), dim3(kThreads), 0, st, SL.args, CL.a, n_dec, SL.hgroups,
                       layers.n);
  } else {
    if (!SL.empty)
      hipLaunchKernelGGL(reinterpret_cast<void (*)(pkv::split::DecodeArgs)>(const_cast<void*>(SL.pass)),
                         dim3(SL.hgroups, SL.num_slots, SL.layers), dim3(SL.hpw * 64), 0, st, SL.args);
    if (!CL.empty) hipLaunchKernelGGL(CL.fn, dim3(CL.num_work, 1, CL.layers), dim3(kThreads), 0, st, CL.a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "mixed: launch failed: %s", hipGetErrorString(e));
  int rc = pkv::split::split_launch_merge(SL, st);
  if (rc != PKV_OK) return rc;
  return chunk_launch_merge(CL, st);
}
}  // namespace

extern "C" int pkv_paged_attention_mixed(
    void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache, int32_t cache_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t table_width,
    int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale, float v_scale,
    const float* k_head_scales, const float* v_head_scales, const int32_t* decode_rows, int32_t num_decode_rows,
    const int32_t* split_plan, int32_t split_slots, int32_t tiles_per_slot, int32_t max_pieces,
    void* split_workspace, size_t split_workspace_bytes, const int32_t* chunk_items, int32_t num_chunk_items,
    const int32_t* chunk_merges, int32_t num_chunk_merges, int32_t num_chunk_partials, void* chunk_workspace,
    int64_t chunk_workspace_bytes, float* lse_out, void* stream) {
  return mixed_attention(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, cu_seqlens_q,
                         table_width, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         max_seq_len, scale, k_scale, v_scale, k_head_scales, v_head_scales, decode_rows,
                         num_decode_rows, split_plan, split_slots, tiles_per_slot, max_pieces, split_workspace,
                         split_workspace_bytes, chunk_items, num_chunk_items, chunk_merges, num_chunk_merges,
                         num_chunk_partials, chunk_workspace, chunk_workspace_bytes, lse_out, pkv::Layers{}, stream);
}

extern "C" int pkv_paged_attention_mixed_layers(
    void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache, int32_t cache_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t table_width,
    int32_t num_seqs, int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale, float v_scale,
    const float* k_head_scales, const float* v_head_scales, const int32_t* decode_rows, int32_t num_decode_rows,
    const int32_t* split_plan, int32_t split_slots, int32_t tiles_per_slot, int32_t max_pieces,
    void* split_workspace, size_t split_workspace_bytes, const int32_t* chunk_items, int32_t num_chunk_items,
    const int32_t* chunk_merges, int32_t num_chunk_merges, int32_t num_chunk_partials, void* chunk_workspace,
    int64_t chunk_workspace_bytes, float* lse_out, const pkv_layers* layers, void* stream) {
  pkv::Layers ls;
  const int rc = pkv::layers_from("mixed_layers", layers, true,
                                  pkv::kLayerIn | pkv::kLayerOut | pkv::kLayerCache | (lse_out ? pkv::kLayerLse : 0u),
                                  &ls);
  if (rc != PKV_OK) return rc;
  return mixed_attention(out, q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, seq_lens, cu_seqlens_q,
                         table_width, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         max_seq_len, scale, k_scale, v_scale, k_head_scales, v_head_scales, decode_rows,
                         num_decode_rows, split_plan, split_slots, tiles_per_slot, max_pieces, split_workspace,
                         split_workspace_bytes, chunk_items, num_chunk_items, chunk_merges, num_chunk_merges,
                         num_chunk_partials, chunk_workspace, chunk_workspace_bytes, lse_out, ls, stream);
}
