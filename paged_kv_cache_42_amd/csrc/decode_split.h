// Internal: the balanced-split decode pass as a device function, its argument block and
// the helpers both need, shared by the decode kernels (decode.hip) and the mixed-step
// kernel that runs decode slots and prefill-chunk items in one launch (prefill.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "mfma_common.h"
#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace split {

constexpr float kLn2 = 0.6931471805599453f;

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
__device__ __forceinline__ LayerPtrs layer_ptrs(const DecodeArgs& a, int64_t l) {
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
__device__ __forceinline__ LayerPtrs layer_ptrs(const DecodeArgs& a) { return layer_ptrs(a, blockIdx.z); }

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


// ---------------------------------------------------------------------------------
// Tiles in each wave's load ring of the balanced-split kernel: while one is consumed,
// NS - 1 are in flight.
constexpr int kSplitRing = 2;
// Tiles folded per softmax step of the balanced-split kernel: two where a 16-token tile of
// a KV head carries 2 KB per plane or less (E4M3 caches, bf16 at head_dim 64), half the
// bytes of a bf16 tile at head_dim 128 through the same per-tile work.
constexpr int split_tps(int cdt, int d) { return cdt == PKV_FP8_E4M3 || d == 64 ? 2 : 1; }

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
template <int CDT, int D, int HPW, int TPS>
constexpr int split_lds_bytes() {
  return HPW * TPS * 16 * ((D * 2 + 16) + (D * 2 + 32));
}

// The pass of one workgroup: KV-head group `hgroup` (waves take KV heads hgroup * HPW + w)
// of slot `slot`, on layer `layer`; lds: split_lds_bytes<CDT, D, HPW, TPS>() bytes of LDS,
// 16-byte aligned. Called by the decode kernel and by the mixed-step kernel.
template <int CDT, int D, int BS, int HPW, int NS = kSplitRing, int TPS = 1>
__device__ __forceinline__ void decode_split_body(const DecodeArgs& a, uint8_t* lds, int hgroup, int slot,
                                                  int layer) {
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
  const int g = hgroup * HPW + w;
  const float zscale_g = a.zscale_h[__builtin_amdgcn_readfirstlane(g) & (pkv::kHeadScales - 1)];
  const int G = a.group;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int hl = lane & 15;
  const int grp = lane >> 4;
  const int hl_q = hl < G ? hl : hl % G;
  const LayerPtrs lp = layer_ptrs(a, layer);
  const uint8_t* kc = lp.kc;
  const uint8_t* vc = lp.vc;
  const int64_t row_bytes = int64_t(Hkv) * D * EB;
  const int lrow = lane / LPR;               // row of this lane in each load
  const int lchunk = lane % LPR;             // 16-byte chunk of the head slice
  const int64_t lane_off = int64_t(lrow) * row_bytes + int64_t(g) * HB + 16 * lchunk;
  const int64_t group_step = int64_t(RPI) * row_bytes;

  // per wave: TPS K tiles (16 rows, stride RSK), then TPS V tiles (16 rows, stride RS)
  static_assert(split_lds_bytes<CDT, D, HPW, TPS>() == HPW * TPS * 16 * (RSK + RS), "LDS layout");
  uint8_t* my_kt = lds + w * (TPS * 16 * (RSK + RS));
  uint8_t* my_vt = my_kt + TPS * 16 * RSK;

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

// Host side: a checked balanced-split launch, built by split_prepare from the arguments
// of pkv_paged_attention_decode_split (same checks and errors); empty when there is
// nothing to launch. The pass kernel is `pass` on grid (hgroups, num_slots, layers) of
// hpw * 64 threads; split_launch_merge launches the merge when the plan needs one.
struct SplitLaunch {
  DecodeArgs args;
  const void* pass;
  int hpw, hgroups, num_slots, layers, num_rows, num_q_heads, head_dim, max_pieces;
  size_t need;
  bool empty;
};
int split_prepare(void* out, const void* q, int32_t q_dtype, const void* k_cache, const void* v_cache,
                  int32_t cache_dtype, const int32_t* block_tables, const int32_t* seq_lens, int32_t table_width,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks, int32_t max_seq_len, float scale, float k_scale,
                  float v_scale, const float* k_head_scales, const float* v_head_scales, const int32_t* rows,
                  int32_t num_rows, const int32_t* cu_seqlens_q, int32_t total_q, const int32_t* plan,
                  int32_t num_slots, int32_t tiles_per_slot, int32_t max_pieces, void* workspace,
                  size_t workspace_bytes, float* lse_out, const Layers& layers, SplitLaunch* L);
int split_launch_merge(const SplitLaunch& L, hipStream_t stream);

}  // namespace split
}  // namespace pkv
