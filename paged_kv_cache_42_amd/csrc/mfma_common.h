// Internal: MFMA building blocks shared by the decode and varlen kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (two words) -> 8 bf16, code j of the 8 bytes -> element j. Exact: every
// E4M3 value is a bf16 value. v_cvt_scalef32_pk_bf16_fp8 with scale 1 widens the two
// codes of one 16-bit half per instruction (OCP E4M3 on this target; it agrees with the
// bit-level decode pkv::fp8_to_f32 on all 256 codes, NaN codes giving NaN).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool high_half) {
  const bf16x2_t v = high_half ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                               : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return make_uint4(fp8x2_to_bf16x2(lo, false), fp8x2_to_bf16x2(lo, true), fp8x2_to_bf16x2(hi, false),
                    fp8x2_to_bf16x2(hi, true));
}

// Two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float a, float b) {
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}


typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Global stores issued as inline assembly, which the compiler's wait-count pass does not
// see. In a loop that keeps loads in flight across iterations, a store the pass can see
// leaves loads and stores outstanding together; it then cannot order them and turns the
// next wait for a load into a full drain. Hidden stores only ever add to the hardware
// count, so every wait the pass computes for its loads stays sufficient. Store data
// registers may be reused right after issue on this target (the pass itself inserts no
// wait for that), and the end of the kernel makes the writes visible. One exception: a
// store of more than 8 bytes reads its data registers late, so a vector ALU write to them
// must wait two cycles; the hazard pass cannot see into inline assembly, so the 16-byte
// store carries its own s_nop (without it the next instruction overwrote the data).
__device__ __forceinline__ void store_b32_untracked(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_b64_untracked(void* p, uint32_t lo, uint32_t hi) {
  const u32x2_t v = {lo, hi};
  asm volatile("global_store_dwordx2 %0, %1, off" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_b128_untracked(void* p, float x, float y, float z, float w) {
  const u32x4_t v = {__float_as_uint(x), __float_as_uint(y), __float_as_uint(z), __float_as_uint(w)};
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// Maximum and sum over the four lane groups of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48)
// with gfx950's row swaps: v_permlane16_swap exchanges 16-lane rows 1 <-> 0 and 3 <-> 2
// between its two operands, v_permlane32_swap rows 2, 3 <-> 0, 1, so swapping a value
// with itself and combining the two results pairs lane l with l ^ 16, then with l ^ 32
// (the same pairs, in the same order, as two xor shuffles). They are ALU instructions,
// where a shuffle through ds_bpermute is an LDS round trip. Every lane must be active.
__device__ __forceinline__ float lane_groups_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_groups_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One 16-byte load with the non-temporal hint (global_load_dwordx4 ... nt), for data a
// launch reads exactly once: the K/V rows of the decode stream. On MI355X a streaming
// read of a large buffer runs 12-15% faster with this hint than with the default policy.
__device__ __forceinline__ uint4 load_b128_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Input of one wave's streaming pass over the context of one (sequence, KV head).
struct DecodeWaveIn {
  const uint16_t* q;       // query row at the first of the G packed heads: [G][D] bf16
  int G;                   // query heads packed on this KV head (<= 16)
  const uint8_t* kc;       // K plane (bytes)
  const uint8_t* vc;       // V plane (bytes)
  int64_t row_bytes;       // bytes of one token row (all KV heads)
  int64_t head_off;        // byte offset of this KV head within a token row
  const int32_t* bt_row;   // the sequence's block table row
  int num_blocks;          // ids outside 0..num_blocks-1 are skipped
  int tok_begin, tok_end;  // context tokens to attend (tok_begin a multiple of BS)
  float zscale;            // softmax scale * k_scale * log2(e)
};

// One wave attends the G packed query heads of one KV head over tokens
// [tok_begin, tok_end). On return lane l holds, for head slot l % 16: m (log2-domain
// running max), lsum (sum of weights over all lane groups) and o[mt] = unnormalised
// output for d = 16*mt + 4*(l/16) + r. my_vt: this wave's LDS V tile, 16 * (2*D+32) bytes.
// Layout of the work: see the description above decode_mfma_kernel in decode.hip.
template <int CDT, int D, int BS>
__device__ __forceinline__ void decode_wave(const DecodeWaveIn& in, uint8_t* my_vt, float& m, float& lsum,
                                            f32x4_t (&o)[D / 16]) {
  constexpr int CH = D / 4;                     // head_dim elements per lane group
  constexpr int KS = D / 32;                    // QK k-steps (16x16x32)
  constexpr int MT = D / 16;                    // PV d-tiles (16x16x16)
  constexpr int EB = CDT == PKV_BF16 ? 2 : 1;   // cache bytes per element
  constexpr int NV = CH * EB / 16;              // 16-byte loads per lane per tile (each of K, V)
  constexpr int SUB = BS / 16;                  // 16-token tiles per block
  constexpr int RS = D * 2 + 32;                // LDS row stride (bytes) of the bf16 V tile
  static_assert(NV >= 1 && CH % 8 == 0, "unsupported head_dim");
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;
  const int grp = lane >> 4;

  // queries: B operand of the QK MFMA, with the head_dim permutation of the K registers.
  // K load i of a lane reads bytes 64*i + 16*grp of its token's head row, so k-step kk of
  // lane group grp holds elements 32*kk + 8*grp .. +7 (bf16 cache) or, as half of a
  // 16-element E4M3 load, 64*(kk/2) + 16*grp + 8*(kk%2) .. +7.
  bf16x8_t qf[KS];
  {
    const uint16_t* qrow = in.q + int64_t(hl) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int d0 = EB == 2 ? 32 * kk + 8 * grp : 64 * (kk / 2) + 16 * grp + 8 * (kk % 2);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (hl < in.G) v = *reinterpret_cast<const uint4*>(qrow + d0);
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  m = -INFINITY;
  lsum = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint8_t* kc = in.kc;
  const uint8_t* vc = in.vc;
  const int64_t row_bytes = in.row_bytes;                           // one token, all KV heads
  const int64_t lane_off = in.head_off + 16 * grp;
  const int32_t* bt_row = in.bt_row;
  const int tok_begin = in.tok_begin, tok_end = in.tok_end;
  const int blk_begin = tok_begin / BS;
  const int blk_end = (tok_end + BS - 1) / BS;
  const int nblk = blk_end - blk_begin;
  const int ntiles = nblk * SUB;

  // block ids are wave-uniform: read them through the constant address space so they
  // become scalar loads (counted apart from the vector K/V loads, never draining them)
  const __attribute__((address_space(4))) int32_t* btc =
      (const __attribute__((address_space(4))) int32_t*)(uintptr_t)(bt_row);

  uint4 kb[2][NV], vb[2][NV];
  int tok0[2];
  bool okb[2];

  // K/V loads are unconditional (a skipped block reads block 0 and is zeroed after), so
  // the number of loads in flight is static and waits stay partial
  auto issue = [&](int n, uint4 (&kr)[NV], uint4 (&vr)[NV], int& t0, bool& ok) {
    const int j = n / SUB;
    const int sub = n % SUB;
    const int blk = btc[blk_begin + j];
    ok = blk >= 0 && blk < in.num_blocks;
    t0 = (blk_begin + j) * BS + sub * 16;
    const int64_t off = (int64_t(ok ? blk : 0) * BS + sub * 16 + hl) * row_bytes + lane_off;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      kr[i] = *reinterpret_cast<const uint4*>(kc + off + 64 * i);
      vr[i] = *reinterpret_cast<const uint4*>(vc + off + 64 * i);
    }
  };

  auto consume = [&](const uint4 (&kr)[NV], const uint4 (&vr)[NV], int t0, bool ok) {
    // ---- scores S^T[token][head] = K . Q^T
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (CDT == PKV_BF16) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[kk]), qf[kk], sc, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const uint4 lo = fp8x8_to_bf16x8(kr[i].x, kr[i].y);
        const uint4 hi = fp8x8_to_bf16x8(kr[i].z, kr[i].w);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo), qf[2 * i], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi), qf[2 * i + 1], sc, 0, 0, 0);
      }
    }
    // ---- V tile -> LDS as bf16 rows; rows of tokens past the context are zeroed
    {
      // load i holds head_dim elements 32*i + 8*grp .. +7 (bf16) or 64*i + 16*grp .. +15 (E4M3)
      const bool row_ok = ok && (t0 + hl < tok_end);
      uint8_t* dst = my_vt + hl * RS;
      if constexpr (CDT == PKV_BF16) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
          *reinterpret_cast<uint4*>(dst + 2 * (32 * i + 8 * grp)) = row_ok ? vr[i] : make_uint4(0, 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const uint4 lo = row_ok ? fp8x8_to_bf16x8(vr[i].x, vr[i].y) : make_uint4(0, 0, 0, 0);
          const uint4 hi = row_ok ? fp8x8_to_bf16x8(vr[i].z, vr[i].w) : make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4*>(dst + 2 * (64 * i + 16 * grp)) = lo;
          *reinterpret_cast<uint4*>(dst + 2 * (64 * i + 16 * grp) + 16) = hi;
        }
      }
    }
    // ---- online softmax for head hl over tokens t0 + 4*grp + r
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 4 * grp + r;
      z[r] = (ok && t < tok_end) ? sc[r] * in.zscale : -INFINITY;
    }
    float mt_ = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt_ = lane_groups_max(mt_);
    const float mn = fmaxf(m, mt_);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = pkv::fast_exp2(m - mref);
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = pkv::fast_exp2(z[r] - mref);
    // the weights are used in bf16 by the PV product; sum the same rounded values
    const uint32_t p01 = pack_bf16x2_rne(pr[0], pr[1]);
    const uint32_t p23 = pack_bf16x2_rne(pr[2], pr[3]);
    lsum = lsum * alpha + (pkv::bf16_lo(p01) + pkv::bf16_hi(p01)) + (pkv::bf16_lo(p23) + pkv::bf16_hi(p23));
    m = mn;
    const s16x4_t pf = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));
    __builtin_amdgcn_wave_barrier();
    // ---- O^T[d][head] += V^T[d][token] . P^T[token][head]
    const uint8_t* src = my_vt + (4 * grp + (hl >> 2)) * RS + (4 * (hl & 3)) * 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const s16x4_t vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 32 * mt));
      f32x4_t acc = o[mt];
      acc[0] *= alpha;
      acc[1] *= alpha;
      acc[2] *= alpha;
      acc[3] *= alpha;
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, acc, 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
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

  // lane-partial sums over the 4 lane groups (m is uniform per head across them)
  lsum = lane_groups_sum(lsum);
}

}  // namespace pkv
