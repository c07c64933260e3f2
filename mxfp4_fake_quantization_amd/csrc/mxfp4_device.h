// mxfp4_device.h -- gfx950 device helpers: cross-lane reductions (DPP,
// ds_swizzle, ds_bpermute), 128-bit global loads/stores, launch constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxfp4_math.h"

namespace mxfp4 {

constexpr int kThreads = 256;  // 4 wave64 per workgroup

// DPP controls (GCN/CDNA encoding): quad_perm [1,0,3,2] and [2,3,0,1] swap
// neighbours at distance 1 and 2; row_ror:4 / row_ror:8 rotate a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// (old = 0 with bound_ctrl lets the compiler fold the move into the max/or
// that consumes it; every source lane used here exists.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// lane ^ 16 inside each 32-lane half (ds_swizzle bit mode: and 0x1F, xor 0x10)
__device__ __forceinline__ uint32_t lane_xor16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
// lane ^ 32 (ds_bpermute takes a byte address of the source lane)
__device__ __forceinline__ uint32_t lane_xor32(uint32_t v) {
  int src = (int)((__lane_id() ^ 32u) << 2);
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v);
}

// ---- reductions over aligned lane groups ---------------------------------
// Groups of 4 consecutive lanes (quad), 16 (a DPP row), or lanes that share
// bits 0-1 and differ in bits 2-3 (stride-4 groups inside a row) or 2-5.
__device__ __forceinline__ uint32_t max_quad(uint32_t v) {
  v = max32(v, dpp<kDppQuadXor1>(v));
  return max32(v, dpp<kDppQuadXor2>(v));
}
__device__ __forceinline__ uint32_t pkmax_quad(uint32_t v) {
  v = pk_max(v, dpp<kDppQuadXor1>(v));
  return pk_max(v, dpp<kDppQuadXor2>(v));
}
__device__ __forceinline__ uint32_t or_quad(uint32_t v) {
  v |= dpp<kDppQuadXor1>(v);
  return v | dpp<kDppQuadXor2>(v);
}
__device__ __forceinline__ uint32_t max_stride4_row(uint32_t v) {  // lane bits 2,3
  v = max32(v, dpp<kDppRowRor4>(v));
  return max32(v, dpp<kDppRowRor8>(v));
}
__device__ __forceinline__ uint32_t or_stride4_row(uint32_t v) {
  v |= dpp<kDppRowRor4>(v);
  return v | dpp<kDppRowRor8>(v);
}
__device__ __forceinline__ uint32_t max_stride4_wave(uint32_t v) {  // lane bits 2..5
  v = max_stride4_row(v);
  v = max32(v, lane_xor16(v));
  return max32(v, lane_xor32(v));
}

// Maximum over the G consecutive lanes that hold one row-wise block
// (G = block / 8: 4 for 32-element blocks, 16 for 128).
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  static_assert(G == 4 || G == 16, "group of 4 or 16 lanes");
  v = max_quad(v);
  if (G == 16) v = max_stride4_row(v);
  return v;
}

// ---- memory --------------------------------------------------------------
// Streaming 16-byte accesses: every element is read once and written once,
// so loads and stores are non-temporal (no reuse to keep in the caches).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const void *p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(void *p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// Small stores (bitmap bytes, packed-code words, scale bytes); a
// non-temporal hint measured no faster for them on MI355X, so it is off.
#ifndef MXFP4_NT_SMALL
#define MXFP4_NT_SMALL 0
#endif
template <typename T>
__device__ __forceinline__ void st_small(T *p, T v) {
  if (MXFP4_NT_SMALL) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// An 8-element piece of one row (16 bytes of bf16, 32 of fp32) as NW words;
// elements past n read as +0.  VEC: the row is 16-byte aligned at the piece,
// so a whole piece is one (bf16) or two (fp32) 16-byte loads.
template <int DT>
struct PieceT {
  static constexpr int NW = DT == kBF16 ? 4 : 8;  // words per 8-element piece
  static constexpr int ES = DT == kBF16 ? 2 : 4;  // bytes per element
};
template <int DT, bool VEC>
__device__ __forceinline__ void load_piece(uint32_t *w, const uint8_t *p, int n) {
  constexpr int NW = PieceT<DT>::NW;
  if (VEC) {
    if (n == 8) {
      uint4 v = ld16(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      if (DT == kF32) {
        uint4 v2 = ld16(p + 16);
        w[4] = v2.x; w[5] = v2.y; w[6] = v2.z; w[7] = v2.w;
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < NW; ++k) w[k] = 0;
  if (!VEC) {
    for (int j = 0; j < n; ++j) {
      if (DT == kBF16) w[j >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(p)[j] << (16 * (j & 1));
      else w[j] = reinterpret_cast<const uint32_t *>(p)[j];
    }
  }
}

__device__ __forceinline__ float bits_f32(uint32_t b) { return __builtin_bit_cast(float, b); }

// Block parameters for one block (or column) from its max magnitude bits.
template <int DT, int RULE>
__device__ __forceinline__ BlockParams block_params(uint32_t amax, float sf) {
  if (RULE == kFloor) return floor_params<DT>(amax);
  float af = bits_f32(DT == kBF16 ? amax << 16 : amax);
  return amct_params<DT>(amct_e8(af, sf));
}

}  // namespace mxfp4

namespace mxfp4 {

// Packed u16 min written as the instruction itself: left to the compiler,
// min(x, 1) on a packed pair is rewritten into per-half compares, selects and
// a byte permute (five instructions instead of one).  ALU only.
__device__ __forceinline__ uint32_t pk_min_v(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// min(x, 1) on both halves with the inline constant 1 (op_sel_hi:[1,0] makes
// the high half read the constant too), so no register holds 0x00010001.
__device__ __forceinline__ uint32_t pk_min1(uint32_t a) {
  uint32_t r;
  asm("v_pk_min_u16 %0, %1, 1 op_sel_hi:[1,0]" : "=v"(r) : "v"(a));
  return r;
}

// ---- per-word outputs, bf16 (two elements per register) -------------------
// Parameters are packed per half (t2 = T025 - tau, h2 = HALF, s2 = SIX), so a
// register may hold two elements of one block or of two different blocks.
// y bits with the sign rule of the block (zc2 = ABS - Z per half)
__device__ __forceinline__ uint32_t y_bf16(uint32_t w, uint32_t t2, uint32_t h2, uint32_t zc2) {
  uint32_t a = w & 0x7FFF7FFFu;
  uint32_t u = pk_subsat(a, t2);
  uint32_t r = pk_add(u, 0x001F001Fu) & 0xFFC0FFC0u;
  uint32_t h = pk_min(pk_subsat(r, 0x01000100u), 0x01400140u);
  uint32_t z = pk_min1(u);
  uint32_t c = pk_min1(pk_subsat(u, 0x00C000C0u));
  return pk_mad(c, 0x00800080u, pk_mad(z, h2, h)) | sign_bf16(w, zc2);
}
// clip bits: bit 0 (low element) and bit 16 (high element)
__device__ __forceinline__ uint32_t m_bf16(uint32_t w, uint32_t s2) {
  return pk_min1(pk_subsat(w & 0x7FFF7FFFu, s2));
}
// nibbles sign<<3 | code in bits 0-3 and 16-19
__device__ __forceinline__ uint32_t n_bf16(uint32_t w, uint32_t t2, uint32_t zc2) {
  uint32_t a = w & 0x7FFF7FFFu;
  uint32_t u = pk_subsat(a, t2);
  uint32_t r = pk_add(u, 0x001F001Fu) & 0xFFC0FFC0u;
  uint32_t h = pk_min(pk_subsat(r, 0x01000100u), 0x01400140u);
  uint32_t z = pk_min1(u);
  uint32_t c = pk_min1(pk_subsat(u, 0x00C000C0u));
  return pk_add(pk_add(z, c), pk_shr(h, 6)) | (sign_bf16(w, zc2) >> 12);
}



// Generic snap of one half (FLOOR blocks with E8M0 byte 0..2, scale 2^k with
// k = e8 - 127 <= -125).  In binary32, x * 2^-k is exact and normal (bf16
// values are multiples of 2^-133 and 2^-k >= 2^125; these kernels keep
// binary32 denormals), so the binary32 closed form at unit scale (threshold
// bits of 0.25, half 0.5) gives the index and the code value, and
// code * 2^k is again exact (>= 2^-128, at most two significant bits) with
// zero low 16 bits.  Two v_ldexp_f32 per value; no per-block tables, which
// keeps the rare path's registers low.
struct HalfOut {
  uint32_t y, m, n;
};
__device__ __forceinline__ HalfOut half_bf16_slow(uint32_t bits16, uint32_t e8) {
  const uint32_t a = bits16 & 0x7FFFu;
  const uint32_t sg = (bits16 & 0x8000u) && a ? 0x8000u : 0u;
  const int k = (int)e8 - 127;
  const uint32_t v = __builtin_bit_cast(uint32_t, __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, a << 16), -k));
  const float q = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, snap_mag_f32(v, 0x3E800000u, 0x3F000000u)), k);
  HalfOut o;
  o.y = (__builtin_bit_cast(uint32_t, q) >> 16) | sg;
  o.m = v > 0x40C00000u ? 1u : 0u;  // x > 6 * 2^k
  o.n = snap_idx_f32(v, 0x3E800000u) | (sg >> 12);
  return o;
}

// ---- fp32 (one element per register) -------------------------------------
__device__ __forceinline__ uint32_t y_f32(uint32_t w, const BlockParams &bp) {
  uint32_t a = w & 0x7FFFFFFFu;
  if (bp.slow) return slow_snap<kF32>(a, bp.e8, nullptr) | sign_f32(w, bp.zc);
  return snap_mag_f32(a, bp.t025, bp.half) | sign_f32(w, bp.zc);
}
__device__ __forceinline__ uint32_t m_f32(uint32_t w, const BlockParams &bp) {
  uint32_t a = w & 0x7FFFFFFFu;
  return a > (bp.slow ? slow_six<kF32>(bp.e8) : bp.six) ? 1u : 0u;
}
__device__ __forceinline__ uint32_t n_f32(uint32_t w, const BlockParams &bp) {
  uint32_t a = w & 0x7FFFFFFFu;
  uint32_t idx;
  if (bp.slow) slow_snap<kF32>(a, bp.e8, &idx);
  else idx = snap_idx_f32(a, bp.t025);
  return idx | (sign_f32(w, bp.zc) >> 28);
}

// 8 nibbles of a bf16 chunk (four words, element 2d in the low half of word
// d) -> one dword, element j in bits 4j..4j+3.
__device__ __forceinline__ uint32_t pack_nibbles_bf16(const uint32_t n[4]) {
  uint32_t w0 = n[0] | (n[1] << 8);  // e0@0 e2@8 e1@16 e3@24
  uint32_t w1 = n[2] | (n[3] << 8);  // e4@0 e6@8 e5@16 e7@24
  uint32_t lo = (w0 & 0x0F0Fu) | (w0 >> 12);
  uint32_t hi = (w1 & 0x0F0Fu) | (w1 >> 12);
  return lo | (hi << 16);
}
// clip bits of a bf16 chunk (bit 0 / bit 16 of four words) -> byte, element j
// in bit j.
__device__ __forceinline__ uint32_t pack_mask_bf16(const uint32_t m[4]) {
  uint32_t t = m[0] | (m[1] << 2) | (m[2] << 4) | (m[3] << 6);
  return (t | (t >> 15)) & 0xFFu;
}

// ---- whole 8-element chunk with one block's parameters (row direction) ----
// SLOW = false: closed form only (the caller has checked that no lane of the
// wave holds a block that needs the generic snap); SLOW = true: lanes whose
// block needs it take the generic threshold count.  Keeping the two apart
// leaves the common path free of calls and of the generic code.
template <int DT, bool SLOW>
__device__ __forceinline__ void chunk_y(const uint32_t *w, const BlockParams &bp, uint32_t *y) {
  if (DT == kBF16) {
    const uint32_t t2 = splat16(bp.t025), h2 = splat16(bp.half), z2 = splat16(bp.zc);
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = y_bf16(w[k], t2, h2, z2);
    if (SLOW && bp.slow) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        HalfOut lo = half_bf16_slow(w[k] & 0xFFFFu, bp.e8), hi = half_bf16_slow(w[k] >> 16, bp.e8);
        y[k] = lo.y | (hi.y << 16);
      }
    }
  } else {
    BlockParams q = bp;
    if (!SLOW) q.slow = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = y_f32(w[k], q);
  }
}
template <int DT, bool SLOW>
__device__ __forceinline__ uint32_t chunk_mask(const uint32_t *w, const BlockParams &bp) {
  if (DT == kBF16) {
    uint32_t m[4];
    const uint32_t s2 = splat16(bp.six);
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = m_bf16(w[k], s2);
    if (SLOW && bp.slow) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        HalfOut lo = half_bf16_slow(w[k] & 0xFFFFu, bp.e8), hi = half_bf16_slow(w[k] >> 16, bp.e8);
        m[k] = lo.m | (hi.m << 16);
      }
    }
    return pack_mask_bf16(m);
  }
  BlockParams q = bp;
  if (!SLOW) q.slow = false;
  uint32_t byte = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) byte |= m_f32(w[k], q) << k;
  return byte;
}
template <int DT, bool SLOW>
__device__ __forceinline__ uint32_t chunk_codes(const uint32_t *w, const BlockParams &bp) {
  if (DT == kBF16) {
    uint32_t n[4];
    const uint32_t t31 = splat16(bp.t025 - 31u), z2 = splat16(bp.zc);
#pragma unroll
    for (int k = 0; k < 4; ++k) n[k] = snap_idx_bf16_tab(w[k] & 0x7FFF7FFFu, t31) | (sign_bf16(w[k], z2) >> 12);
    if (SLOW && bp.slow) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        HalfOut lo = half_bf16_slow(w[k] & 0xFFFFu, bp.e8), hi = half_bf16_slow(w[k] >> 16, bp.e8);
        n[k] = lo.n | (hi.n << 16);
      }
    }
    return pack_nibbles_bf16(n);
  }
  BlockParams q = bp;
  if (!SLOW) q.slow = false;
  uint32_t nib = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) nib |= n_f32(w[k], q) << (4 * k);
  return nib;
}

}  // namespace mxfp4
