// mxfp4_math.h -- integer-domain MXFP4 arithmetic shared by the gfx950 kernels.
//
// Everything here works on IEEE bit patterns of |x| ("magnitude bits" a), so
// the block maximum, the scale exponent, the E2M1 snap, the clip mask, the
// sign and the packed nibble are integer operations with no rounding at all.
// bf16 elements are processed two per 32-bit register with packed 16-bit ALU
// ops (v_pk_*_u16); fp32 elements one per register.  The functions are
// __host__ __device__ so the same code can be checked on the CPU.
//
// Method (amct PR "MXFP4 QAT fake-quant Linear (with STE)", README section 1
// and fake_quant.py _block_scale / _round_to_e2m1 / _quant_dequant_torch):
// with block scale 2^k, |x|/2^k is snapped to the E2M1 code nearest to it by
// the midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 and the result is clipped at
// 6 * 2^k; the clipped-STE mask is |x| > 6 * 2^k.
//
// Notation: MB = mantissa bits (bf16 7, fp32 23), Q = 2^(MB-1) = one step of a
// 1-bit mantissa, E = biased scale exponent (E8M0 byte, k = E - 127).
// For E >= 3 every threshold and code c*2^k (c >= 0.25) is a normal number
// and the snap has a closed form in a-space:
//   T025 = (E-2) << MB        bits of 0.25*2^k  (HALF - 2Q, ONE - 4Q)
//   HALF = T025 + 2Q          bits of 0.5*2^k
//   SIX  = T025 + 9Q          bits of 6*2^k
//   u = sat(a - (T025 - tau))          tau = 0 (FLOOR, ties down) / 1 (AMCT, ties up)
//   r = (u + Q/2 - 1) & ~(Q-1)         keep one mantissa bit of 2^? >= 1.0 values
//   h = min(sat(r - 4Q), 5Q)           offset above 1.0*2^k, clipped at 6*2^k
//   z = min(u, 1)                      |x| passes the 0.25 midpoint
//   c = min(sat(u - 3Q), 1)            |x| passes the 0.75 midpoint
//   mag = h + z*HALF + c*2Q            bits of code*2^k
//   idx = z + c + h/Q                  E2M1 magnitude code 0..7
// (T025 is a multiple of Q, so rounding u rounds a.)  For E < 3 (only FLOOR
// blocks with amax < 2^-122) a generic threshold count is used instead.
//
// Sign: the output (and the nibble's sign bit) is negative iff x < 0 and
// |x| > Z, with Z = 0 for FLOOR (exact arithmetic: -0.0 -> +0.0, any other
// negative keeps its sign).  AMCT follows the pages' binary32 arithmetic,
// where the sign is that of the rounded quotient fl32(x / 2^k): it underflows
// to zero (torch.sign 0, output +0) when |x| <= 2^(k-150), so Z = that power
// of two (0 when no positive value of the dtype is that small).  Kept as an
// addend zc = ABS - Z: bit 15 (bf16 half) or 31 (fp32) of a + zc is set
// exactly when a > Z.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MXFP4_HD __host__ __device__ __forceinline__
#else
#define MXFP4_HD inline
#endif

namespace mxfp4 {

enum { kF32 = 0, kBF16 = 1 };
enum { kFloor = 0, kAmct = 1 };

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

MXFP4_HD u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
MXFP4_HD uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// ---- packed 16-bit helpers (two bf16 per register) -------------------------
MXFP4_HD uint32_t pk_subsat(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_sub_sat(as_u16x2(a), as_u16x2(b)));
}
MXFP4_HD uint32_t pk_min(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_min(as_u16x2(a), as_u16x2(b)));
}
MXFP4_HD uint32_t pk_max(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
}
MXFP4_HD uint32_t pk_add(uint32_t a, uint32_t b) { return as_u32(as_u16x2(a) + as_u16x2(b)); }
MXFP4_HD uint32_t pk_sub(uint32_t a, uint32_t b) { return as_u32(as_u16x2(a) - as_u16x2(b)); }
MXFP4_HD uint32_t pk_mad(uint32_t a, uint32_t b, uint32_t c) {
  return as_u32(as_u16x2(a) * as_u16x2(b) + as_u16x2(c));
}
MXFP4_HD uint32_t pk_shr(uint32_t a, unsigned s) {
  u16x2 sh = {(unsigned short)s, (unsigned short)s};
  return as_u32(as_u16x2(a) >> sh);
}
MXFP4_HD uint32_t pk_shl7(uint32_t a) {
  u16x2 sh = {7, 7};
  return as_u32(as_u16x2(a) << sh);
}
MXFP4_HD uint32_t splat16(uint32_t v) { return (v & 0xFFFFu) | (v << 16); }

MXFP4_HD uint32_t subsat32(uint32_t a, uint32_t b) { return a > b ? a - b : 0u; }
MXFP4_HD uint32_t min32(uint32_t a, uint32_t b) { return a < b ? a : b; }
MXFP4_HD uint32_t max32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ---- per-dtype constants -----------------------------------------------------
template <int DT> struct Fmt;
template <> struct Fmt<kBF16> {
  static constexpr int MB = 7;
  static constexpr uint32_t Q = 1u << 6;
  static constexpr uint32_t ABS = 0x7FFFu;
  static constexpr uint32_t SIGN = 0x8000u;
};
template <> struct Fmt<kF32> {
  static constexpr int MB = 23;
  static constexpr uint32_t Q = 1u << 22;
  static constexpr uint32_t ABS = 0x7FFFFFFFu;
  static constexpr uint32_t SIGN = 0x80000000u;
};

// Block parameters derived from the block's max magnitude bits.
struct BlockParams {
  uint32_t e8;    // E8M0 byte (k + 127) reported for the block
  uint32_t t025;  // T025 - tau  (u threshold)
  uint32_t half;  // bits of 0.5 * 2^k
  uint32_t six;   // bits of 6 * 2^k (mask: a > six)
  uint32_t zc;    // ABS - Z: the sign is kept iff a + zc reaches the sign bit
  bool slow;      // FLOOR with 0 < amax < 2^-122: use the generic snap
};

// FLOOR scale: k = floor(log2 amax) - 2 clamped at -127.  From the bits,
// E = max(Eb - 2, 0) with Eb the biased exponent field of amax (0 for
// subnormal or zero amax).  The closed-form snap is used with Ec = max(E, 3);
// for a zero block any Ec >= 3 gives zeros, other E < 3 blocks go slow.
template <int DT>
MXFP4_HD BlockParams floor_params(uint32_t amax) {
  constexpr int MB = Fmt<DT>::MB;
  constexpr uint32_t Q = Fmt<DT>::Q;
  uint32_t eb = amax >> MB;
  BlockParams p;
  p.e8 = eb > 2 ? eb - 2 : 0;
  uint32_t ec = (eb > 5 ? eb : 5) - 2;
  p.t025 = (ec - 2) << MB;
  p.half = p.t025 + 2 * Q;
  p.six = p.t025 + 9 * Q;
  p.zc = Fmt<DT>::ABS;
  p.slow = (amax != 0) && (eb < 5);
  return p;
}

// FLOOR parameters of two bf16 columns at once (one per half of cm, the
// packed column maxima): E8M0 bytes, T025, HALF, SIX, and the halves that
// need the generic snap (nonzero max with an exponent field below 5).
struct PackedParams {
  uint32_t e8, t2, h2, s2;
  bool slow;
};
MXFP4_HD PackedParams floor_params_pk(uint32_t cm) {
  PackedParams p;
  const uint32_t eb = pk_shr(cm, 7);
  p.e8 = pk_subsat(eb, 0x00020002u);
  p.t2 = pk_shl7(pk_subsat(pk_max(eb, 0x00050005u), 0x00040004u));
  p.h2 = pk_add(p.t2, 0x00800080u);
  p.s2 = pk_add(p.t2, 0x02400240u);
  // slow <=> 0 < cm_half < 5 << 7, i.e. (cm_half - 1) mod 2^16 < 639
  const uint32_t m1 = pk_sub(cm, 0x00010001u);
  p.slow = (m1 & 0xFFFFu) < 639u || (m1 >> 16) < 639u;
  return p;
}

// AMCT E8M0 byte from the block max, as the pages' binary32 arithmetic
// computes it: r = fl32(amax / sf) (IEEE division), r = max(r, 2^-30),
// L = log2 r rounded to the nearest binary32, k = L rounded half to even
// (torch.round).  With r = 2^e * m (m in [1, 2), mantissa field M):
//   - away from log2 m = 1/2, L rounds to the integer nearest to log2 r,
//     e + (m > sqrt 2) (0x3504F3 is the largest field below sqrt 2 - 1);
//   - L is exactly the half-integer e + 1/2 when |log2 m - 1/2| is below half
//     an ulp of e + 1/2, i.e. 2^(j - 24) with j = floor(log2 |e + 1/2|); then
//     the tie goes to the even integer, k = e + (e & 1).
// Those fields M form a window around sqrt 2 that widens with j; with
// i = j + 1 = floor(log2 |2e + 1|) in 0..7 (e in [-30, 127]) it is
// [0x3504F3 - lo_i, 0x3504F3 + hi_i], lo = 0 0 0 1 3 7 15 31 and
// hi = 0 0 1 2 4 8 15 31, found by evaluating 2^(1/2 -+ 2^(j-24)) to 50
// digits (the byte tables below, one byte per i).
MXFP4_HD uint32_t amct_e8(float amax_f, float sf) {
  float r = amax_f / sf;
  if (!(r >= 0x1p-30f)) r = 0x1p-30f;
  const uint32_t rb = __builtin_bit_cast(uint32_t, r);
  const uint32_t eb = rb >> 23, m = rb & 0x7FFFFFu;
  const int e = (int)eb - 127;
  const uint32_t t = (uint32_t)(e < 0 ? -(2 * e + 1) : 2 * e + 1);  // |2e + 1|, 1..255
  const unsigned i = 31u - (unsigned)__builtin_clz(t);
  const uint32_t lo = (uint32_t)(0x1F0F070301000000ull >> (8 * i)) & 0xFFu;
  const uint32_t hi = (uint32_t)(0x1F0F080402010000ull >> (8 * i)) & 0xFFu;
  const bool tie = m + lo >= 0x3504F3u && m <= 0x3504F3u + hi;
  const uint32_t up = tie ? (uint32_t)(e & 1) : (m > 0x3504F3u ? 1u : 0u);
  const uint32_t e8 = eb + up;
  return e8 > 254u ? 254u : e8;
}

template <int DT>
MXFP4_HD BlockParams amct_params(uint32_t e8) {
  constexpr int MB = Fmt<DT>::MB;
  constexpr uint32_t Q = Fmt<DT>::Q;
  BlockParams p;
  p.e8 = e8;  // >= 97 always, so the closed form applies
  uint32_t t025 = (e8 - 2) << MB;
  p.t025 = t025 - 1;
  p.half = t025 + 2 * Q;
  p.six = t025 + 9 * Q;
  // Z = bits of 2^(k-150) = 2^(e8-277): normal from e8 = 151, a subnormal of
  // the dtype (unit 2^-133 bf16, 2^-149 fp32) from e8 = 144 / 128, else 0.
  constexpr uint32_t sub0 = DT == kBF16 ? 144u : 128u;
  const uint32_t z = e8 >= 151u ? (e8 - 150u) << MB : (e8 >= sub0 ? 1u << (e8 - sub0) : 0u);
  p.zc = Fmt<DT>::ABS - z;
  p.slow = false;
  return p;
}

// ---- closed-form snap --------------------------------------------------------
// bf16: two elements per register, constants replicated (or per-half).
struct SnapBF16 {
  uint32_t mag;  // packed magnitude bits of code * 2^k
  uint32_t idx;  // packed E2M1 magnitude codes (0..7)
};

MXFP4_HD uint32_t snap_mag_bf16(uint32_t a, uint32_t t025p2, uint32_t half2) {
  uint32_t u = pk_subsat(a, t025p2);
  uint32_t r = pk_add(u, 0x001F001Fu) & 0xFFC0FFC0u;
  uint32_t h = pk_min(pk_subsat(r, 0x01000100u), 0x01400140u);
  uint32_t z = pk_min(u, 0x00010001u);
  uint32_t c = pk_min(pk_subsat(u, 0x00C000C0u), 0x00010001u);
  return pk_mad(c, 0x00800080u, pk_mad(z, half2, h));
}

MXFP4_HD uint32_t snap_idx_bf16(uint32_t a, uint32_t t025p2) {
  uint32_t u = pk_subsat(a, t025p2);
  uint32_t r = pk_add(u, 0x001F001Fu) & 0xFFC0FFC0u;
  uint32_t h = pk_min(pk_subsat(r, 0x01000100u), 0x01400140u);
  uint32_t z = pk_min(u, 0x00010001u);
  uint32_t c = pk_min(pk_subsat(u, 0x00C000C0u), 0x00010001u);
  return pk_add(pk_add(z, c), pk_shr(h, 6));
}

// Byte permute of the 8-byte pool {hi:lo} (bytes 0-3 from lo, 4-7 from hi):
// result byte i = pool[sel byte i] for selector values 0..7, 0x00 for 12
// (v_perm_b32; the host form covers exactly these values).
MXFP4_HD uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(hi, lo, sel);
#else
  const uint64_t pool = ((uint64_t)hi << 32) | lo;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (sel >> (8 * i)) & 0xFFu;
    const uint32_t v = b < 8 ? (uint32_t)(pool >> (8 * b)) & 0xFFu : 0u;  // 12 -> 0x00
    r |= v << (8 * i);
  }
  return r;
#endif
}

// E2M1 codes of two bf16 magnitudes by table: with u = sat(a - T) as in
// snap_idx_bf16 (T = T025 - tau) and v = ceil(u / (Q/2)) (Q/2 = 32), the
// thresholds 0.25 0.75 1.25 1.75 2.5 3.5 5 (times 2^k) are passed exactly when
// v >= 1, 7, 10, 12, 14, 16, 18, so
//   idx = L[min(v, 7)] + min((v - 8) >> 1 saturated at 0, 5),
//   L = {0, 1, 1, 1, 1, 1, 1, 2} (one v_perm lookup for both halves).
// t31 = T - 31 per half (T >= 127 for every block that takes the closed
// form), which folds the ceiling into the saturated subtraction.
MXFP4_HD uint32_t snap_idx_bf16_tab(uint32_t a, uint32_t t31) {
  const uint32_t v = pk_shr(pk_subsat(a, t31), 5);
  const uint32_t lo = perm_b32(0x02010101u, 0x01010100u, pk_min(v, 0x00070007u));
  const uint32_t hi = pk_min(pk_shr(pk_subsat(v, 0x00080008u), 1), 0x00050005u);
  return pk_add(lo, hi);
}

// sign bits kept for negative inputs with |x| > Z (zc2 = ABS - Z per half;
// FLOOR: Z = 0, so only -0.0 loses its sign)
MXFP4_HD uint32_t sign_bf16(uint32_t p, uint32_t zc2) {
  return p & pk_add(p & 0x7FFF7FFFu, zc2) & 0x80008000u;
}
// the FLOOR case (Z = 0) in fewer registers: bit 15 of p - 1 is set for every
// negative half but -0.0
MXFP4_HD uint32_t sign_bf16_floor(uint32_t p) { return p & pk_sub(p, 0x00010001u) & 0x80008000u; }
MXFP4_HD uint32_t mask_bits_bf16(uint32_t a, uint32_t six2) {
  return pk_min(pk_subsat(a, six2), 0x00010001u);
}

// fp32: one element per register.
MXFP4_HD uint32_t snap_mag_f32(uint32_t a, uint32_t t025p, uint32_t half) {
  constexpr uint32_t Q = Fmt<kF32>::Q;
  uint32_t u = subsat32(a, t025p);
  uint32_t r = (u + (Q / 2 - 1)) & ~(Q - 1);
  uint32_t h = min32(subsat32(r, 4 * Q), 5 * Q);
  uint32_t z = min32(u, 1u);
  uint32_t c = min32(subsat32(u, 3 * Q), 1u);
  return h + z * half + c * (2 * Q);
}
MXFP4_HD uint32_t snap_idx_f32(uint32_t a, uint32_t t025p) {
  constexpr uint32_t Q = Fmt<kF32>::Q;
  uint32_t u = subsat32(a, t025p);
  uint32_t r = (u + (Q / 2 - 1)) & ~(Q - 1);
  uint32_t h = min32(subsat32(r, 4 * Q), 5 * Q);
  uint32_t z = min32(u, 1u);
  uint32_t c = min32(subsat32(u, 3 * Q), 1u);
  return z + c + (h >> 22);
}
MXFP4_HD uint32_t sign_f32(uint32_t p, uint32_t zc) { return p & ((p & 0x7FFFFFFFu) + zc) & 0x80000000u; }

// ---- generic snap for FLOOR blocks with E8M0 byte 0, 1 or 2 ------------------
// Values are handled as integer multiples L of the dtype's smallest subnormal
// (bf16 2^-133, fp32 2^-149); lin_to_bits turns such an L (with at most MB+1
// significant bits) into IEEE magnitude bits, subnormal or normal.
template <int DT>
MXFP4_HD uint32_t lin_to_bits(uint32_t L) {
  constexpr int MB = Fmt<DT>::MB;
  if (L < (2u << MB)) return L;
  int msb = 31 - __builtin_clz(L);
  int e = msb - MB;
  return ((uint32_t)e << MB) + (L >> e);
}

// Snap one magnitude (32-bit, low bits) for E8M0 byte e8 in {0,1,2}: count the
// midpoints m*2^k (m = n/4, n = 1 3 5 7 10 14 20) that |x| exceeds, then
// return the bits of code*2^k (code*4 = 0 2 4 6 8 12 16 24, i.e. 2*idx for
// idx < 2 and (2 + idx%2) << idx/2 above).
template <int DT>
MXFP4_HD uint32_t slow_snap(uint32_t a, uint32_t e8, uint32_t *idx_out) {
  constexpr int MB = Fmt<DT>::MB;
  const unsigned sh = e8 + MB - 3;  // 2^(k-2) in subnormal units
  uint32_t idx = 0;
  idx += (a > lin_to_bits<DT>(1u << sh)) ? 1u : 0u;
  idx += (a > lin_to_bits<DT>(3u << sh)) ? 1u : 0u;
  idx += (a > lin_to_bits<DT>(5u << sh)) ? 1u : 0u;
  idx += (a > lin_to_bits<DT>(7u << sh)) ? 1u : 0u;
  idx += (a > lin_to_bits<DT>(10u << sh)) ? 1u : 0u;
  idx += (a > lin_to_bits<DT>(14u << sh)) ? 1u : 0u;
  idx += (a > lin_to_bits<DT>(20u << sh)) ? 1u : 0u;
  if (idx_out) *idx_out = idx;
  const uint32_t c4 = idx < 2 ? 2 * idx : (2 + (idx & 1)) << (idx >> 1);
  return lin_to_bits<DT>(c4 << sh);
}
template <int DT>
MXFP4_HD uint32_t slow_six(uint32_t e8) {
  constexpr int MB = Fmt<DT>::MB;
  return lin_to_bits<DT>(24u << (e8 + MB - 3));
}


// ---- decoding a packed nibble --------------------------------------------
// value = (-1)^s * code * 2^(e8 - 127).  For code index i >= 1 the code is
// 2^((i>>1) - 1) * (1 + m/2) with m = (i >= 2) & i, so the biased result
// exponent is Eb = e8 + (i>>1) - 1: normal for 1 <= Eb <= 254, +-inf above
// (the product exceeds the largest finite value), and for Eb in {-1, 0} the
// subnormal (2 + m) * 2^(Eb - 128).  For 2 <= e8 <= 252 every code is normal
// (the closed form the kernels use); this generic form covers every byte.
// Returns bf16 bits (fp32 bits are these << 16: same exponent range, and
// every decoded value has at most two significant bits).
MXFP4_HD uint32_t decode_bf16_generic(uint32_t nib, uint32_t e8) {
  const uint32_t i = nib & 7u, sg = (nib & 8u) << 12;
  if (i == 0) return sg;
  const int eb = (int)e8 + (int)(i >> 1) - 1;
  const uint32_t m = i >= 2 ? (i & 1u) : 0u;
  uint32_t mag;
  if (eb >= 255) mag = 0x7F80u;
  else if (eb >= 1) mag = ((uint32_t)eb << 7) | (m << 6);
  else mag = (2u + m) << (5 + eb);  // bf16 subnormal unit 2^-133
  return mag | sg;
}

}  // namespace mxfp4
