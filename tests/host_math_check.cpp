// Host build of the kernels' integer MXFP4 math (csrc/mxfp4_math.h), driven
// row-wise exactly as a kernel lane does it: block max of magnitude bits, block
// parameters, closed-form or generic snap, sign, mask, nibble.  Compiled for
// the CPU by tests/test_host_math.py and compared with the oracle; it shares
// no code with the oracle.
#include <stdint.h>
#include <string.h>

#include "mxfp4_math.h"

using namespace mxfp4;

template <int DT>
static void run_block(const uint32_t *p, int n, int rule, float sf, uint32_t *y,
                      uint8_t *clip, uint8_t *nib, uint8_t *e8out) {
  constexpr uint32_t ABS = Fmt<DT>::ABS;
  uint32_t amax = 0;
  for (int j = 0; j < n; ++j) amax = max32(amax, p[j] & ABS);
  BlockParams bp;
  if (rule == kFloor) {
    bp = floor_params<DT>(amax);
  } else {
    float af = __builtin_bit_cast(float, DT == kBF16 ? amax << 16 : amax);
    bp = amct_params<DT>(amct_e8(af, sf));
  }
  *e8out = (uint8_t)bp.e8;
  for (int j = 0; j < n; ++j) {
    uint32_t a = p[j] & ABS;
    uint32_t mag, idx, six, sgn;
    if (bp.slow) {
      mag = slow_snap<DT>(a, bp.e8, &idx);
      six = slow_six<DT>(bp.e8);
    } else if (DT == kBF16) {
      // run the packed form with the element in the high half and a zero in
      // the low half, so both lanes of the packed ops are exercised
      uint32_t a2 = a << 16;
      uint32_t m2 = snap_mag_bf16(a2, splat16(bp.t025), splat16(bp.half));
      uint32_t i2 = snap_idx_bf16(a2, splat16(bp.t025));
      if ((m2 & 0xFFFF) != 0 || (i2 & 0xFFFF) != 0) { mag = 0xDEAD; idx = 15; six = 0; }
      else { mag = m2 >> 16; idx = i2 >> 16; six = bp.six; }
      uint32_t mb = mask_bits_bf16(a2, splat16(bp.six));
      if ((mb >> 16) != (a > bp.six ? 1u : 0u)) mag = 0xBEEF;
    } else {
      mag = snap_mag_f32(a, bp.t025, bp.half);
      idx = snap_idx_f32(a, bp.t025);
      six = bp.six;
    }
    if (DT == kBF16) {
      uint32_t s2 = sign_bf16(p[j] << 16 | p[j], splat16(bp.zc));
      sgn = s2 & 0x8000u;
      if ((s2 >> 16) != sgn) sgn = 0x4000;  // both halves must agree
    } else {
      sgn = sign_f32(p[j], bp.zc);
    }
    y[j] = mag | sgn;
    clip[j] = a > six;
    nib[j] = (uint8_t)(idx | (sgn ? 8 : 0));
  }
}

extern "C" int host_qdq_rows(int dtype, int64_t rows, int64_t cols, int block, int rule,
                             float sf, const void *x, void *y, uint8_t *clip, uint8_t *e8,
                             uint8_t *nib) {
  int64_t nb = (cols + block - 1) / block;
  uint32_t p[128], q[128];
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      int64_t c0 = b * block;
      int n = (int)((cols - c0) < block ? (cols - c0) : block);
      int64_t o = r * cols + c0;
      for (int j = 0; j < n; ++j)
        p[j] = dtype == kBF16 ? ((const uint16_t *)x)[o + j] : ((const uint32_t *)x)[o + j];
      if (dtype == kBF16)
        run_block<kBF16>(p, n, rule, sf, q, clip + o, nib + o, e8 + r * nb + b);
      else
        run_block<kF32>(p, n, rule, sf, q, clip + o, nib + o, e8 + r * nb + b);
      for (int j = 0; j < n; ++j) {
        if (dtype == kBF16) ((uint16_t *)y)[o + j] = (uint16_t)q[j];
        else ((uint32_t *)y)[o + j] = q[j];
      }
    }
  return 0;
}

// Packed FLOOR parameters of two bf16 columns vs the scalar rule, for every
// 16-bit max in the low half against a sweep of high halves.  Returns the
// number of mismatches.
extern "C" int host_check_packed_params(void) {
  int bad = 0;
  const uint32_t his[] = {0, 1, 0x7F, 0x80, 0x27F, 0x280, 0x3F80, 0x7F7F};
  for (uint32_t lo = 0; lo < 0x8000; ++lo)
    for (uint32_t hi : his) {
      const PackedParams p = floor_params_pk(lo | (hi << 16));
      const BlockParams a = floor_params<kBF16>(lo), b = floor_params<kBF16>(hi);
      bad += (p.e8 != (a.e8 | (b.e8 << 16)));
      bad += (p.t2 != (a.t025 | (b.t025 << 16)));
      bad += (p.h2 != (a.half | (b.half << 16)));
      bad += (p.s2 != (a.six | (b.six << 16)));
      bad += (p.slow != (a.slow || b.slow));
    }
  return bad;
}

// Generic decode of every (nibble, E8M0 byte) pair: out[e8 * 16 + nib] holds
// bf16 bits, out32 the fp32 bits the kernels derive from them (<< 16).
extern "C" void host_decode_all(uint16_t *out, uint32_t *out32) {
  for (uint32_t e8 = 0; e8 < 256; ++e8)
    for (uint32_t n = 0; n < 16; ++n) {
      uint32_t v = decode_bf16_generic(n, e8);
      out[e8 * 16 + n] = (uint16_t)v;
      out32[e8 * 16 + n] = v << 16;
    }
}

// Table-based packed E2M1 index vs the closed form, for every bf16 magnitude
// in both halves and every closed-form T (FLOOR T025 for E8M0 3..252, AMCT
// T025 - 1 for 97..254).  Returns the number of mismatches.
extern "C" int host_check_idx_table(void) {
  int bad = 0;
  for (uint32_t e8 = 3; e8 <= 254; ++e8) {
    for (int tau = 0; tau <= 1; ++tau) {
      if (tau == 1 && e8 < 97) continue;
      if (tau == 0 && e8 > 252) continue;
      const uint32_t t = ((e8 - 2) << 7) - (uint32_t)tau;
      const uint32_t t2 = splat16(t), t31 = splat16(t - 31);
      for (uint32_t a = 0; a < 0x8000; ++a) {
        const uint32_t p = a | ((a ^ 0x1234u) & 0x7FFFu) << 16;
        bad += snap_idx_bf16_tab(p, t31) != snap_idx_bf16(p, t2);
      }
    }
  }
  return bad;
}
