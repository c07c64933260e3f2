// col_kernels.hip -- column-wise, dual-direction and grouped MXFP4 fake
// quantization on gfx950.
//
// Column-wise blocks are `block` consecutive rows of one column (the
// hyper-parallel page's column-direction operand); grouped blocks restart at
// every expert-group start (its "grouped dynamic quantization" along tokens);
// the dual-direction launch produces the row-wise and the column-wise view of
// the same tensor from one read of x.
//
// Tiling: a wave owns 32 rows x 128 columns.  Lane = rg + 4*cc holds rows
// 8*rg .. 8*rg+7 of the slab and the 8 columns 8*cc .. 8*cc+7 (one 16-byte bf16
// piece per row, i.e. 256-byte row segments per load instruction).
//   - column max: in-register max over the lane's 8 rows, then a DPP quad
//     reduction over rg; for 128-row blocks the four waves of the workgroup
//     (stacked vertically) exchange their partial maxima through LDS;
//   - row max (dual): DPP row_ror 4/8 over the 4 lanes of a 32-column block
//     (plus ds_swizzle / ds_bpermute steps for 128-column blocks);
//   - column bitmap words (bit = row) are assembled by OR-ing each lane's
//     8-row byte across the quad, then every lane stores 2 words so the wave
//     writes one contiguous 512-byte stretch.
// For block 32 the workgroup is 4 waves side by side (32 x 512), for block
// 128 4 waves stacked (128 x 128): one workgroup = one block-row x one column
// tile, which makes grouped block-rows (arbitrary start rows) free of any
// alignment constraint on the loads.
#include "mxfp4_device.h"
#include "mxfp4_groups.h"
#include "mxfp4_kernels.h"

namespace mxfp4 {
namespace {

enum { kKindCol = 0, kKindDual = 1, kKindGrouped = 2 };
// Minimum workgroups per CU requested from the compiler, which caps the
// VGPRs (3 -> 168, 4 -> 128); chosen by measurement on MI355X.
#ifndef MXFP4_COL_MINWG
#define MXFP4_COL_MINWG 3
#endif
#ifndef MXFP4_DUAL_MINWG
#define MXFP4_DUAL_MINWG 3
#endif
#ifndef MXFP4_GROUPED_MINWG
#define MXFP4_GROUPED_MINWG 4
#endif
constexpr int kWaveCols = 128;
// Waves side by side in a block-32 workgroup (each 32 rows x 128 columns).
#ifndef MXFP4_COL_WX
#define MXFP4_COL_WX 4
#endif
template <int B>
constexpr int col_threads() { return B == 32 ? 64 * MXFP4_COL_WX : 256; }

struct ColArgs {
  const uint8_t *x;
  uint8_t *y_col;
  uint32_t *mask_col;
  uint8_t *scales_col;
  uint8_t *y_row;
  uint32_t *mask_row;
  uint8_t *scales_row;
  const int64_t *group_list;
  int64_t rows, cols;
  int64_t nct;     // column tiles per block-row
  int64_t nw_row;  // row-bitmap words per row
  int64_t nb_row;  // row-wise blocks per row
  int num_groups, list_type;
  float sf;
};

template <int DT>
using ColT = PieceT<DT>;

template <int DT, bool VEC>
__device__ __forceinline__ void store_piece(uint8_t *p, const uint32_t *w, int n) {
  if (VEC) {
    if (n == 8) {
      st16(p, make_uint4(w[0], w[1], w[2], w[3]));
      if (DT == kF32) st16(p + 16, make_uint4(w[4], w[5], w[6], w[7]));
    }
    return;
  }
  for (int j = 0; j < n; ++j) {
    if (DT == kBF16) reinterpret_cast<uint16_t *>(p)[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    else reinterpret_cast<uint32_t *>(p)[j] = w[j];
  }
}

// Generic snap for the halves of a word whose column max is nonzero but has
// an exponent field below 5 (FLOOR E8M0 byte 0..2).
__device__ __forceinline__ void fix_slow_word(uint32_t w, uint32_t cm, uint32_t e8p, uint32_t *y,
                                           uint32_t *m) {
  const uint32_t lo = cm & 0xFFFFu, hi = cm >> 16;
  if (lo != 0 && (lo >> 7) < 5) {
    HalfOut o = half_bf16_slow(w & 0xFFFFu, e8p & 0xFFu);
    *y = (*y & 0xFFFF0000u) | o.y;
    *m = (*m & 0xFFFF0000u) | o.m;
  }
  if (hi != 0 && (hi >> 7) < 5) {
    HalfOut o = half_bf16_slow(w >> 16, (e8p >> 16) & 0xFFu);
    *y = (*y & 0xFFFFu) | (o.y << 16);
    *m = (*m & 0xFFFFu) | (o.m << 16);
  }
}

// One of four values by a lane-varying index, as register selects (an array
// indexed by a lane value would be placed in LDS by the compiler).
__device__ __forceinline__ uint32_t pick4(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                          int sel) {
  const uint32_t lo = (sel & 1) ? v1 : v0;
  const uint32_t hi = (sel & 1) ? v3 : v2;
  return (sel & 2) ? hi : lo;
}

// Column-direction outputs of one lane: y_col rows and the bitmap words of
// its columns.  SLOW = true only when some lane of the wave holds a column
// that needs the generic snap.
template <int DT, int RULE, bool VEC, bool SLOW>
__device__ __forceinline__ void col_outputs(const ColArgs &A, const uint32_t (&w)[8][ColT<DT>::NW],
                                            const uint32_t *pt, const uint32_t *ph, const uint32_t *ps,
                                            const uint32_t *pz, const uint32_t *pe, const uint32_t *cm,
                                            const BlockParams *cbp, int64_t off0, int64_t rstride,
                                            int rbase, int64_t len, int ncol, int rg, int64_t c0,
                                            int64_t wrow, bool slab_live) {
  constexpr int NW = ColT<DT>::NW;
    uint32_t acc[NW];  // clip bits of this lane's 8 rows (bf16: bit i / 16+i)
#pragma unroll
  for (int k = 0; k < NW; ++k) acc[k] = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t yv[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      if (DT == kBF16) {
        yv[k] = y_bf16(w[i][k], pt[k], ph[k], pz[k]);
        uint32_t mb = m_bf16(w[i][k], ps[k]);
        if (SLOW && RULE == kFloor) fix_slow_word(w[i][k], cm[k], pe[k], &yv[k], &mb);
        acc[k] |= mb << i;
      } else {
        yv[k] = y_f32(w[i][k], cbp[DT == kF32 ? k : 0]);
        acc[k] |= m_f32(w[i][k], cbp[DT == kF32 ? k : 0]) << i;
      }
    }
    if (A.y_col && rbase + i < len) store_piece<DT, VEC>(A.y_col + off0 + i * rstride, yv, ncol);
  }
  if (A.mask_col) {
    // column word = OR over the quad of (8-row byte << 8*rg); lane rg then
    // stores the words of its columns 2rg and 2rg+1
    uint32_t mw[8];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      if (DT == kBF16) {
        mw[2 * k] = or_quad((acc[k] & 0xFFu) << (8 * rg));
        mw[2 * k + 1] = or_quad(((acc[k] >> 16) & 0xFFu) << (8 * rg));
      } else {
        mw[k] = or_quad(acc[k] << (8 * rg));
      }
    }
    // every lane of the quad now holds the 8 words; lane rg == 0 writes them
    if (slab_live && rg == 0) {
      uint32_t *dst = A.mask_col + wrow * A.cols + c0;
      if (VEC) {
        if (ncol == 8) {
          *reinterpret_cast<uint4 *>(dst) = make_uint4(mw[0], mw[1], mw[2], mw[3]);
          *reinterpret_cast<uint4 *>(dst + 4) = make_uint4(mw[4], mw[5], mw[6], mw[7]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < ncol) dst[k] = mw[k];
      }
    }
  }
}

template <int DT, int B, int RULE, int KIND, bool VEC>
__global__ __launch_bounds__(col_threads<B>(), KIND == kKindDual      ? MXFP4_DUAL_MINWG
                                       : KIND == kKindGrouped ? MXFP4_GROUPED_MINWG
                                                              : MXFP4_COL_MINWG)
void col_fwd_kernel(ColArgs A) {
  constexpr int NW = ColT<DT>::NW;
  constexpr int ES = ColT<DT>::ES;
  constexpr int WX = B == 32 ? MXFP4_COL_WX : 1;  // waves side by side
  constexpr int G_ROW = B / 8;         // lanes per row-wise block (dual)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int rg = lane & 3;
  const int cc = lane >> 2;
  const int wx = B == 32 ? wave : 0;
  const int wy = B == 32 ? 0 : wave;

  const int64_t bt = blockIdx.x / A.nct;
  const int64_t ct = blockIdx.x - bt * A.nct;

  int64_t start, len;
  if (KIND == kKindGrouped) {
    block_row_uniform(A.group_list, A.num_groups, A.list_type, A.rows, B == 32 ? 5 : 7, bt, &start,
                      &len);
    if (len <= 0) return;  // every wave of the workgroup decodes the same block-row
  } else {
    start = bt * B;
    len = A.rows - start < B ? A.rows - start : B;
  }

  const int64_t col0 = ct * (kWaveCols * WX) + kWaveCols * wx;
  const int64_t c0 = col0 + 8 * cc;
  const int64_t crem = A.cols - c0;
  const int ncol = crem >= 8 ? 8 : (crem > 0 ? (int)crem : 0);
  const int slab = 32 * wy;
  const int rbase = slab + 8 * rg;            // first row of this lane in the block-row
  const int64_t rstride = A.cols * ES;        // bytes per row
  const int64_t off0 = ((start + rbase) * A.cols + c0) * ES;

  // ---- load 8 rows x 8 columns per lane ---------------------------------
  // A wave whose 32 rows and 128 columns are all inside the tensor issues its
  // eight loads unconditionally, so all of them are in flight together (a
  // load under a per-lane branch is waited for before the branch closes).
  uint32_t w[8][NW];
  const bool full = VEC && slab + 32 <= len && col0 + kWaveCols <= A.cols;  // wave-uniform
  if (full) {
#pragma unroll
    for (int i = 0; i < 8; ++i) load_piece<DT, true>(w[i], A.x + off0 + i * rstride, 8);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = rbase + i < len ? ncol : 0;
      load_piece<DT, VEC>(w[i], A.x + off0 + i * rstride, n);
    }
  }

  // ---- column direction ---------------------------------------------------
  // column maxima: bf16 packed per word (2 columns), fp32 one per word
  uint32_t cm[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (DT == kBF16) m = pk_max(m, w[i][k] & 0x7FFF7FFFu);
      else m = max32(m, w[i][k] & 0x7FFFFFFFu);
    }
    cm[k] = DT == kBF16 ? pkmax_quad(m) : max_quad(m);
  }
  if (B == 128) {
    __shared__ uint32_t s_cm[4][16][NW];
    if (rg == 0) {
#pragma unroll
      for (int k = 0; k < NW; ++k) s_cm[wave][cc][k] = cm[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      uint32_t m = s_cm[0][cc][k];
#pragma unroll
      for (int v = 1; v < 4; ++v) m = DT == kBF16 ? pk_max(m, s_cm[v][cc][k]) : max32(m, s_cm[v][cc][k]);
      cm[k] = m;
    }
  }

  // per-column parameters: bf16 packed per word (E8M0 bytes in bits 0-7 and
  // 16-23), fp32 one block per column
  uint32_t pt[NW], ph[NW], ps[NW], pz[NW], pe[NW];
  bool slow_any = false;
  BlockParams cbp[DT == kF32 ? 8 : 1];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (DT == kBF16 && RULE == kFloor) {
      const PackedParams q = floor_params_pk(cm[k]);
      pt[k] = q.t2; ph[k] = q.h2; ps[k] = q.s2; pz[k] = 0x7FFF7FFFu; pe[k] = q.e8;
      slow_any = slow_any || q.slow;
    } else if (DT == kBF16) {
      const BlockParams lo = block_params<DT, RULE>(cm[k] & 0xFFFFu, A.sf);
      const BlockParams hi = block_params<DT, RULE>(cm[k] >> 16, A.sf);
      pt[k] = lo.t025 | (hi.t025 << 16);
      ph[k] = lo.half | (hi.half << 16);
      ps[k] = lo.six | (hi.six << 16);
      pz[k] = lo.zc | (hi.zc << 16);
      pe[k] = lo.e8 | (hi.e8 << 16);
    } else {
      cbp[DT == kF32 ? k : 0] = block_params<DT, RULE>(cm[k], A.sf);
      pe[k] = cbp[DT == kF32 ? k : 0].e8;
    }
  }

  const bool slab_live = KIND == kKindGrouped ? true : (slab < len);
  const int64_t wrow = bt * (B / 32) + wy;  // bitmap word-row of this slab

  if (A.y_col || A.mask_col) {
    if (__builtin_expect(__any(slow_any), 0))
      col_outputs<DT, RULE, VEC, true>(A, w, pt, ph, ps, pz, pe, cm, cbp, off0, rstride, rbase, len, ncol,
                                       rg, c0, wrow, slab_live);
    else
      col_outputs<DT, RULE, VEC, false>(A, w, pt, ph, ps, pz, pe, cm, cbp, off0, rstride, rbase, len, ncol,
                                        rg, c0, wrow, slab_live);
  }
  if (A.scales_col && rg == 0 && wy == 0) {
    uint8_t *dst = A.scales_col + bt * A.cols + c0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      if (DT == kBF16) {
        if (2 * k < ncol) dst[2 * k] = (uint8_t)(pe[k] & 0xFFu);
        if (2 * k + 1 < ncol) dst[2 * k + 1] = (uint8_t)((pe[k] >> 16) & 0xFFu);
      } else {
        if (k < ncol) dst[k] = (uint8_t)pe[k];
      }
    }
  }

  // ---- row direction (dual) ----------------------------------------------
  if (KIND == kKindDual) {
    uint32_t rw[8];  // row-bitmap partial words
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = rbase + i;
      uint32_t am;
      if (DT == kBF16) {
        uint32_t m = pk_max(pk_max(w[i][0] & 0x7FFF7FFFu, w[i][1] & 0x7FFF7FFFu),
                            pk_max(w[i][2] & 0x7FFF7FFFu, w[i][3] & 0x7FFF7FFFu));
        am = max32(m & 0xFFFFu, m >> 16);
      } else {
        am = 0;
#pragma unroll
        for (int k = 0; k < NW; ++k) am = max32(am, w[i][k] & 0x7FFFFFFFu);
      }
      am = B == 32 ? max_stride4_row(am) : max_stride4_wave(am);
      const BlockParams bp = block_params<DT, RULE>(am, A.sf);
      const bool rslow = __builtin_expect(__any(bp.slow), 0);
      if (A.y_row) {
        uint32_t yv[NW];
        if (rslow) chunk_y<DT, true>(w[i], bp, yv);
        else chunk_y<DT, false>(w[i], bp, yv);
        if (rr < len) store_piece<DT, VEC>(A.y_row + off0 + i * rstride, yv, ncol);
      }
      uint32_t mbyte = 0;
      if (A.mask_row) mbyte = rslow ? chunk_mask<DT, true>(w[i], bp) : chunk_mask<DT, false>(w[i], bp);
      rw[i] = A.mask_row ? or_stride4_row(mbyte << (8 * (cc & 3))) : 0;
      if (A.scales_row && (cc % G_ROW) == 0 && rr < len && ncol > 0)
        A.scales_row[(start + rr) * A.nb_row + c0 / B] = (uint8_t)bp.e8;
    }
    if (A.mask_row) {
      // the 4 lanes of a 32-column word hold all 8 rows' words: lane j stores
      // rows j and j + 4
      const int j = cc & 3;
      const int64_t wi = c0 >> 5;
      const uint32_t lo = pick4(rw[0], rw[1], rw[2], rw[3], j);
      const uint32_t hi = pick4(rw[4], rw[5], rw[6], rw[7], j);
      const int r_lo = rbase + j, r_hi = r_lo + 4;
      if (wi < A.nw_row) {
        if (r_lo < len) A.mask_row[(start + r_lo) * A.nw_row + wi] = lo;
        if (r_hi < len) A.mask_row[(start + r_hi) * A.nw_row + wi] = hi;
      }
    }
  }
}

template <int DT, int B, int RULE, int KIND>
hipError_t launch_kind(bool vec, const ColArgs &a, dim3 grid, hipStream_t st) {
  if (vec) hipLaunchKernelGGL((col_fwd_kernel<DT, B, RULE, KIND, true>), grid, dim3(col_threads<B>()), 0, st, a);
  else hipLaunchKernelGGL((col_fwd_kernel<DT, B, RULE, KIND, false>), grid, dim3(col_threads<B>()), 0, st, a);
  return hipGetLastError();
}

template <int DT, int B, int RULE>
hipError_t launch_rule(int kind, bool vec, const ColArgs &a, dim3 grid, hipStream_t st) {
  switch (kind) {
    case kKindCol: return launch_kind<DT, B, RULE, kKindCol>(vec, a, grid, st);
    case kKindDual: return launch_kind<DT, B, RULE, kKindDual>(vec, a, grid, st);
    default: return launch_kind<DT, B, RULE, kKindGrouped>(vec, a, grid, st);
  }
}

template <int DT, int B>
hipError_t launch_b(int rule, int kind, bool vec, const ColArgs &a, dim3 grid, hipStream_t st) {
  return rule == kFloor ? launch_rule<DT, B, kFloor>(kind, vec, a, grid, st)
                        : launch_rule<DT, B, kAmct>(kind, vec, a, grid, st);
}

}  // namespace

hipError_t launch_col_fwd(const ColLaunch &L, hipStream_t st) {
  ColArgs a;
  a.x = static_cast<const uint8_t *>(L.x);
  a.y_col = static_cast<uint8_t *>(L.y_col);
  a.mask_col = L.mask_col;
  a.scales_col = L.scales_col;
  a.y_row = static_cast<uint8_t *>(L.y_row);
  a.mask_row = L.mask_row;
  a.scales_row = L.scales_row;
  a.group_list = L.group_list;
  a.rows = L.rows;
  a.cols = L.cols;
  const int64_t tile_cols = L.block == 32 ? MXFP4_COL_WX * kWaveCols : kWaveCols;
  a.nct = (L.cols + tile_cols - 1) / tile_cols;
  a.nw_row = (L.cols + 31) / 32;
  a.nb_row = (L.cols + L.block - 1) / L.block;
  a.num_groups = L.num_groups;
  a.list_type = L.list_type;
  a.sf = L.sf;
  const bool grouped = L.group_list != nullptr;
  const bool dual = !grouped && (L.y_row || L.mask_row || L.scales_row);
  const int kind = grouped ? kKindGrouped : (dual ? kKindDual : kKindCol);
  const int64_t nbr = grouped ? (L.rows + L.block - 1) / L.block + L.num_groups
                              : (L.rows + L.block - 1) / L.block;
  const int64_t nwg = nbr * a.nct;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool vec = L.cols % 8 == 0;
  dim3 grid((unsigned)nwg);
  if (L.dtype == kBF16)
    return L.block == 32 ? launch_b<kBF16, 32>(L.rule, kind, vec, a, grid, st)
                         : launch_b<kBF16, 128>(L.rule, kind, vec, a, grid, st);
  return L.block == 32 ? launch_b<kF32, 32>(L.rule, kind, vec, a, grid, st)
                       : launch_b<kF32, 128>(L.rule, kind, vec, a, grid, st);
}

}  // namespace mxfp4
