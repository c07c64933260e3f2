// ste_kernels.hip -- straight-through-estimator backward on gfx950.
//
// _MXFP4FakeQuantSTE.backward of the amct PR: the clipped STE returns
// grad_output.masked_fill(saturated, 0.0); the plain STE returns grad_output
// unchanged.  Here the saturation mask is the bitmap the forward wrote, so the
// backward is one streaming pass: read g (16 B per lane-piece) and the mask
// bits, write +0.0 where a bit is set and g elsewhere.
//   ROW bitmaps: one mask byte per 8-element piece, same chunk walk as the
//     row-wise forward.
//   COL / GROUPED bitmaps: 32-row slabs; a lane loads the 8 words of its 8
//     columns once and serves its 8 rows from them.
#include "mxfp4_device.h"
#include "mxfp4_groups.h"
#include "mxfp4_kernels.h"

namespace mxfp4 {
namespace {

// Pieces per thread and workgroup size (measured on MI355X): one piece per
// thread in one-wave workgroups streams both the 4096x4096 and the
// 28672x8192 gradient best; short workgroups keep loads and stores
// overlapped across waves.
#ifndef MXFP4_STE_U_SMALL
#define MXFP4_STE_U_SMALL 1
#endif
#ifndef MXFP4_STE_U_BIG
#define MXFP4_STE_U_BIG 1
#endif
constexpr int64_t kSteBigChunks = int64_t(8) << 20;
#ifndef MXFP4_STE_THREADS
#define MXFP4_STE_THREADS 64
#endif
constexpr int kSteThreads = MXFP4_STE_THREADS;  // threads per workgroup (row walk)
enum { kModeFlat = 0, kModeRowsVec = 1, kModeRowsScalar = 2 };

// Clear the elements whose bit is set.  bf16 word k holds elements 2k, 2k+1
// (bits 2k, 2k+1 of `bits`); fp32 word k holds element k.
template <int DT>
__device__ __forceinline__ void apply_bits(uint32_t *w, uint32_t bits) {
  if (DT == kBF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 2 * k, 1);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 2 * k + 1, 1);
      const uint32_t sel = (lo & 0xFFFFu) | (hi & 0xFFFF0000u);
      w[k] &= ~sel;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] &= ~(uint32_t)__builtin_amdgcn_sbfe((int)bits, k, 1);
  }
}

struct SteRowArgs {
  const uint8_t *g;
  uint8_t *gi;
  const uint8_t *mask;  // NULL: plain STE
  int64_t cols, nchunks, cpr, mask_row_bytes;
};

template <int DT, int MODE, int U, bool FULL>
__device__ __forceinline__ void ste_row_body(const SteRowArgs &A, int64_t wg) {
  constexpr int NW = DT == kBF16 ? 4 : 8;
  constexpr int ES = DT == kBF16 ? 2 : 4;
  const int tid = threadIdx.x;
  const int64_t base = wg * (kSteThreads * U);
  uint32_t w[U][NW];
  uint32_t bits[U];
  int64_t off[U];
  int nval[U];
#pragma unroll
  for (int s = 0; s < U; ++s) {
    const int64_t i = base + s * kSteThreads + tid;
    int64_t mb;
    if (MODE == kModeFlat) {
      off[s] = i * 8;
      nval[s] = (FULL || i < A.nchunks) ? 8 : 0;
      mb = i;
    } else {
      const int64_t r = i / A.cpr, c = i - r * A.cpr;
      off[s] = r * A.cols + c * 8;
      const int64_t rem = A.cols - c * 8;
      nval[s] = i < A.nchunks ? (int)(rem >= 8 ? 8 : (rem > 0 ? rem : 0)) : 0;
      mb = r * A.mask_row_bytes + c;
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) w[s][k] = 0;
    bits[s] = 0;
    if (FULL || nval[s] > 0) {
      const uint8_t *p = A.g + off[s] * ES;
      if (MODE != kModeRowsScalar) {
        uint4 v = ld16(p);
        w[s][0] = v.x; w[s][1] = v.y; w[s][2] = v.z; w[s][3] = v.w;
        if (DT == kF32) {
          uint4 v2 = ld16(p + 16);
          w[s][4] = v2.x; w[s][5] = v2.y; w[s][6] = v2.z; w[s][7] = v2.w;
        }
      } else {
        for (int j = 0; j < nval[s]; ++j) {
          if (DT == kBF16) w[s][j >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(p)[j] << (16 * (j & 1));
          else w[s][j] = reinterpret_cast<const uint32_t *>(p)[j];
        }
      }
      if (A.mask) bits[s] = A.mask[mb];
    }
  }
#pragma unroll
  for (int s = 0; s < U; ++s) {
    if (!FULL && nval[s] == 0) continue;
    apply_bits<DT>(w[s], bits[s]);
    uint8_t *p = A.gi + off[s] * ES;
    if (MODE != kModeRowsScalar) {
      st16(p, make_uint4(w[s][0], w[s][1], w[s][2], w[s][3]));
      if (DT == kF32) st16(p + 16, make_uint4(w[s][4], w[s][5], w[s][6], w[s][7]));
    } else {
      for (int j = 0; j < nval[s]; ++j) {
        if (DT == kBF16) reinterpret_cast<uint16_t *>(p)[j] = (uint16_t)(w[s][j >> 1] >> (16 * (j & 1)));
        else reinterpret_cast<uint32_t *>(p)[j] = w[s][j];
      }
    }
  }
}

// Workgroups whose pieces are all in range (flat layout) load unconditionally.
template <int DT, int MODE, int U>
__global__ __launch_bounds__(kSteThreads) void ste_row_kernel(SteRowArgs A) {
  if (MODE == kModeFlat && (int64_t)(blockIdx.x + 1) * (kSteThreads * U) <= A.nchunks)
    ste_row_body<DT, MODE, U, true>(A, blockIdx.x);
  else
    ste_row_body<DT, MODE, U, false>(A, blockIdx.x);
}

// Several gradients in one launch: tensor j owns workgroups [wg0[j],
// wg0[j + 1]), one piece per lane, in its own layout mode.
struct SteBatchArgs {
  SteRowArgs item[kBatchMax];
  int64_t wg0[kBatchMax + 1];
  int mode[kBatchMax];
  int n;
};

template <int DT>
__global__ __launch_bounds__(kSteThreads) void ste_row_batch_kernel(SteBatchArgs P) {
  const int64_t w = blockIdx.x;
  int j = 0;
  while (j + 1 < P.n && w >= P.wg0[j + 1]) ++j;
  const SteRowArgs &A = P.item[j];
  const int64_t wg = w - P.wg0[j];
  switch (P.mode[j]) {
    case kModeFlat:
      if ((wg + 1) * kSteThreads <= A.nchunks) ste_row_body<DT, kModeFlat, 1, true>(A, wg);
      else ste_row_body<DT, kModeFlat, 1, false>(A, wg);
      break;
    case kModeRowsVec: ste_row_body<DT, kModeRowsVec, 1, false>(A, wg); break;
    default: ste_row_body<DT, kModeRowsScalar, 1, false>(A, wg); break;
  }
}

struct SteColArgs {
  const uint8_t *g;
  uint8_t *gi;
  const uint32_t *mask;
  const int64_t *group_list;
  int64_t rows, cols, nct;
  int num_groups, list_type, block_log2;
};

// One workgroup = one 32-row slab x 512 columns (4 waves side by side).
template <int DT, bool GROUPED, bool VEC>
__global__ __launch_bounds__(kThreads) void ste_col_kernel(SteColArgs A) {
  constexpr int NW = DT == kBF16 ? 4 : 8;
  constexpr int ES = DT == kBF16 ? 2 : 4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = lane & 3, cc = lane >> 2;
  const int64_t ts = blockIdx.x / A.nct;
  const int64_t ct = blockIdx.x - ts * A.nct;
  int64_t start, len;
  if (GROUPED) {
    const int sub_log2 = A.block_log2 - 5;  // 32-row slabs per block-row (log2)
    const int64_t t = ts >> sub_log2;
    const int64_t q = ts - (t << sub_log2);
    int64_t bstart, blen;
    block_row_uniform(A.group_list, A.num_groups, A.list_type, A.rows, A.block_log2, t, &bstart,
                      &blen);
    start = bstart + 32 * q;
    len = blen - 32 * q;
    if (len <= 0) return;
    if (len > 32) len = 32;
  } else {
    start = 32 * ts;
    len = A.rows - start < 32 ? A.rows - start : 32;
  }
  const int64_t c0 = ct * 512 + 128 * wave + 8 * cc;
  const int64_t crem = A.cols - c0;
  const int ncol = crem >= 8 ? 8 : (crem > 0 ? (int)crem : 0);
  if (ncol == 0) return;  // no barrier follows

  // the 8 bitmap words of this lane's columns
  uint32_t mw[8];
  const uint32_t *mp = A.mask + ts * A.cols + c0;
  if (VEC) {
    uint4 a = *reinterpret_cast<const uint4 *>(mp);
    uint4 b = *reinterpret_cast<const uint4 *>(mp + 4);
    mw[0] = a.x; mw[1] = a.y; mw[2] = a.z; mw[3] = a.w;
    mw[4] = b.x; mw[5] = b.y; mw[6] = b.z; mw[7] = b.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) mw[k] = k < ncol ? mp[k] : 0;
  }
  if (VEC && len == 32 && ncol == 8 && c0 - 8 * cc + 128 <= A.cols) {
    // full slab for this wave: all loads first, no per-lane branches
    const int64_t rstride = A.cols * ES;
    const uint8_t *p0 = A.g + ((start + 8 * rg) * A.cols + c0) * ES;
    uint8_t *q0 = A.gi + ((start + 8 * rg) * A.cols + c0) * ES;
    uint32_t w[8][NW];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint4 v = ld16(p0 + i * rstride);
      w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
      if (DT == kF32) {
        uint4 v2 = ld16(p0 + i * rstride + 16);
        w[i][4] = v2.x; w[i][5] = v2.y; w[i][6] = v2.z; w[i][7] = v2.w;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = 8 * rg + i;
      uint32_t bits = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) bits |= ((mw[k] >> rr) & 1u) << k;
      apply_bits<DT>(w[i], bits);
      st16(q0 + i * rstride, make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]));
      if (DT == kF32) st16(q0 + i * rstride + 16, make_uint4(w[i][4], w[i][5], w[i][6], w[i][7]));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rr = 8 * rg + i;
    if (rr >= len) continue;
    const uint8_t *p = A.g + ((start + rr) * A.cols + c0) * ES;
    uint8_t *q = A.gi + ((start + rr) * A.cols + c0) * ES;
    uint32_t w[NW];
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) bits |= ((mw[k] >> rr) & 1u) << k;
    if (VEC) {
      uint4 v = ld16(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      if (DT == kF32) {
        uint4 v2 = ld16(p + 16);
        w[4] = v2.x; w[5] = v2.y; w[6] = v2.z; w[7] = v2.w;
      }
      apply_bits<DT>(w, bits);
      st16(q, make_uint4(w[0], w[1], w[2], w[3]));
      if (DT == kF32) st16(q + 16, make_uint4(w[4], w[5], w[6], w[7]));
    } else {
      for (int j = 0; j < ncol; ++j) {
        uint32_t e = DT == kBF16 ? reinterpret_cast<const uint16_t *>(p)[j] : reinterpret_cast<const uint32_t *>(p)[j];
        if ((bits >> j) & 1u) e = 0;
        if (DT == kBF16) reinterpret_cast<uint16_t *>(q)[j] = (uint16_t)e;
        else reinterpret_cast<uint32_t *>(q)[j] = e;
      }
    }
  }
}

template <int DT, int U>
void ste_row_launch(int mode, dim3 grid, const SteRowArgs &a, hipStream_t st) {
  switch (mode) {
    case kModeFlat: hipLaunchKernelGGL((ste_row_kernel<DT, kModeFlat, U>), grid, dim3(kSteThreads), 0, st, a); break;
    case kModeRowsVec: hipLaunchKernelGGL((ste_row_kernel<DT, kModeRowsVec, U>), grid, dim3(kSteThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((ste_row_kernel<DT, kModeRowsScalar, U>), grid, dim3(kSteThreads), 0, st, a); break;
  }
}

// Kernel arguments and layout mode of one gradient (ROW bitmap or none).
int ste_row_args(const SteLaunch &L, SteRowArgs &a) {
  a.g = static_cast<const uint8_t *>(L.g);
  a.gi = static_cast<uint8_t *>(L.g_in);
  a.mask = reinterpret_cast<const uint8_t *>(L.mask);
  a.cols = L.cols;
  a.cpr = (L.cols + 7) / 8;
  a.mask_row_bytes = 4 * ((L.cols + 31) / 32);
  if (L.cols % 32 == 0) {
    a.nchunks = L.rows * L.cols / 8;
    return kModeFlat;
  }
  a.nchunks = L.rows * a.cpr;
  return L.cols % 8 == 0 ? kModeRowsVec : kModeRowsScalar;
}

template <int DT>
hipError_t launch_row(const SteLaunch &L, hipStream_t st) {
  SteRowArgs a;
  const int mode = ste_row_args(L, a);
  const int u = a.nchunks > kSteBigChunks ? MXFP4_STE_U_BIG : MXFP4_STE_U_SMALL;
  const int64_t per = (int64_t)kSteThreads * u;
  const int64_t nwg = (a.nchunks + per - 1) / per;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  switch (u) {
    case 1: ste_row_launch<DT, 1>(mode, grid, a, st); break;
    case 2: ste_row_launch<DT, 2>(mode, grid, a, st); break;
    case 4: ste_row_launch<DT, 4>(mode, grid, a, st); break;
    case 8: ste_row_launch<DT, 8>(mode, grid, a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_col(const SteLaunch &L, hipStream_t st) {
  SteColArgs a;
  a.g = static_cast<const uint8_t *>(L.g);
  a.gi = static_cast<uint8_t *>(L.g_in);
  a.mask = L.mask;
  a.group_list = L.group_list;
  a.rows = L.rows;
  a.cols = L.cols;
  a.nct = (L.cols + 511) / 512;
  a.num_groups = L.num_groups;
  a.list_type = L.list_type;
  a.block_log2 = L.block == 32 ? 5 : 7;
  const bool grouped = L.layout == 4;
  int64_t slabs = (L.rows + 31) / 32;
  if (grouped) slabs = ((L.rows + L.block - 1) / L.block + L.num_groups) * (L.block / 32);
  const int64_t nwg = slabs * a.nct;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  const bool vec = L.cols % 8 == 0;
  if (grouped) {
    if (vec) hipLaunchKernelGGL((ste_col_kernel<DT, true, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((ste_col_kernel<DT, true, false>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((ste_col_kernel<DT, false, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((ste_col_kernel<DT, false, false>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

// Saturation bitmap (ROW or COL layout) -> one byte per element, 1 where
// the bit is set and 0 elsewhere, in x's row-major order: the pages' bool
// mask.  A lane writes 16 consecutive bytes of the flat output (one 16-byte
// store when the output is 16-byte aligned and the 16 bytes are in range).
constexpr int kBoolThreads = 256;

template <int LAYOUT>
__global__ void __launch_bounds__(kBoolThreads)
    mask_bool_kernel(const uint32_t *__restrict__ mask, uint8_t *__restrict__ out, int64_t cols,
                     int64_t words_per_row, int64_t n, bool vec) {
  const int64_t f0 = ((int64_t)blockIdx.x * kBoolThreads + threadIdx.x) * 16;
  if (f0 >= n) return;
  int64_t r = f0 / cols, c = f0 - r * cols;
  const int64_t left = n - f0;
  uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < left) {
      const uint32_t w = LAYOUT == 1 ? mask[r * words_per_row + (c >> 5)] : mask[(r >> 5) * cols + c];
      const uint32_t bit = (w >> (LAYOUT == 1 ? (c & 31) : (r & 31))) & 1u;
      b[j >> 2] |= bit << (8 * (j & 3));
      if (++c == cols) {
        c = 0;
        ++r;
      }
    }
  }
  if (vec && left >= 16) {
    const u32x4 v = {b[0], b[1], b[2], b[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out + f0));
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < left) out[f0 + j] = (uint8_t)(b[j >> 2] >> (8 * (j & 3)));
  }
}

}  // namespace

hipError_t launch_ste_bwd(const SteLaunch &L, hipStream_t st) {
  // plain STE and ROW bitmaps share the chunk walk (mask NULL = copy)
  if (L.mask == nullptr || L.layout == 1)
    return L.dtype == kBF16 ? launch_row<kBF16>(L, st) : launch_row<kF32>(L, st);
  return L.dtype == kBF16 ? launch_col<kBF16>(L, st) : launch_col<kF32>(L, st);
}

hipError_t launch_mask_bool(int layout, int64_t rows, int64_t cols, const uint32_t *mask, uint8_t *out,
                            hipStream_t st) {
  const int64_t n = rows * cols;
  const int64_t nwg = (n + 16 * kBoolThreads - 1) / (16 * kBoolThreads);
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool vec = (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const int64_t wpr = (cols + 31) / 32;
  if (layout == 1)
    hipLaunchKernelGGL((mask_bool_kernel<1>), dim3((unsigned)nwg), dim3(kBoolThreads), 0, st, mask, out, cols, wpr,
                       n, vec);
  else
    hipLaunchKernelGGL((mask_bool_kernel<2>), dim3((unsigned)nwg), dim3(kBoolThreads), 0, st, mask, out, cols, wpr,
                       n, vec);
  return hipGetLastError();
}

hipError_t launch_ste_row_batch(const SteLaunch *L, int n, hipStream_t st) {
  if (n < 1 || n > kBatchMax) return hipErrorInvalidValue;
  SteBatchArgs p{};
  p.n = n;
  int64_t wg = 0;
  for (int j = 0; j < n; ++j) {
    p.mode[j] = ste_row_args(L[j], p.item[j]);
    p.wg0[j] = wg;
    wg += (p.item[j].nchunks + kSteThreads - 1) / kSteThreads;
  }
  for (int j = n; j <= kBatchMax; ++j) p.wg0[j] = wg;
  if (wg == 0) return hipSuccess;
  if (wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wg);
  if (L[0].dtype == kBF16)
    hipLaunchKernelGGL(ste_row_batch_kernel<kBF16>, grid, dim3(kSteThreads), 0, st, p);
  else
    hipLaunchKernelGGL(ste_row_batch_kernel<kF32>, grid, dim3(kSteThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxfp4
