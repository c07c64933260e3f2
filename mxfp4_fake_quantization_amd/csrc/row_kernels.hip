// row_kernels.hip -- row-wise MXFP4 fake quantization on gfx950.
//
// Blocks of 32 or 128 consecutive elements along each row (the pages'
// last-dim blocking, fake_quant.py _block_view; a row's last block is short
// when cols % block != 0 and blocks never straddle rows).  One pass reads x
// once and emits any of: the dequantized values y, the clipped-STE bitmap,
// the E8M0 scale bytes, and the packed E2M1 nibbles (two per byte).
//
// Work split: a "chunk" is 8 consecutive elements of one row (16 bytes of
// bf16, 32 bytes of fp32) held by one lane; a block is 4 (block 32) or 16
// (block 128) consecutive lanes, reduced with DPP.  Each thread issues all of
// its U (1, 2 or 4) chunk loads before any arithmetic, and consecutive lanes
// read consecutive 16-byte pieces, so every load instruction covers one
// contiguous 1 KiB (bf16) stretch of HBM.
#include "mxfp4_device.h"
#include "mxfp4_kernels.h"

namespace mxfp4 {
namespace {

// Chunks per thread and workgroup size, measured on MI355X at 4096x4096 and
// 28672x8192: the y / bitmap forward streams best with one chunk per thread
// in one-wave workgroups (many short workgroups keep loads and stores
// overlapped across waves); the packing forward with two chunks per thread
// (four for bf16 block 128: 103 -> 99 us at 28672x8192; an fp32 chunk is
// already 32 bytes) in four-wave workgroups.
#ifndef MXFP4_ROW_U_SMALL
#define MXFP4_ROW_U_SMALL 1
#endif
#ifndef MXFP4_ROW_U_BIG
#define MXFP4_ROW_U_BIG 1
#endif
#ifndef MXFP4_PACK_U
#define MXFP4_PACK_U 2
#endif
#ifndef MXFP4_PACK_U_B128
#define MXFP4_PACK_U_B128 4
#endif
constexpr int64_t kRowBigChunks = int64_t(8) << 20;
#ifndef MXFP4_ROW_THREADS
#define MXFP4_ROW_THREADS 64
#endif
#ifndef MXFP4_PACK_THREADS
#define MXFP4_PACK_THREADS 256
#endif
constexpr int kRowThreads = MXFP4_ROW_THREADS;    // threads per workgroup, y / bitmap
constexpr int kPackThreads = MXFP4_PACK_THREADS;  // threads per workgroup, packed codes

enum { kModeFlat = 0, kModeRowsVec = 1, kModeRowsScalar = 2 };

struct RowArgs {
  const uint8_t *x;
  uint8_t *y;
  uint8_t *mask;    // bitmap as bytes: byte (r, j) holds columns 8j..8j+7
  uint8_t *scales;
  uint8_t *codes;
  int64_t cols;
  int64_t nchunks;  // chunks in the launch (a multiple of the group size)
  int64_t cpr;      // chunks per row, padded to whole blocks (row modes)
  int64_t nb;       // blocks per row
  int64_t mask_row_bytes;  // 4 * ceil(cols / 32)
  int64_t code_row_bytes;  // ceil(cols / 2)
  float sf;
  uint32_t emit;
};

template <int DT>
struct ChunkT {
  static constexpr int NW = DT == kBF16 ? 4 : 8;  // 32-bit words per chunk
  static constexpr int ES = DT == kBF16 ? 2 : 4;  // element bytes
};

template <int DT>
__device__ __forceinline__ void load_vec(uint32_t *w, const uint8_t *p) {
  uint4 v = ld16(p);
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  if (DT == kF32) {
    uint4 v2 = ld16(p + 16);
    w[4] = v2.x; w[5] = v2.y; w[6] = v2.z; w[7] = v2.w;
  }
}

template <int DT>
__device__ __forceinline__ void store_vec(uint8_t *p, const uint32_t *w) {
  st16(p, make_uint4(w[0], w[1], w[2], w[3]));
  if (DT == kF32) st16(p + 16, make_uint4(w[4], w[5], w[6], w[7]));
}

template <int DT>
__device__ __forceinline__ void load_scalar(uint32_t *w, const uint8_t *p, int n) {
  constexpr int NW = ChunkT<DT>::NW;
#pragma unroll
  for (int k = 0; k < NW; ++k) w[k] = 0;
  for (int j = 0; j < n; ++j) {
    if (DT == kBF16) w[j >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(p)[j] << (16 * (j & 1));
    else w[j] = reinterpret_cast<const uint32_t *>(p)[j];
  }
}

template <int DT>
__device__ __forceinline__ void store_scalar(uint8_t *p, const uint32_t *w, int n) {
  for (int j = 0; j < n; ++j) {
    if (DT == kBF16) reinterpret_cast<uint16_t *>(p)[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    else reinterpret_cast<uint32_t *>(p)[j] = w[j];
  }
}

// Outputs of one chunk: y, bitmap byte, packed nibbles (scales are written by
// the caller).  SLOW selects the variant that can handle generic-snap blocks.
template <int DT, int G, int MODE, int U, bool FULL, bool SLOW>
__device__ __forceinline__ void row_emit(const RowArgs &A, const uint32_t *wv, const BlockParams &bp,
                                         int64_t off, int64_t row, int64_t cr, int nval, int64_t idx) {
  constexpr int NW = ChunkT<DT>::NW;
  constexpr int ES = ChunkT<DT>::ES;
  const uint32_t emit = A.emit;
    const bool live = nval > 0;
    if (emit & kEmitY) {
      uint32_t yv[NW];
      chunk_y<DT, SLOW>(wv, bp, yv);
      uint8_t *dst = A.y + off * ES;
      if (MODE == kModeRowsScalar) {
        if (live) store_scalar<DT>(dst, yv, nval);
      } else if (nval == 8) {
        store_vec<DT>(dst, yv);
      }
    }
    if (emit & kEmitMask) {
      const uint32_t byte = chunk_mask<DT, SLOW>(wv, bp);
      if (MODE == kModeFlat) {
        if (live) st_small(A.mask + cr, (uint8_t)byte);
      } else if (idx < A.nchunks && cr < A.mask_row_bytes) {
        st_small(A.mask + row * A.mask_row_bytes + cr, (uint8_t)byte);
      }
    }
    if (emit & kEmitCodes) {
      const uint32_t nib = chunk_codes<DT, SLOW>(wv, bp);
      if (MODE == kModeFlat) {
        if (live) st_small(reinterpret_cast<uint32_t *>(A.codes) + cr, nib);
      } else if (MODE == kModeRowsVec) {
        if (nval == 8)
          st_small(reinterpret_cast<uint32_t *>(A.codes + row * A.code_row_bytes + 4 * cr), nib);
      } else if (live) {
        uint8_t *dst = A.codes + row * A.code_row_bytes + 4 * cr;
        for (int j = 0; j < (nval + 1) / 2; ++j) dst[j] = (uint8_t)(nib >> (8 * j));
      }
    }
}

template <int DT, int B, int RULE, int MODE, int U, int T, bool FULL>
__device__ __forceinline__ void row_fwd_body(const RowArgs &A, int64_t wg) {
  constexpr int G = B / 8;
  constexpr int NW = ChunkT<DT>::NW;
  constexpr int ES = ChunkT<DT>::ES;
  const int tid = threadIdx.x;
  const int64_t base = wg * (T * U);

  uint32_t w[U][NW];
  int64_t off[U], row[U], cr[U];
  int nval[U];
#pragma unroll
  for (int s = 0; s < U; ++s) {
    const int64_t i = base + s * T + tid;
    if (MODE == kModeFlat) {
      row[s] = 0;
      cr[s] = i;
      off[s] = i * 8;
      nval[s] = (FULL || i < A.nchunks) ? 8 : 0;
    } else {
      const int64_t r = i / A.cpr;
      const int64_t c = i - r * A.cpr;
      row[s] = r;
      cr[s] = c;
      off[s] = r * A.cols + c * 8;
      const int64_t rem = A.cols - c * 8;
      nval[s] = i < A.nchunks ? (int)(rem >= 8 ? 8 : (rem > 0 ? rem : 0)) : 0;
    }
    if (MODE == kModeRowsScalar) {
      load_scalar<DT>(w[s], A.x + off[s] * ES, nval[s]);
    } else if (FULL || nval[s] == 8) {
      load_vec<DT>(w[s], A.x + off[s] * ES);
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) w[s][k] = 0;
    }
  }

#pragma unroll
  for (int s = 0; s < U; ++s) {
    // block max of the magnitude bits (integer max == float max for finite x)
    uint32_t am;
    if (DT == kBF16) {
      uint32_t m = pk_max(pk_max(w[s][0] & 0x7FFF7FFFu, w[s][1] & 0x7FFF7FFFu),
                          pk_max(w[s][2] & 0x7FFF7FFFu, w[s][3] & 0x7FFF7FFFu));
      am = max32(m & 0xFFFFu, m >> 16);
    } else {
      am = 0;
#pragma unroll
      for (int k = 0; k < NW; ++k) am = max32(am, w[s][k] & 0x7FFFFFFFu);
    }
    am = group_max<G>(am);
    const BlockParams bp = block_params<DT, RULE>(am, A.sf);

    if (__builtin_expect(__any(bp.slow), 0))
      row_emit<DT, G, MODE, U, FULL, true>(A, w[s], bp, off[s], row[s], cr[s], nval[s],
                                          base + s * T + tid);
    else
      row_emit<DT, G, MODE, U, FULL, false>(A, w[s], bp, off[s], row[s], cr[s], nval[s],
                                           base + s * T + tid);
    if ((A.emit & kEmitScales) && (tid % G) == 0 && base + s * T + tid < A.nchunks) {
      const int64_t bi = MODE == kModeFlat ? cr[s] / G : row[s] * A.nb + cr[s] / G;
      st_small(A.scales + bi, (uint8_t)bp.e8);
    }
  }
}

// A workgroup whose chunks are all in range (every one but possibly the
// last, in the flat layout) takes the branch-free load path.
template <int DT, int B, int RULE, int MODE, int U, int T>
__global__ __launch_bounds__(T) void row_fwd_kernel(RowArgs A) {
  if (MODE == kModeFlat && (int64_t)(blockIdx.x + 1) * (T * U) <= A.nchunks)
    row_fwd_body<DT, B, RULE, MODE, U, T, true>(A, blockIdx.x);
  else
    row_fwd_body<DT, B, RULE, MODE, U, T, false>(A, blockIdx.x);
}

// Several tensors in one launch (small tensors are launch-bound): tensor j
// owns workgroups [wg0[j], wg0[j + 1]); each runs the single-tensor body in
// its own layout mode.
struct RowBatchArgs {
  RowArgs item[kBatchMax];
  int64_t wg0[kBatchMax + 1];
  int mode[kBatchMax];
  int n;
};

template <int DT, int B, int RULE>
__global__ __launch_bounds__(kRowThreads) void row_fwd_batch_kernel(RowBatchArgs P) {
  const int64_t w = blockIdx.x;
  int j = 0;
  while (j + 1 < P.n && w >= P.wg0[j + 1]) ++j;
  const RowArgs &A = P.item[j];
  const int64_t wg = w - P.wg0[j];
  switch (P.mode[j]) {
    case kModeFlat:
      if ((wg + 1) * kRowThreads <= A.nchunks) row_fwd_body<DT, B, RULE, kModeFlat, 1, kRowThreads, true>(A, wg);
      else row_fwd_body<DT, B, RULE, kModeFlat, 1, kRowThreads, false>(A, wg);
      break;
    case kModeRowsVec: row_fwd_body<DT, B, RULE, kModeRowsVec, 1, kRowThreads, false>(A, wg); break;
    default: row_fwd_body<DT, B, RULE, kModeRowsScalar, 1, kRowThreads, false>(A, wg); break;
  }
}

template <int DT, int B, int RULE, int MODE, int U, int T>
hipError_t launch_shape(const RowArgs &a, hipStream_t st) {
  const int64_t nwg = (a.nchunks + (int64_t)T * U - 1) / ((int64_t)T * U);
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((row_fwd_kernel<DT, B, RULE, MODE, U, T>), dim3((unsigned)nwg), dim3(T), 0, st, a);
  return hipGetLastError();
}

template <int DT, int B, int RULE, int MODE>
hipError_t launch_u(const RowArgs &a, hipStream_t st) {
  if constexpr (MODE == kModeFlat) {
    if (a.emit & kEmitCodes)
      return launch_shape<DT, B, RULE, MODE, DT == kBF16 && B == 128 ? MXFP4_PACK_U_B128 : MXFP4_PACK_U,
                          kPackThreads>(a, st);
    if (a.nchunks > kRowBigChunks) return launch_shape<DT, B, RULE, MODE, MXFP4_ROW_U_BIG, kRowThreads>(a, st);
    return launch_shape<DT, B, RULE, MODE, MXFP4_ROW_U_SMALL, kRowThreads>(a, st);
  } else {
    return launch_shape<DT, B, RULE, MODE, 1, kRowThreads>(a, st);
  }
}

template <int DT, int B, int RULE>
hipError_t dispatch_mode(int mode, const RowArgs &a, hipStream_t st) {
  switch (mode) {
    case kModeFlat: return launch_u<DT, B, RULE, kModeFlat>(a, st);
    case kModeRowsVec: return launch_u<DT, B, RULE, kModeRowsVec>(a, st);
    default: return launch_u<DT, B, RULE, kModeRowsScalar>(a, st);
  }
}

template <int DT, int B>
hipError_t dispatch_rule(int rule, int mode, const RowArgs &a, hipStream_t st) {
  return rule == kFloor ? dispatch_mode<DT, B, kFloor>(mode, a, st)
                        : dispatch_mode<DT, B, kAmct>(mode, a, st);
}

// Kernel arguments and layout mode of one tensor.
int row_args(const RowLaunch &L, RowArgs &a) {
  a.x = static_cast<const uint8_t *>(L.x);
  a.y = static_cast<uint8_t *>(L.y);
  a.mask = reinterpret_cast<uint8_t *>(L.mask);
  a.scales = L.scales;
  a.codes = L.codes;
  a.cols = L.cols;
  a.nb = (L.cols + L.block - 1) / L.block;
  a.cpr = a.nb * (L.block / 8);
  a.mask_row_bytes = 4 * ((L.cols + 31) / 32);
  a.code_row_bytes = (L.cols + 1) / 2;
  a.sf = L.sf;
  a.emit = (L.y ? kEmitY : 0) | (L.mask ? kEmitMask : 0) | (L.scales ? kEmitScales : 0) |
           (L.codes ? kEmitCodes : 0);
  if (L.cols % L.block == 0) {
    a.nchunks = L.rows * L.cols / 8;
    return kModeFlat;
  }
  a.nchunks = L.rows * a.cpr;
  return (L.cols % 8 == 0) ? kModeRowsVec : kModeRowsScalar;
}

template <int DT, int B>
hipError_t batch_rule(int rule, dim3 grid, const RowBatchArgs &p, hipStream_t st) {
  if (rule == kFloor)
    hipLaunchKernelGGL((row_fwd_batch_kernel<DT, B, kFloor>), grid, dim3(kRowThreads), 0, st, p);
  else
    hipLaunchKernelGGL((row_fwd_batch_kernel<DT, B, kAmct>), grid, dim3(kRowThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_row_fwd(const RowLaunch &L, hipStream_t st) {
  RowArgs a;
  const int mode = row_args(L, a);
  if (L.dtype == kBF16)
    return L.block == 32 ? dispatch_rule<kBF16, 32>(L.rule, mode, a, st)
                         : dispatch_rule<kBF16, 128>(L.rule, mode, a, st);
  return L.block == 32 ? dispatch_rule<kF32, 32>(L.rule, mode, a, st)
                       : dispatch_rule<kF32, 128>(L.rule, mode, a, st);
}

hipError_t launch_row_fwd_batch(const RowLaunch *L, int n, hipStream_t st) {
  if (n < 1 || n > kBatchMax) return hipErrorInvalidValue;
  RowBatchArgs p{};
  p.n = n;
  int64_t wg = 0;
  for (int j = 0; j < n; ++j) {
    p.mode[j] = row_args(L[j], p.item[j]);
    p.wg0[j] = wg;
    wg += (p.item[j].nchunks + kRowThreads - 1) / kRowThreads;
  }
  for (int j = n; j <= kBatchMax; ++j) p.wg0[j] = wg;
  for (int j = n; j < kBatchMax; ++j) p.mode[j] = kModeFlat;
  if (wg == 0) return hipSuccess;
  if (wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wg);
  const int dt = L[0].dtype, b = L[0].block, rule = L[0].rule;
  if (dt == kBF16)
    return b == 32 ? batch_rule<kBF16, 32>(rule, grid, p, st) : batch_rule<kBF16, 128>(rule, grid, p, st);
  return b == 32 ? batch_rule<kF32, 32>(rule, grid, p, st) : batch_rule<kF32, 128>(rule, grid, p, st);
}

}  // namespace mxfp4
