// mxfp8_kernels.hip -- MXFP8 (OCP MX) quantization of the grad_output operand
// on gfx950.
//
// The hyper-parallel page feeds grad_output to the W4A8 grouped matmul through
// npu_dynamic_mx_quant (the "ordinary MXFP8 GMM contract"); this is the OCP
// Microscaling conversion: blocks of 32 along each row (128 in the page's
// block-128 mode, whose quantizer works in blocks of 128), one E8M0 scale 2^k
// per block with k = floor(log2 amax) - emax (E4M3 8, E5M2 15), clamped below
// at -127, and every element x / 2^k rounded to nearest, ties to even,
// saturating at the format's largest normal.
//
// Work split: a lane holds 8 consecutive elements of a row (one 16-byte bf16
// load), a block is 4 lanes (16 for blocks of 128; DPP max).  The scale exponent comes from the
// exponent field of the block max, so x * 2^-k is an exact fp32 product; it is
// clamped to +-max with v_med3_f32 and converted two at a time by the hardware
// fp8 conversion (round to nearest even).  8 code bytes per lane leave in one
// 8-byte store (512 contiguous bytes per wave).
#include "mxfp4_device.h"
#include "mxfp4_groups.h"
#include "mxfp4_kernels.h"

namespace mxfp4 {
namespace {

enum { kMx8Flat = 0, kMx8RowsVec = 1, kMx8RowsScalar = 2 };

struct Mx8Args {
  const uint8_t *x;
  uint8_t *q;
  uint8_t *scales;
  int64_t cols;
  int64_t nchunks;  // chunks in the launch
  int64_t cpr;      // chunks per row, padded to whole blocks (row modes)
  int64_t nb;       // blocks per row
};

template <int FMT>
struct Fp8T {
  static constexpr int EMAX = FMT == kE4M3 ? 8 : 15;
  static constexpr float MAXN = FMT == kE4M3 ? 448.0f : 57344.0f;
};

// two scaled, clamped values -> two fp8 bytes in word HI of `old`
template <int FMT, bool HI>
__device__ __forceinline__ int cvt2(float a, float b, int old) {
  if (FMT == kE4M3) return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// Two-wave workgroups: measured on MI355X (32768x7168 bf16, E4M3) 117 us
// against 121 us with four waves, 123 us with one and 120 us with eight.
constexpr int kMx8Threads = 128;

template <int DT, int FMT, int MODE, int G>
__global__ __launch_bounds__(kMx8Threads) void mxfp8_rows_kernel(Mx8Args A) {
  constexpr int NW = PieceT<DT>::NW;
  constexpr int ES = PieceT<DT>::ES;
  constexpr float MAXN = Fp8T<FMT>::MAXN;
  const int64_t i = (int64_t)blockIdx.x * kMx8Threads + threadIdx.x;

  int64_t row = 0, cr = i, off = i * 8;
  int nval = i < A.nchunks ? 8 : 0;
  if (MODE != kMx8Flat) {
    row = i / A.cpr;
    cr = i - row * A.cpr;
    off = row * A.cols + cr * 8;
    const int64_t rem = A.cols - cr * 8;
    nval = i < A.nchunks ? (int)(rem >= 8 ? 8 : (rem > 0 ? rem : 0)) : 0;
  }
  uint32_t w[NW];
  if (MODE == kMx8RowsScalar) load_piece<DT, false>(w, A.x + off * ES, nval);
  else load_piece<DT, true>(w, A.x + off * ES, nval);  // all or nothing

  // block max of the magnitude bits, then the E8M0 byte from its exponent
  uint32_t am = 0;
  if (DT == kBF16) {
    const uint32_t m = pk_max(pk_max(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                              pk_max(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
    am = max32(m & 0xFFFFu, m >> 16) << 16;
  } else {
#pragma unroll
    for (int k = 0; k < NW; ++k) am = max32(am, w[k] & 0x7FFFFFFFu);
  }
  am = group_max<G>(am);
  const int eb = (int)(am >> 23);  // biased exponent of the block max (0: zero / subnormal)
  const int e8 = eb - Fp8T<FMT>::EMAX > 0 ? eb - Fp8T<FMT>::EMAX : 0;
  const float s = __builtin_bit_cast(float, (uint32_t)(254 - e8) << 23);  // 2^(127 - e8) = 2^-k

  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = DT == kBF16 ? (j & 1 ? w[j >> 1] & 0xFFFF0000u : w[j >> 1] << 16) : w[j];
    v[j] = __builtin_amdgcn_fmed3f(__builtin_bit_cast(float, b) * s, -MAXN, MAXN);
  }
  int lo = cvt2<FMT, false>(v[0], v[1], 0);
  lo = cvt2<FMT, true>(v[2], v[3], lo);
  int hi = cvt2<FMT, false>(v[4], v[5], 0);
  hi = cvt2<FMT, true>(v[6], v[7], hi);

  uint8_t *dst = A.q + off;
  if (MODE != kMx8RowsScalar) {
    if (nval == 8) {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 pk = {(uint32_t)lo, (uint32_t)hi};
      __builtin_nontemporal_store(pk, reinterpret_cast<u32x2 *>(dst));
    }
  } else {
    const uint64_t pk = (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32);
    for (int j = 0; j < nval; ++j) dst[j] = (uint8_t)(pk >> (8 * j));
  }
  if ((threadIdx.x & (G - 1)) == 0 && i < A.nchunks) {
    const int64_t bi = MODE == kMx8Flat ? cr / G : row * A.nb + cr / G;
    if (MODE == kMx8Flat || cr * 8 < A.cols) A.scales[bi] = (uint8_t)e8;
  }
}

template <int DT, int FMT, int G>
hipError_t mx8_launch_g(int mode, const Mx8Args &a, hipStream_t st) {
  const int64_t nwg = (a.nchunks + kMx8Threads - 1) / kMx8Threads;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  switch (mode) {
    case kMx8Flat: hipLaunchKernelGGL((mxfp8_rows_kernel<DT, FMT, kMx8Flat, G>), grid, dim3(kMx8Threads), 0, st, a); break;
    case kMx8RowsVec: hipLaunchKernelGGL((mxfp8_rows_kernel<DT, FMT, kMx8RowsVec, G>), grid, dim3(kMx8Threads), 0, st, a); break;
    default: hipLaunchKernelGGL((mxfp8_rows_kernel<DT, FMT, kMx8RowsScalar, G>), grid, dim3(kMx8Threads), 0, st, a); break;
  }
  return hipGetLastError();
}

template <int DT, int FMT>
hipError_t mx8_launch(int block, int mode, const Mx8Args &a, hipStream_t st) {
  return block == 128 ? mx8_launch_g<DT, FMT, 16>(mode, a, st) : mx8_launch_g<DT, FMT, 4>(mode, a, st);
}

// ---- K-major MXFP8 of column-wise / grouped 32-row blocks ---------------------
//
// The TN weight-gradient product reduces over tokens, so its two operands
// (x and grad_output) are quantized in blocks of 32 rows of each column (the
// hyper-parallel page's grouped quantization for block 32: blocks restart at
// every expert's first token) and stored with the tokens contiguous: column c
// becomes row c of q_t, block-row t fills K positions 32t .. 32t + 31 (zero
// codes past a short block's length).
//
// A workgroup takes 4 consecutive block-rows x 128 columns (256-byte bf16 row
// segments read more efficiently than 128-byte ones).  Rows arrive with
// coalesced 16-byte loads into LDS (rows past a block's length as zeros);
// then every thread owns one (column, block-row): the block max, the exact
// scaling, the clamp and the hardware fp8 conversion as in the row-wise
// kernel, and 32 code bytes leave in two 16-byte stores (the 4 block-rows of
// a column are 4 neighbouring lanes: 128 contiguous bytes).

constexpr int kKm8Cols = 128;
constexpr int kKm8Blk = 4;
constexpr int kKm8Threads = kKm8Cols * kKm8Blk;  // one thread per (column, block-row)

struct Km8Args {
  const uint8_t *x;
  uint8_t *q;
  uint8_t *scales;
  const int64_t *group_list;
  int64_t rows, cols, k_blocks, nbt, ntiles_c;
  int num_groups, list_type;
};

template <int DT, int FMT>
__global__ __launch_bounds__(kKm8Threads) void mxfp8_kmajor_kernel(Km8Args A) {
  constexpr int ES = DT == kBF16 ? 2 : 4;
  constexpr int ROWB = kKm8Cols * ES;              // bytes of a tile row
  // block stride in LDS: +32 bytes puts the 4 block-rows that a compute-phase
  // read touches (lanes b = tid & 3) 8 banks apart, so the 32 lanes of a
  // half-wave (4 block-rows x 8 columns' words) hit 32 different banks
  constexpr int BSTRIDE = 32 * ROWB + 32;
  constexpr float MAXN = Fp8T<FMT>::MAXN;
  __shared__ __align__(16) uint8_t tile[kKm8Blk * BSTRIDE];

  const int tid = threadIdx.x;
  const int64_t tc = blockIdx.x % A.ntiles_c;
  const int64_t t0 = (blockIdx.x / A.ntiles_c) * kKm8Blk;
  const int64_t c0 = tc * kKm8Cols;
  const int ncol = A.cols - c0 < kKm8Cols ? (int)(A.cols - c0) : kKm8Cols;

  // block-rows t0 .. t0 + 3: first row and length (0 past the last)
  int64_t start[kKm8Blk], len[kKm8Blk];
  if (A.group_list) {
    const int64_t tt[kKm8Blk] = {t0, t0 + 1, t0 + 2, t0 + 3};
    int grp[kKm8Blk];
    block_rows_lookup<kKm8Blk>(A.group_list, A.num_groups, A.list_type, A.rows, 5, tt, start, len, grp);
  } else {
#pragma unroll
    for (int b = 0; b < kKm8Blk; ++b) {
      start[b] = (t0 + b) * 32;
      const int64_t rem = A.rows - start[b];
      len[b] = t0 + b < A.nbt ? (rem < 32 ? rem : 32) : 0;
    }
  }

  // load: 16 bytes per thread per pass (ROWB / 16 threads per row).  With
  // whole 16-byte pieces (the usual case) every load is issued before any is
  // stored, rows past a block's length reading the tensor's first bytes and
  // storing zeros, so a workgroup has all of its 16 KiB (bf16) in flight;
  // loads under a per-lane branch would each be waited for in turn.
  constexpr int TPR = ROWB / 16;                   // threads per row
  constexpr int RPP = kKm8Threads / TPR;           // rows per pass
  constexpr int NP = 32 / RPP;                     // passes per block
  const int lr = tid / TPR, lc = tid % TPR;
  const bool full_w = ncol == kKm8Cols && (A.cols * ES) % 16 == 0;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if (full_w) {
    u32x4 v[kKm8Blk][NP];
#pragma unroll
    for (int b = 0; b < kKm8Blk; ++b)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int r = lr + RPP * p;
        const bool ok = r < len[b];
        const uint8_t *src = ok ? A.x + ((start[b] + r) * A.cols + c0) * ES + 16 * lc : A.x;
        v[b][p] = *reinterpret_cast<const u32x4 *>(src);
      }
#pragma unroll
    for (int b = 0; b < kKm8Blk; ++b)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int r = lr + RPP * p;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(&tile[b * BSTRIDE + r * ROWB + 16 * lc]) = r < len[b] ? v[b][p] : z;
      }
  } else {
#pragma unroll
    for (int b = 0; b < kKm8Blk; ++b) {
#pragma unroll
      for (int r = lr; r < 32; r += RPP) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < len[b]) {
          // ragged right edge or unaligned rows: element by element
          const uint8_t *src = A.x + ((start[b] + r) * A.cols + c0) * ES + 16 * lc;
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int e = 0; e < 16 / ES; ++e) {
            const int col = lc * (16 / ES) + e;
            if (col < ncol) {
              const uint32_t u = ES == 2 ? (uint32_t) * reinterpret_cast<const uint16_t *>(src + e * ES)
                                         : *reinterpret_cast<const uint32_t *>(src + e * ES);
              w[(e * ES) / 4] |= ES == 2 ? u << (16 * (e & 1)) : u;
            }
          }
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
        *reinterpret_cast<u32x4 *>(&tile[b * BSTRIDE + r * ROWB + 16 * lc]) = v;
      }
    }
  }
  __syncthreads();

  // compute: lane -> (column, block-row); 4 neighbouring lanes share a column
  const int b = tid & (kKm8Blk - 1), c = tid >> 2;
  if (c >= ncol || len[b] == 0) return;
  float v[32];
  uint32_t am = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const uint8_t *p = &tile[b * BSTRIDE + r * ROWB + c * ES];
    const uint32_t u = ES == 2 ? (uint32_t) * reinterpret_cast<const uint16_t *>(p) << 16
                               : *reinterpret_cast<const uint32_t *>(p);
    am = max32(am, u & 0x7FFFFFFFu);
    v[r] = __builtin_bit_cast(float, u);
  }
  const int eb = (int)(am >> 23);  // biased exponent of the block max (0: zero / subnormal)
  const int e8 = eb - Fp8T<FMT>::EMAX > 0 ? eb - Fp8T<FMT>::EMAX : 0;
  const float sc = __builtin_bit_cast(float, (uint32_t)(254 - e8) << 23);  // 2^(127 - e8) = 2^-k
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float a0 = __builtin_amdgcn_fmed3f(v[4 * k] * sc, -MAXN, MAXN);
    const float a1 = __builtin_amdgcn_fmed3f(v[4 * k + 1] * sc, -MAXN, MAXN);
    const float a2 = __builtin_amdgcn_fmed3f(v[4 * k + 2] * sc, -MAXN, MAXN);
    const float a3 = __builtin_amdgcn_fmed3f(v[4 * k + 3] * sc, -MAXN, MAXN);
    w[k] = (uint32_t)cvt2<FMT, true>(a2, a3, cvt2<FMT, false>(a0, a1, 0));
  }
  uint8_t *dst = A.q + (c0 + c) * A.k_blocks * 32 + (t0 + b) * 32;
  *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{w[4], w[5], w[6], w[7]};
  A.scales[(c0 + c) * A.k_blocks + t0 + b] = (uint8_t)e8;
}

}  // namespace

hipError_t launch_mxfp8_kmajor(const Km8Launch &L, hipStream_t st) {
  Km8Args a;
  a.x = static_cast<const uint8_t *>(L.x);
  a.q = L.q;
  a.scales = L.scales;
  a.group_list = L.group_list;
  a.rows = L.rows;
  a.cols = L.cols;
  a.k_blocks = L.k_blocks;
  a.num_groups = L.num_groups;
  a.list_type = L.list_type;
  a.nbt = L.group_list ? L.k_blocks : (L.rows + 31) / 32;
  a.ntiles_c = (L.cols + kKm8Cols - 1) / kKm8Cols;
  const int64_t ntiles = (a.nbt + kKm8Blk - 1) / kKm8Blk * a.ntiles_c;
  if (ntiles == 0) return hipSuccess;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ntiles);
  if (L.dtype == kBF16) {
    if (L.fmt == kE4M3) hipLaunchKernelGGL((mxfp8_kmajor_kernel<kBF16, kE4M3>), grid, dim3(kKm8Threads), 0, st, a);
    else hipLaunchKernelGGL((mxfp8_kmajor_kernel<kBF16, kE5M2>), grid, dim3(kKm8Threads), 0, st, a);
  } else {
    if (L.fmt == kE4M3) hipLaunchKernelGGL((mxfp8_kmajor_kernel<kF32, kE4M3>), grid, dim3(kKm8Threads), 0, st, a);
    else hipLaunchKernelGGL((mxfp8_kmajor_kernel<kF32, kE5M2>), grid, dim3(kKm8Threads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_mxfp8_rows(const Mx8Launch &L, hipStream_t st) {
  Mx8Args a;
  a.x = static_cast<const uint8_t *>(L.x);
  a.q = L.q;
  a.scales = L.scales;
  a.cols = L.cols;
  a.nb = (L.cols + L.block - 1) / L.block;
  a.cpr = a.nb * (L.block / 8);
  int mode;
  if (L.cols % L.block == 0) {
    mode = kMx8Flat;
    a.nchunks = L.rows * L.cols / 8;
  } else {
    mode = L.cols % 8 == 0 ? kMx8RowsVec : kMx8RowsScalar;
    a.nchunks = L.rows * a.cpr;
  }
  const int b = L.block;
  if (L.dtype == kBF16)
    return L.fmt == kE4M3 ? mx8_launch<kBF16, kE4M3>(b, mode, a, st) : mx8_launch<kBF16, kE5M2>(b, mode, a, st);
  return L.fmt == kE4M3 ? mx8_launch<kF32, kE4M3>(b, mode, a, st) : mx8_launch<kF32, kE5M2>(b, mode, a, st);
}

}  // namespace mxfp4
