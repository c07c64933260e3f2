// mxfp8_kernels.hip -- MXFP8 (OCP MX) quantization of the grad_output operand
// on gfx950.
//
// The hyper-parallel page feeds grad_output to the W4A8 grouped matmul through
// npu_dynamic_mx_quant (the "ordinary MXFP8 GMM contract"); this is the OCP
// Microscaling conversion: blocks of 32 along each row, one E8M0 scale 2^k per
// block with k = floor(log2 amax) - emax (E4M3 8, E5M2 15), clamped below at
// -127, and every element x / 2^k rounded to nearest, ties to even,
// saturating at the format's largest normal.
//
// Work split: a lane holds 8 consecutive elements of a row (one 16-byte bf16
// load), a block is 4 lanes (DPP max).  The scale exponent comes from the
// exponent field of the block max, so x * 2^-k is an exact fp32 product; it is
// clamped to +-max with v_med3_f32 and converted two at a time by the hardware
// fp8 conversion (round to nearest even).  8 code bytes per lane leave in one
// 8-byte store (512 contiguous bytes per wave).
#include "mxfp4_device.h"
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

template <int DT, int FMT, int MODE>
__global__ __launch_bounds__(kThreads) void mxfp8_rows_kernel(Mx8Args A) {
  constexpr int NW = PieceT<DT>::NW;
  constexpr int ES = PieceT<DT>::ES;
  constexpr float MAXN = Fp8T<FMT>::MAXN;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;

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
  am = group_max<4>(am);
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
  if ((threadIdx.x & 3) == 0 && i < A.nchunks) {
    const int64_t bi = MODE == kMx8Flat ? cr >> 2 : row * A.nb + (cr >> 2);
    if (MODE == kMx8Flat || cr * 8 < A.cols) A.scales[bi] = (uint8_t)e8;
  }
}

template <int DT, int FMT>
hipError_t mx8_launch(int mode, const Mx8Args &a, hipStream_t st) {
  const int64_t nwg = (a.nchunks + kThreads - 1) / kThreads;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg);
  switch (mode) {
    case kMx8Flat: hipLaunchKernelGGL((mxfp8_rows_kernel<DT, FMT, kMx8Flat>), grid, dim3(kThreads), 0, st, a); break;
    case kMx8RowsVec: hipLaunchKernelGGL((mxfp8_rows_kernel<DT, FMT, kMx8RowsVec>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((mxfp8_rows_kernel<DT, FMT, kMx8RowsScalar>), grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp8_rows(const Mx8Launch &L, hipStream_t st) {
  Mx8Args a;
  a.x = static_cast<const uint8_t *>(L.x);
  a.q = L.q;
  a.scales = L.scales;
  a.cols = L.cols;
  a.nb = (L.cols + 31) / 32;
  a.cpr = a.nb * 4;
  int mode;
  if (L.cols % 32 == 0) {
    mode = kMx8Flat;
    a.nchunks = L.rows * L.cols / 8;
  } else {
    mode = L.cols % 8 == 0 ? kMx8RowsVec : kMx8RowsScalar;
    a.nchunks = L.rows * a.cpr;
  }
  if (L.dtype == kBF16)
    return L.fmt == kE4M3 ? mx8_launch<kBF16, kE4M3>(mode, a, st) : mx8_launch<kBF16, kE5M2>(mode, a, st);
  return L.fmt == kE4M3 ? mx8_launch<kF32, kE4M3>(mode, a, st) : mx8_launch<kF32, kE5M2>(mode, a, st);
}

}  // namespace mxfp4
