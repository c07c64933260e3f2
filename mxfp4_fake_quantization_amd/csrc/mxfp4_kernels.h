// mxfp4_kernels.h -- host-side launch descriptors of the gfx950 kernels.
// The C-ABI layer (api.hip) validates arguments and calls these launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

enum { kEmitY = 1, kEmitMask = 2, kEmitScales = 4, kEmitCodes = 8 };

// Row-wise forward: y / mask / scales / codes in one pass.
struct RowLaunch {
  int dtype, block, rule;
  int64_t rows, cols;
  float sf;
  const void *x;
  void *y;
  uint32_t *mask;
  uint8_t *scales;
  uint8_t *codes;
};
hipError_t launch_row_fwd(const RowLaunch &L, hipStream_t stream);
// Up to kBatchMax row-wise forwards in one launch (same dtype, block, rule
// and scale factor; y / mask / scales only).
constexpr int kBatchMax = 8;
hipError_t launch_row_fwd_batch(const RowLaunch *L, int n, hipStream_t stream);

// Column-wise / dual-direction / grouped forward (block-row tiles).
struct ColLaunch {
  int dtype, block, rule;
  int64_t rows, cols;
  float sf;
  const void *x;
  void *y_col;          // column-direction outputs
  uint32_t *mask_col;
  uint8_t *scales_col;
  void *y_row;          // row-direction outputs (dual only)
  uint32_t *mask_row;
  uint8_t *scales_row;
  const int64_t *group_list;  // grouped only
  int num_groups, list_type;
};
hipError_t launch_col_fwd(const ColLaunch &L, hipStream_t stream);

// STE backward.
struct SteLaunch {
  int dtype, block, layout;  // layout: 1 row, 2 col, 4 grouped
  int64_t rows, cols;
  const void *g;
  const uint32_t *mask;  // NULL: plain STE (copy)
  void *g_in;
  const int64_t *group_list;
  int num_groups, list_type;
};
hipError_t launch_ste_bwd(const SteLaunch &L, hipStream_t stream);
// Up to kBatchMax STE backwards with ROW bitmaps (or none) in one launch.
hipError_t launch_ste_row_batch(const SteLaunch *L, int n, hipStream_t stream);
// ROW / COL saturation bitmap -> one 0/1 byte per element (layout 1 or 2).
hipError_t launch_mask_bool(int layout, int64_t rows, int64_t cols, const uint32_t *mask, uint8_t *out,
                            hipStream_t stream);


// K-major packed form of column-wise / grouped blocks.
struct KmLaunch {
  int dtype, block, rule;
  int64_t rows, cols;
  float sf;
  const void *x;
  const int64_t *group_list;  // NULL: dense column-wise blocks
  int num_groups, list_type;
  int64_t k_blocks;
  uint8_t *codes;   // [cols, k_blocks * block / 2]
  uint8_t *scales;  // [cols, k_blocks]
};
hipError_t launch_kmajor_pack(const KmLaunch &L, hipStream_t stream);

// Decode of row-wise packed codes.
struct DqLaunch {
  int dtype, block;
  int64_t rows, cols;
  const uint8_t *codes;
  const uint8_t *scales;
  void *y;
};
hipError_t launch_dequant(const DqLaunch &L, hipStream_t stream);


// MXFP8 (OCP MX) row-wise quantization.
enum { kE4M3 = 0, kE5M2 = 1 };
struct Mx8Launch {
  int dtype, fmt;
  int64_t rows, cols;
  const void *x;
  uint8_t *q;       // [rows, cols] fp8 bytes
  uint8_t *scales;  // [rows, ceil(cols/block)] E8M0
  int block;        // 32 or 128
};
hipError_t launch_mxfp8_rows(const Mx8Launch &L, hipStream_t stream);

// K-major MXFP8 of column-wise / grouped 32-row blocks.
struct Km8Launch {
  int dtype, fmt;
  int64_t rows, cols;
  const void *x;
  const int64_t *group_list;  // NULL: dense column-wise blocks
  int num_groups, list_type;
  int64_t k_blocks;
  uint8_t *q;       // [cols, k_blocks * 32]
  uint8_t *scales;  // [cols, k_blocks]
};
hipError_t launch_mxfp8_kmajor(const Km8Launch &L, hipStream_t stream);

// Grouped MX matrix product C = A . B^T (both operands K-contiguous).
// Element formats as the MFMA format codes: 0 E4M3, 1 E5M2, 4 E2M1.
enum { kFmtE4M3 = 0, kFmtE5M2 = 1, kFmtE2M1 = 4 };
struct GemmLaunch {
  int group_type;        // 0: groups split rows of A (B per group); 2: groups split K
  int a_fmt, b_fmt, a_block, b_block, out_f32;
  int64_t M, N, K, k_blocks;
  const uint8_t *a, *as;  // [M, lda] codes, [M, ldas] E8M0
  const uint8_t *b, *bs;  // [N, ldb] codes, [N, ldbs] E8M0 (+ g * b_gs / b_gss)
  int64_t lda, ldas, ldb, ldbs, b_gs, b_gss, ldc;
  void *c;
  const int64_t *group_list;
  int num_groups, list_type;
};
hipError_t launch_mx_gemm(const GemmLaunch &L, hipStream_t stream);

}  // namespace mxfp4
