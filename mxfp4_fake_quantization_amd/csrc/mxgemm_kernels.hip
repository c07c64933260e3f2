// mxgemm_kernels.hip -- grouped MX matrix product on gfx950 scaled MFMA.
//
// The hyper-parallel page's FakeW4A8GroupedLinear hands its directional
// operands to a grouped matmul in three layouts: NN (forward: tokens x the
// column-wise weight view), NT (input gradient: grad_output x the row-wise
// weight view, transposed) and TN (weight gradient: column-wise x^T times
// column-wise grad_output, per expert).  With both operands stored with the
// reduction dimension K contiguous, all three are one product per group,
//     C[m, n] = sum_k A[m, k] * B[n, k],
// where A is MXFP8 (E4M3 / E5M2 bytes + E8M0 per 32 or 128 along K) and B is
// MXFP4 (E2M1 nibble pairs, low nibble = even K) or MXFP8.  Groups either
// split the rows of A and pick B_g (NN / NT), or split K into block-aligned
// spans with one output matrix per group (TN).
//
// One v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32x64 A slice by a 64x32
// B slice, applying the E8M0 scales of both in the matrix core: lane l
// supplies row / column l % 32 and K half h = l / 32, one scale byte per lane
// for K-block h.  Measured operand layout of the instruction (A fp8: bytes
// 0-15 are K 16h..16h+15, bytes 16-31 are K 32+16h..; B fp4: nibble j is K
// 32h+j; result register v of lane l is row 8(v/4) + 4h + v%4, column l%32).
//
// Work split (GemmShape below): a 512-thread workgroup computes a 256 x 256
// tile as 4 x 2 waves of 2 x 4 MFMA tiles (two waves per SIMD, so one
// wave's LDS and address work overlaps the other's MFMAs), one workgroup per
// CU.  A row-split product of at most 8 N-tiles per row whose tiles leave a
// last round at most half full (with one tile per CU, R tiles = full rounds
// + R mod CUs) runs the full rounds in one launch, dealt to the XCDs by the
// real tile count, and the tail in a second launch of 128 x 128 tiles (2 x 2
// waves of 2 x 2 MFMA tiles, two workgroups per CU), four per big tile, so
// that the tail spreads over more CUs.  K advances by 128 per step.  Both operand
// slices go global -> registers -> LDS (double-buffered, 128-byte rows at a
// 144-byte stride: conflict-free 16-lane read phases, and every fragment
// read is a per-lane base plus an immediate) while the previous step's
// MFMAs run.  An E2M1 B row holds only 64 bytes per K step, half a
// 128-byte cache line; B is therefore staged two K steps at a time (one
// whole line per row, half of the tile's rows loaded during each step), so
// every B request fetches a full line.  Scale bytes travel in chunks of 16
// K-blocks per tile row (4 steps), also double-buffered in LDS and streamed
// one coalesced slice per step, so every lane reads a tile row's scale bytes
// for a whole step with one LDS load (the two K halves take bytes 0 and 2 of
// that register through the MFMA's op_sel).  The loop body is one basic
// block: the next step's global loads, the fragment reads and MFMAs, then
// the prefetch's LDS stores and one barrier.  Blocks outside a K range load as zero
// codes with scale 2^0; rows and columns past the tile edge load a valid
// neighbour and are not stored.
#include "mxfp4_device.h"
#include "mxfp4_groups.h"
#include "mxfp4_kernels.h"

#include <atomic>
#include <type_traits>

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Tile shape (both B formats): 8 waves per workgroup (2 per SIMD, so one
// wave's LDS and address work overlaps the other's MFMAs), 4 x 2 waves of
// 2 x 4 MFMA tiles = 256 x 256, one workgroup per CU (160 KiB of LDS).  The
// fp8-B form (fragments twice as large) used 128 x 128 tiles, two workgroups
// per CU, while its 256 x 256 form spilled; with the scale and address
// registers trimmed it fits (no scratch) and measured 644 -> 566 us on the
// MoE weight gradient.
// SMALL: 128 x 128 tiles (2 x 2 waves of 2 x 2 MFMA tiles, 4 waves, two
// workgroups per CU) for the tail of a row-split product: the last, partly
// filled round of 256 x 256 tiles, each cut into four.
template <int BF, bool SMALL = false>
struct GemmShape {
  static constexpr int wavesM = SMALL ? 2 : 4, wavesN = 2, tilesM = 2, tilesN = SMALL ? 2 : 4;
  static constexpr int threads = 64 * wavesM * wavesN;
  static constexpr int BM = 32 * tilesM * wavesM, BN = 32 * tilesN * wavesN;
  // minimum waves per SIMD (the second __launch_bounds__ argument): the
  // 256 x 256 workgroup already puts two on each SIMD; a SMALL workgroup has
  // one per SIMD, and 2 keeps its registers low enough for two workgroups
  // per CU (80 KiB of LDS each)
  static constexpr int per_cu = SMALL ? 2 : 1;
};
// Row-split products are tiled in 256 x 256 units whatever the shape.
constexpr int kBigLog = 8;

struct GemmArgs {
  const uint8_t *a, *as, *b, *bs;
  void *c;
  int64_t lda, ldas, ldb, ldbs, b_gs, b_gss, ldc;
  int64_t M, N, K;
  int64_t k_blocks;      // reduction-split groups: K-block capacity of the operands
  const int64_t *gl;
  int G, list_type, group_type, out_f32;
  int a_sb, b_sb;        // log2(scale block / 32): 0 or 2
  int s4;                // both scale arrays have dword-aligned rows: dword slice loads
  int c16;               // bf16 output with 16-byte aligned rows: whole tiles stored through LDS
  int ncu;               // compute units of the device (row-split tail decision)
  int64_t tiles_m, tiles_n, total;
};

typedef const uint8_t __attribute__((address_space(1))) *gp8;
typedef const uint32_t __attribute__((address_space(1))) *gp32;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Tile id -> (M-tile, N-tile) in bands of `band` M-tiles walked N-tile by
// N-tile, so that the tiles an XCD runs at the same time cover a few M-tiles
// and a few N-tiles instead of one M-tile's whole row of N-tiles (whose
// weights would not stay in its L2).
__device__ __forceinline__ void band_tile(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t band, int64_t *tm,
                                          int64_t *tn) {
  const int64_t b = t / (band * tiles_n);
  const int64_t r = t - b * band * tiles_n;
  const int64_t rows = tiles_m - b * band < band ? tiles_m - b * band : band;
  *tn = r / rows;
  *tm = b * band + (r - *tn * rows);
}

// Workgroup id -> tile id such that each XCD (workgroups are dealt to the 8
// XCDs round-robin) runs a contiguous range of tiles and shares its L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t id, int64_t total) {
  const int64_t q = total >> 3, r = total & 7;
  const int64_t x = id & 7, loc = id >> 3;
  return x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
}

// Workgroup id -> slot in [0, total) with each XCD given a contiguous, equal
// share (ids beyond an XCD's share return false).  Unlike xcd_tile, total is
// the count known only on the device, so the grid may be larger.
__device__ __forceinline__ bool xcd_slot(int64_t id, int64_t total, int64_t *slot) {
  const int64_t q = total >> 3, r = total & 7;
  const int64_t x = id & 7, loc = id >> 3;
  if (loc >= (x < r ? q + 1 : q)) return false;
  *slot = x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
  return true;
}

// One scaled MFMA taking byte OS of each scale register.
template <int AF, int BF, int OS>
__device__ __forceinline__ v16f mfma_sel(v8i a, v8i b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, AF, BF, OS, (int)sa, OS, (int)sb);
}

template <int AF, int BF, bool S4, bool SMALL>
__global__ __launch_bounds__((GemmShape<BF, SMALL>::threads), (GemmShape<BF, SMALL>::per_cu)) void mxgemm_kernel(GemmArgs P) {
  using Sh = GemmShape<BF, SMALL>;
  constexpr int WVM = Sh::wavesM, WVN = Sh::wavesN, WM = Sh::tilesM, WN = Sh::tilesN;
  constexpr int NT = Sh::threads;
  constexpr int BM = Sh::BM, BN = Sh::BN;
  constexpr bool B4 = BF == kFmtE2M1;
  // B4: a 128-byte LDS row holds two K steps (pair) of E2M1 codes; fp8 B:
  // one K step.  Either way 8 slots of 16 bytes per row.
  constexpr int A_LD = BM * 8 / NT;             // 16-byte A loads per thread per step
  constexpr int RSTEP = NT / 8;                 // rows per load pass (A and B)
  constexpr int B_LD = BN * 8 / NT / (B4 ? 2 : 1);  // 16-byte B loads per thread per step
  static_assert(WVM * WVN * 64 == NT && BM == 32 * WM * WVM && BN == 32 * WN * WVN, "tile shape");
  static_assert(BM / 8 * 8 == NT / 2 && BN / 8 * 8 == NT / 2, "one scale dword per thread per step");
  // operand rows of 128 bytes at a 144-byte stride: 16 lanes reading the
  // same 16-byte slot of 16 consecutive rows hit all 64 banks once, and a
  // lane's slot offsets are immediates
  constexpr int RS = 144;
  __shared__ __align__(16) uint8_t sA[2][BM * RS];
  __shared__ __align__(16) uint8_t sB[2][BN * RS];
  __shared__ __align__(16) uint8_t sSA[2][BM * 16];  // scale chunks (16 K-blocks per row)
  __shared__ __align__(16) uint8_t sSB[2][BN * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  // ---- tile -> rows, columns, K range, operand and output bases ----
  int64_t m0, mlen, n0, kb0, kb1, klo = 0;  // steps start at kb0; blocks below klo are masked
  const uint8_t *bbase = P.b, *bsbase = P.bs;
  int64_t cbase = 0;  // element offset of the output matrix
  if (P.group_type == 0) {
    // The grid is sized for an upper bound of the 256 x 256 tiles.  Rows of
    // at most 8 N-tiles (NN on the MoE layer) are walked in row order: the
    // groups give the real tile count R; with one big tile per CU, R = full
    // rounds + a tail T = R mod CUs, and a tail of at most half a round goes
    // to the SMALL launch as four 128 x 128 tiles per big tile while the other
    // tiles are dealt to the XCDs in equal contiguous shares of the real
    // count.  Rows of more than 8 N-tiles (NT: 28) go in bands of 4 M-tiles
    // over the upper bound (weight re-reads 9.0x -> 5.4x the unique bytes,
    // time unchanged), dealt by xcd_tile, with no tail launch: the tail
    // split measured 2 % slower there (NT on the MoE layer 526 -> 537 us).
    int64_t v, sub = 0, tm, tn;
    if (P.tiles_n <= 8) {
      int64_t rm;
      if (P.gl) {
        int64_t before, last;
        group_block_span(P.gl, P.G, P.list_type, P.M, kBigLog, P.G - 1, &before, &last);
        rm = before + last;
      } else {
        rm = (P.M + 255) >> kBigLog;
      }
      const int64_t R = rm * P.tiles_n;
      const int64_t T = R % P.ncu;
      const bool split = T > 0 && 2 * T <= P.ncu;
      const int64_t DP = split ? R - T : R;
      if (!SMALL) {
        if (!xcd_slot(blockIdx.x, DP, &v)) return;
      } else {
        int64_t s;
        if (!split || !xcd_slot(blockIdx.x, 4 * T, &s)) return;
        v = DP + (s >> 2);
        sub = s & 3;
      }
      tm = v / P.tiles_n;
      tn = v - tm * P.tiles_n;
    } else {
      if (SMALL) return;
      v = xcd_tile(blockIdx.x, P.total);
      band_tile(v, P.tiles_m, P.tiles_n, 4, &tm, &tn);
    }
    n0 = tn << kBigLog;
    int g = 0;
    if (P.gl) {
      block_row_uniform<false>(P.gl, P.G, P.list_type, P.M, kBigLog, tm, &m0, &mlen, &g);
    } else {
      m0 = tm << kBigLog;
      mlen = P.M - m0 < 256 ? P.M - m0 : 256;
    }
    if (SMALL) {
      m0 += BM * (sub >> 1);
      mlen -= BM * (sub >> 1);
      mlen = mlen < BM ? mlen : BM;
      n0 += BN * (sub & 1);
    }
    if (mlen <= 0 || n0 >= P.N) return;  // workgroup-uniform
    bbase += (int64_t)g * P.b_gs;
    bsbase += (int64_t)g * P.b_gss;
    kb0 = 0;
    kb1 = (P.K + 31) >> 5;
  } else {
    if (SMALL) return;  // K-split products are launched with the 256 x 256 shape only
    const int64_t tile = xcd_tile(blockIdx.x, P.total);
    const int64_t per = P.tiles_m * P.tiles_n;
    const int g = (int)(tile / per);
    const int64_t r = tile - (int64_t)g * per;
    // bands of 4 M-tiles (TN on the MoE layer, 256 x 256 tiles: 578 us with
    // bands of 8, 565 with 2, 561 with 4; with the earlier 128 x 128 tiles
    // bands of 8 took the re-reads from 10.2x to 5.1x the unique bytes)
    int64_t tm, tn;
    band_tile(r, P.tiles_m, P.tiles_n, 4, &tm, &tn);
    m0 = tm * BM;
    mlen = P.M - m0 < BM ? P.M - m0 : BM;
    n0 = tn * BN;
    int64_t nb;
    group_block_span(P.gl, P.G, P.list_type, P.K, 5, g, &kb0, &nb);
    kb1 = kb0 + nb < P.k_blocks ? kb0 + nb : P.k_blocks;
    if (kb0 > kb1) kb0 = kb1;
    // steps start on a multiple of 4 blocks (dword-aligned scale chunks);
    // the blocks of the previous group in the first step are masked
    klo = kb0;
    kb0 &= ~(int64_t)3;
    cbase = (int64_t)g * P.M * P.ldc;
  }
  const int64_t nlen = P.N - n0 < BN ? P.N - n0 : BN;

  // ---- per-thread load offsets (32-bit, from per-tile bases) ----
  // Thread (row r, slot c): r = tid / 8 + RSTEP * i, c = tid % 8 (16 bytes).
  const uint8_t *abase = P.a + m0 * P.lda;
  const uint8_t *asbase = P.as + m0 * P.ldas;
  bbase += n0 * P.ldb;
  bsbase += n0 * P.ldbs;
  const int lr = tid >> 3, lc = tid & 7;
  uint32_t aoff[A_LD], boff0[B_LD], boff1[B_LD];  // boff1: E2M1 B, second half of the rows
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int row = lr + RSTEP * i;
    aoff[i] = (uint32_t)((row < mlen ? row : mlen - 1) * P.lda) + 16 * lc;
  }
#pragma unroll
  for (int t = 0; t < (B4 ? 2 : 1); ++t)
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int row = t * (BN / 2) + lr + RSTEP * i;  // B4: half t of the rows
      const uint32_t o = (uint32_t)((row < nlen ? row : nlen - 1) * P.ldb) + 16 * lc;
      if (t) boff1[i] = o;
      else boff0[i] = o;
    }
  const int wr0 = (wave / WVN) * 32 * WM, wc0 = (wave % WVN) * 32 * WN;

  // ---- scale bytes: chunks of 16 K-blocks (4 steps) staged in LDS ----
  // Chunk c holds, for every tile row, the scale bytes of blocks
  // [kb0 + 16c, kb0 + 16c + 16) (16 bytes, or 4 for 128-element blocks).
  // While chunk c is in use, chunk c + 1 arrives one quarter per step:
  // step 4c + p stores rows [Rp, Rp + R) of A (waves of the first half) or
  // of B (second half), R = NT / 8 rows (a tile has 4R rows), one dword per
  // thread, 4 threads per 16-byte row, loaded from global memory during the
  // step before.
  // Bytes outside [klo, kb1) are replaced by 127 (2^0) when stored, so the
  // MFMAs of masked blocks (zero codes) see a finite scale.
  // A wave loads either A or B slices: the values below are wave-uniform and
  // kept in scalar registers.  Row offsets fit 32 bits (rows <= 256, scale
  // row strides <= 2^24 bytes).
  const bool sl_b = tid >= NT / 2;
  const int sr = (tid & (NT / 2 - 1)) >> 2, sd = tid & 3;
  const int sb_log = __builtin_amdgcn_readfirstlane(sl_b ? P.b_sb : P.a_sb);
  const int s_lo = (int)(klo >> sb_log);                                // first valid byte
  const int s_hi = (int)((kb1 + (1 << sb_log) - 1) >> sb_log);         // past the last
  const uint64_t sbp = (uint64_t)(sl_b ? bsbase : asbase);
  const gp8 s_base = (gp8)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(sbp >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sbp));
  const uint32_t s_ld = (uint32_t)__builtin_amdgcn_readfirstlane((int)(sl_b ? P.ldbs : P.ldas));
  const int s_rows = __builtin_amdgcn_readfirstlane((int)(sl_b ? nlen : mlen));
  // A slice is loaded one step before it is stored (pv: loaded during the
  // previous step, pc: its bytes as one dword, being stored), so that the
  // step's last wait for its loads does not wait for the scattered scale rows.
  uint32_t pv[S4 ? 1 : 4], pc;
  auto load_slice = [&](int64_t chunk, int piece) {
    const int rw = piece * (NT / 8) + sr;
    const int row = rw < s_rows ? rw : s_rows - 1;
    const int pbyte = (int)((kb0 + 16 * chunk) >> sb_log) + (sb_log ? 0 : 4 * sd);
    const gp8 rp = s_base + (uint32_t)row * s_ld;
    const int at = pbyte < s_hi ? pbyte : s_hi - 1;  // in bounds (s_hi <= row length)
    if (S4) {
      pv[0] = *(gp32)(rp + (at & ~3));
    } else {
#pragma unroll
      for (int e = 0; e < (S4 ? 1 : 4); ++e) pv[e] = rp[at + e < s_hi ? at + e : s_hi - 1];
    }
  };
  auto take_slice = [&]() {
    pc = pv[0];
#pragma unroll
    for (int e = 1; e < (S4 ? 1 : 4); ++e) pc |= pv[e] << (8 * e);
  };
  auto store_slice = [&](int64_t chunk, int sbuf, int piece) {
    const int pbyte = (int)((kb0 + 16 * chunk) >> sb_log) + (sb_log ? 0 : 4 * sd);
    uint32_t v = pc;
    // keep bytes pbyte + e inside [s_lo, s_hi)
    const int lead = s_lo - pbyte, cnt = s_hi - pbyte;
    const int nlead = lead <= 0 ? 0 : (lead >= 4 ? 4 : lead);
    const int nval = cnt <= 0 ? 0 : (cnt >= 4 ? 4 : cnt);
    const uint32_t hi_m = nval >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nval)) - 1u);
    const uint32_t lo_m = nlead >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nlead)) - 1u);
    const uint32_t keep = hi_m & ~lo_m;
    v = (v & keep) | (0x7F7F7F7Fu & ~keep);
    // 128-element blocks: the chunk's 4 bytes are one per step; thread sd
    // writes step sd's byte once per 32-element block, so that a chunk row
    // reads the same way for both block sizes
    if (sb_log) v = ((v >> (8 * sd)) & 0xFFu) * 0x01010101u;
    uint8_t *dst = sl_b ? &sSB[sbuf][0] : &sSA[sbuf][0];
    *reinterpret_cast<uint32_t *>(dst + (piece * (NT / 8) + sr) * 16 + 4 * sd) = v;
  };

  // Codes global -> registers.  A: the K step starting at block kb (slot c =
  // blocks kb + c/2).  B fp8: the same; B E2M1: half t of the rows of the
  // pair of steps starting at block kb (slot c = block kb + c).  The masked
  // forms (steps or pairs that can be partial) read clamped in-bounds
  // addresses and zero slots outside [klo, kb1) when storing.
  u32x4 ra[A_LD], rb[B_LD];
  bool ain = true, bin = true;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  constexpr int BSH = B4 ? 4 : 5;  // log2 bytes per 32-element block of B
  constexpr int BBLK = B4 ? 1 : 2; // slots per block of B
  auto load_a = [&](int64_t kb, bool masked) {
    int64_t at = kb << 5;
    if (masked) {
      const int64_t ablk = kb + (lc >> 1);
      ain = ablk >= klo && ablk < kb1;
      if (!ain) at = ((kb1 - 1) << 5) - 16 * lc;
    }
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(abase + at + aoff[i]);
  };
  auto load_b = [&](int64_t kb, int t, bool masked) {
    int64_t bt = kb << BSH;
    if (masked) {
      const int64_t bblk = kb + lc / BBLK;
      bin = bblk >= klo && bblk < kb1;
      if (!bin) bt = ((kb1 - 1) << BSH) - 16 * lc;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(bbase + bt + (B4 && t ? boff1[i] : boff0[i]));
  };
  auto store_a = [&](int buf, bool masked) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int row = lr + RSTEP * i;
      *reinterpret_cast<u32x4 *>(&sA[buf][row * RS + 16 * lc]) = (!masked || ain) ? ra[i] : zero4;
    }
  };
  auto store_b = [&](int buf, int t, bool masked) {
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int row = t * (BN / 2) + lr + RSTEP * i;
      *reinterpret_cast<u32x4 *>(&sB[buf][row * RS + 16 * lc]) = (!masked || bin) ? rb[i] : zero4;
    }
  };

  v16f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // One K step: this step's scales from LDS, the prefetches (PA for A and the
  // scale slice, PB for B; 0 none, 1 unmasked, 2 masked), the MFMAs, then the
  // LDS stores of the prefetch and the barrier.  fp8 B follows A's step; E2M1
  // B loads half of the next pair of steps during each step of a pair.
  auto step = [&](int64_t st, auto pfa, auto pfb) {
    constexpr int PA = decltype(pfa)::value, PB = decltype(pfb)::value;
    const int buf = (int)(st & 1), sbuf = (int)((st >> 2) & 1), piece = (int)(st & 3);
    const int bbuf = B4 ? (int)((st >> 1) & 1) : buf;
    const int t = (int)(st & 1);
    const int64_t kb = kb0 + 4 * st;
    const int64_t kbn = B4 ? kb0 + 8 * ((st >> 1) + 1) : kb + 4;  // B's prefetch target
    // scale bytes of blocks kb + h (s = 0) and kb + 2 + h (s = 1): bytes
    // 4 * piece + h and 4 * piece + 2 + h of the chunk row (kb0 is a
    // multiple of 4), shifted down by h bytes into bytes 0 and 2 of one
    // register, which the MFMAs of the two halves pick with op_sel 0 and 2
    uint32_t csa[WM], csb[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
      csa[i] = *reinterpret_cast<const uint32_t *>(&sSA[sbuf][(wr0 + 32 * i + l32) * 16 + 4 * piece]) >> (8 * h);
#pragma unroll
    for (int j = 0; j < WN; ++j)
      csb[j] = *reinterpret_cast<const uint32_t *>(&sSB[sbuf][(wc0 + 32 * j + l32) * 16 + 4 * piece]) >> (8 * h);
    // the next step's global loads: with fp8 B before the first fragment
    // reads; with E2M1 B right after them, so that the reads' latency covers
    // issuing the loads (2 % faster on the MoE layer)
    auto prefetch = [&]() {
      if (PA != 0) load_a(kb + 4, PA == 2);
      if (PB != 0) load_b(kbn, B4 ? t : 0, PB == 2);
      if (PA != 0) {
        take_slice();
        load_slice(((st + 1) >> 2) + 1, (int)((st + 1) & 3));
      }
    };
    if (!B4) prefetch();

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // memory operations stay in their half; address and mask arithmetic may
      // move between the MFMAs
      __builtin_amdgcn_sched_barrier(0x6);
      v8i fa[WM], fb[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr0 + 32 * i + l32;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(&sA[buf][r * RS + 16 * (4 * s + h)]);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(&sA[buf][r * RS + 16 * (4 * s + 2 + h)]);
        fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if (B4) {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int n = wc0 + 32 * j + l32;
          const u32x4 v = *reinterpret_cast<const u32x4 *>(&sB[bbuf][n * RS + 16 * (4 * t + 2 * s + h)]);
          fb[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
        if (s == 0) prefetch();
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = s == 0 ? mfma_sel<AF, BF, 0>(fa[i], fb[j], acc[i][j], csa[i], csb[j])
                               : mfma_sel<AF, BF, 2>(fa[i], fb[j], acc[i][j], csa[i], csb[j]);
        if (s == 0 && PA == 1 && PB == 1) {
          // in this order: the fragment reads, the prefetch loads, the MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * WM + WN, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, A_LD + B_LD + 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, WM * WN, 0);
        }
      } else {
        // fp8 B fragments are 8 registers each: one at a time, so that the fp8 x
        // fp8 form stays close to the register budget
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int n = wc0 + 32 * j + l32;
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(&sB[buf][n * RS + 16 * (4 * s + h)]);
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(&sB[buf][n * RS + 16 * (4 * s + 2 + h)]);
          fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
          for (int i = 0; i < WM; ++i)
            acc[i][j] = s == 0 ? mfma_sel<AF, BF, 0>(fa[i], fb[j], acc[i][j], csa[i], csb[j])
                               : mfma_sel<AF, BF, 2>(fa[i], fb[j], acc[i][j], csa[i], csb[j]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0x6);  // keep the waits for the prefetch after the MFMAs
    if (PA != 0) store_a(buf ^ 1, PA == 2);
    if (PB != 0) store_b(bbuf ^ 1, B4 ? t : 0, PB == 2);
    if (PA != 0 || PB != 0) {
      if (PA != 0) store_slice((st >> 2) + 1, sbuf ^ 1, piece);
      __syncthreads();
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  const int64_t nsteps = (kb1 - kb0 + 3) >> 2;
  if (nsteps > 0) {
    load_a(kb0, true);
    store_a(0, true);
#pragma unroll
    for (int t = 0; t < (B4 ? 2 : 1); ++t) {
      load_b(kb0, t, true);
      store_b(0, t, true);
    }
    for (int piece = 0; piece < 4; ++piece) {
      load_slice(0, piece);
      take_slice();
      store_slice(0, 0, piece);
    }
    __syncthreads();
    load_slice(1, 0);  // stored during step 0
    int64_t st = 0;
    if (B4) {
      // only the first and the last step (A) or pair (B) can be partial: the
      // steps before the last two pairs prefetch unmasked; then straight-line
      // code for the last (up to four) steps
      const int64_t npairs = (nsteps + 1) >> 1;
      if (npairs >= 2) {
        for (; st < 2 * npairs - 4; ++st) step(st, I1{}, I1{});
        step(st++, I2{}, I2{});
        step(st++, I2{}, I2{});
      }
      if (nsteps - st == 2) step(st++, I2{}, I0{});
      step(st, I0{}, I0{});
    } else {
      for (; st + 2 < nsteps; ++st) step(st, I1{}, I1{});
      if (st + 1 < nsteps) step(st++, I2{}, I2{});
      step(st, I0{}, I0{});
    }
  }

  // ---- epilogue: row 8(v/4) + 4h + v%4, column l32 of each 32x32 tile ----
  auto store = [&](int64_t off, float v) {
    if (P.out_f32) static_cast<float *>(P.c)[off] = v;
    else static_cast<uint16_t *>(P.c)[off] = f32_to_bf16_rne(v);
  };
  const int64_t cb = cbase + m0 * P.ldc + n0;
  if (P.c16 && mlen == BM && nlen == BN) {
    // bf16 tile staged in LDS (the first half of the rows in the A buffers,
    // the second in the B buffers, rows of 2 * BN + 16 bytes) and written as
    // 16-byte row pieces: 16 stores per lane instead of 128 two-byte ones
    constexpr int OS = 2 * BN + 16, HR = BM / 2, CH = BN / 8, RPI = NT / CH;
    static_assert(HR * OS <= 2 * BM * RS && HR * OS <= 2 * BN * RS && BM % RPI == 0, "output staging");
    __syncthreads();  // every wave is past its last fragment read
    uint8_t *half = wr0 < HR ? &sA[0][0] : &sB[0][0];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (wr0 & (HR - 1)) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          *reinterpret_cast<uint16_t *>(half + r * OS + 2 * (wc0 + 32 * j + l32)) = f32_to_bf16_rne(acc[i][j][v]);
        }
    __syncthreads();
    const int ch = tid % CH;
#pragma unroll
    for (int k = 0; k < BM / RPI; ++k) {
      const int row = tid / CH + RPI * k;
      const uint8_t *src = (row < HR ? &sA[0][0] : &sB[0][0]) + (row & (HR - 1)) * OS + 16 * ch;
      // non-temporal: the output is not read again by this launch (NN / NT
      // 1-2 % faster on the MoE layer)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(src),
                                  reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(P.c) + cb + row * P.ldc + 8 * ch));
    }
  } else if (mlen == BM && nlen == BN) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wr0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          store(cb + row * P.ldc + wc0 + 32 * j + l32, acc[i][j][v]);
        }
  } else {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int col = wc0 + 32 * j + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wr0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          if (row < mlen && col < nlen) store(cb + row * P.ldc + col, acc[i][j][v]);
        }
      }
  }
}

template <int AF, int BF, bool SMALL>
hipError_t gemm_launch_one(const GemmArgs &a, int64_t grid, hipStream_t st) {
  const dim3 block(GemmShape<BF, SMALL>::threads);
  if (a.s4)
    hipLaunchKernelGGL((mxgemm_kernel<AF, BF, true, SMALL>), dim3((unsigned)grid), block, 0, st, a);
  else
    hipLaunchKernelGGL((mxgemm_kernel<AF, BF, false, SMALL>), dim3((unsigned)grid), block, 0, st, a);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int AF, int BF>
hipError_t gemm_launch(const GemmArgs &a0, hipStream_t st) {
  GemmArgs a = a0;
  constexpr int64_t BM = GemmShape<BF>::BM, BN = GemmShape<BF>::BN;
  static_assert(BM == 256 && BN == 256, "row-split tiles are 256 x 256 units");
  a.tiles_n = (a.N + BN - 1) / BN;
  if (a.group_type == 0) {
    // upper bound of the M tiles: every group adds at most one partial tile
    a.tiles_m = (a.M + BM - 1) / BM + (a.gl ? a.G : 0);
    a.total = a.tiles_m * a.tiles_n;
    if (a.total <= 0) return hipSuccess;
    if (a.total > 0x7FFFFFFF) return hipErrorInvalidValue;
    a.ncu = device_cus();
    const int64_t half = a.ncu / 2;
    // the big tiles (none when even the upper bound is a tail of at most
    // half a round), then, for rows of at most 8 N-tiles, the tail's small
    // tiles: 4 per big tile, at most half a round of big tiles (workgroups
    // without a tile return at once)
    if (a.total > half || a.tiles_n > 8) {
      const hipError_t e = gemm_launch_one<AF, BF, false>(a, a.total, st);
      if (e != hipSuccess) return e;
    }
    const int64_t small = 4 * (a.total < half ? a.total : half);
    return small > 0 && a.tiles_n <= 8 ? gemm_launch_one<AF, BF, true>(a, small, st) : hipSuccess;
  }
  a.tiles_m = (a.M + BM - 1) / BM;
  a.total = a.tiles_m * a.tiles_n * a.G;
  if (a.total <= 0) return hipSuccess;
  if (a.total > 0x7FFFFFFF) return hipErrorInvalidValue;
  return gemm_launch_one<AF, BF, false>(a, a.total, st);
}

template <int AF>
hipError_t gemm_launch_b(int bf, const GemmArgs &a, hipStream_t st) {
  switch (bf) {
    case kFmtE4M3: return gemm_launch<AF, kFmtE4M3>(a, st);
    case kFmtE5M2: return gemm_launch<AF, kFmtE5M2>(a, st);
    default: return gemm_launch<AF, kFmtE2M1>(a, st);
  }
}

}  // namespace

hipError_t launch_mx_gemm(const GemmLaunch &L, hipStream_t st) {
  GemmArgs a{};
  a.a = L.a;
  a.as = L.as;
  a.b = L.b;
  a.bs = L.bs;
  a.c = L.c;
  a.lda = L.lda;
  a.ldas = L.ldas;
  a.ldb = L.ldb;
  a.ldbs = L.ldbs;
  a.b_gs = L.b_gs;
  a.b_gss = L.b_gss;
  a.ldc = L.ldc;
  a.M = L.M;
  a.N = L.N;
  a.K = L.K;
  a.k_blocks = L.k_blocks;
  a.gl = L.group_list;
  a.G = L.num_groups;
  a.list_type = L.list_type;
  a.group_type = L.group_type;
  a.out_f32 = L.out_f32;
  a.a_sb = L.a_block == 128 ? 2 : 0;
  a.b_sb = L.b_block == 128 ? 2 : 0;
  a.s4 = ((uintptr_t)L.as % 4 == 0 && (uintptr_t)L.bs % 4 == 0 && L.ldas % 4 == 0 && L.ldbs % 4 == 0 &&
          L.b_gss % 4 == 0);
  a.c16 = !L.out_f32 && (uintptr_t)L.c % 16 == 0 && L.ldc % 8 == 0;
  return L.a_fmt == kFmtE4M3 ? gemm_launch_b<kFmtE4M3>(L.b_fmt, a, st) : gemm_launch_b<kFmtE5M2>(L.b_fmt, a, st);
}

}  // namespace mxfp4
