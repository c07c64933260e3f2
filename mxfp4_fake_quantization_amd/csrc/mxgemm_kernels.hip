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
// Work split: a 512-thread workgroup computes a 256 x 256 tile as 4 x 2
// waves of 2 x 4 MFMA tiles (two waves per SIMD, so one wave's LDS and
// address work overlaps the other's MFMAs), stepping K by 128.  Both operand
// slices go global -> registers -> LDS (double-buffered, XOR-swizzled 16-byte
// slots, conflict-free for 16- and 32-lane read phases) while the previous
// step's MFMAs run.  An E2M1 B row holds only 64 bytes per K step, half a
// 128-byte cache line; B is therefore staged two K steps at a time (one
// whole line per row, half of the tile's rows loaded during each step), so
// every B request fetches a full line.  Scale bytes travel in chunks of 32
// K-blocks per tile row (8 steps), also double-buffered in LDS and streamed
// one coalesced slice per step, so every lane reads its scale bytes with one
// LDS load per tile.  The loop body is one basic block: prefetch, MFMAs, then
// the prefetch waits and LDS stores.  Blocks outside a K range load as zero
// codes with scale 2^0; rows and columns past the tile edge load a valid
// neighbour and are not stored.
#include "mxfp4_device.h"
#include "mxfp4_groups.h"
#include "mxfp4_kernels.h"

#include <type_traits>

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 8 waves per workgroup (2 per SIMD, so one wave's LDS and address work
// overlaps the other's MFMAs): 4 x 2 waves of 2 x 4 MFMA tiles = 256 x 256.
constexpr int kWavesM = 4, kWavesN = 2, kTilesM = 2, kTilesN = 4;
constexpr int kGemmThreads = 64 * kWavesM * kWavesN;
constexpr int kBM = 32 * kTilesM * kWavesM, kBN = 32 * kTilesN * kWavesN;

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
  int64_t tiles_m, tiles_n, total;
};

// slot swizzle: conflict-free ds_read_b128 for 8 or 16 consecutive rows
__device__ __forceinline__ int swz_a(int r, int c) { return (c ^ ((r ^ (r >> 3)) & 7)) << 4; }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Workgroup id -> tile id such that each XCD (workgroups are dealt to the 8
// XCDs round-robin) runs a contiguous range of tiles and shares its L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t id, int64_t total) {
  const int64_t q = total >> 3, r = total & 7;
  const int64_t x = id & 7, loc = id >> 3;
  return x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
}

template <int AF, int BF, bool S4>
__global__ __launch_bounds__(kGemmThreads, 1) void mxgemm_kernel(GemmArgs P) {
  constexpr int WVM = kWavesM, WVN = kWavesN, WM = kTilesM, WN = kTilesN;
  constexpr int NT = kGemmThreads;
  constexpr int BM = kBM, BN = kBN;
  constexpr bool B4 = BF == kFmtE2M1;
  // B4: a 128-byte LDS row holds two K steps (pair) of E2M1 codes; fp8 B:
  // one K step.  Either way 8 slots of 16 bytes per row.
  constexpr int A_LD = BM * 8 / NT;             // 16-byte A loads per thread per step
  constexpr int RSTEP = NT / 8;                 // rows per load pass (A and B)
  constexpr int B_LD = BN * 8 / NT / (B4 ? 2 : 1);  // 16-byte B loads per thread per step
  static_assert(WVM * WVN * 64 == NT && BM == 32 * WM * WVM && BN == 32 * WN * WVN, "tile shape");
  static_assert(BM / 8 * 8 == NT / 2 && BN / 8 * 8 == NT / 2, "one scale dword per thread per step");
  __shared__ __align__(16) uint8_t sA[2][BM * 128];
  __shared__ __align__(16) uint8_t sB[2][BN * 128];
  __shared__ __align__(16) uint8_t sSA[2][BM * 32];  // scale chunks (32 K-blocks per row)
  __shared__ __align__(16) uint8_t sSB[2][BN * 32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t tile = xcd_tile(blockIdx.x, P.total);

  // ---- tile -> rows, columns, K range, operand and output bases ----
  int64_t m0, mlen, n0, kb0, kb1, klo = 0;  // steps start at kb0; blocks below klo are masked
  const uint8_t *bbase = P.b, *bsbase = P.bs;
  int64_t cbase = 0;  // element offset of the output matrix
  if (P.group_type == 0) {
    const int64_t tm = tile / P.tiles_n;
    n0 = (tile - tm * P.tiles_n) * BN;
    int g = 0;
    if (P.gl) {
      block_row_uniform<false>(P.gl, P.G, P.list_type, P.M, __builtin_ctz(BM), tm, &m0, &mlen, &g);
    } else {
      m0 = tm * BM;
      mlen = P.M - m0 < BM ? P.M - m0 : BM;
    }
    if (mlen <= 0) return;  // past the groups' total (workgroup-uniform)
    bbase += (int64_t)g * P.b_gs;
    bsbase += (int64_t)g * P.b_gss;
    kb0 = 0;
    kb1 = (P.K + 31) >> 5;
  } else {
    const int64_t per = P.tiles_m * P.tiles_n;
    const int g = (int)(tile / per);
    const int64_t r = tile - (int64_t)g * per;
    const int64_t tm = r / P.tiles_n;
    m0 = tm * BM;
    mlen = P.M - m0 < BM ? P.M - m0 : BM;
    n0 = (r - tm * P.tiles_n) * BN;
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
  uint32_t aoff[A_LD], boff[B4 ? 2 : 1][B_LD];
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
      boff[t][i] = (uint32_t)((row < nlen ? row : nlen - 1) * P.ldb) + 16 * lc;
    }
  const int wr0 = (wave / WVN) * 32 * WM, wc0 = (wave % WVN) * 32 * WN;

  // ---- scale bytes: chunks of 32 K-blocks (8 steps) staged in LDS ----
  // Chunk c holds, for every tile row, the scale bytes of blocks
  // [kb0 + 32c, kb0 + 32c + 32) (32 bytes, or 8 for 128-element blocks).
  // While chunk c is in use, chunk c + 1 arrives one 1/8 slice per step:
  // step 8c + p loads rows [32p, 32p + 32) of A (waves of the first half) or
  // of B (second half), one dword per thread, 8 threads per 32-byte row.
  // Bytes outside [klo, kb1) are replaced by 127 (2^0) when stored, so the
  // MFMAs of masked blocks (zero codes) see a finite scale.
  const bool sl_b = tid >= NT / 2;
  const int sr = (tid & (NT / 2 - 1)) >> 3, sd = tid & 7;
  const int sb_log = sl_b ? P.b_sb : P.a_sb;
  const int64_t s_lo = klo >> sb_log;                                   // first valid byte
  const int64_t s_hi = (kb1 + (1 << sb_log) - 1) >> sb_log;            // past the last
  const uint8_t *s_base = sl_b ? bsbase : asbase;
  const int64_t s_ld = sl_b ? P.ldbs : P.ldas;
  const int64_t s_rows = sl_b ? nlen : mlen;
  uint32_t pv[S4 ? 1 : 4];
  int64_t pbyte = 0;
  auto load_slice = [&](int64_t chunk, int piece) {
    const int row = piece * 32 + sr;
    pbyte = ((kb0 + 32 * chunk) >> sb_log) + 4 * sd;
    const uint8_t *rp = s_base + (int64_t)(row < s_rows ? row : s_rows - 1) * s_ld;
    const int64_t at = pbyte < s_hi ? pbyte : s_hi - 1;  // in bounds (s_hi <= row length)
    if (S4) {
      pv[0] = *reinterpret_cast<const uint32_t *>(rp + (at & ~(int64_t)3));
    } else {
#pragma unroll
      for (int e = 0; e < (S4 ? 1 : 4); ++e) pv[e] = rp[at + e < s_hi ? at + e : s_hi - 1];
    }
  };
  auto store_slice = [&](int sbuf, int piece) {
    uint32_t v = pv[0];
    if (!S4) {
#pragma unroll
      for (int e = 1; e < (S4 ? 1 : 4); ++e) v |= pv[e] << (8 * e);
    }
    // keep bytes pbyte + e inside [s_lo, s_hi) and inside the chunk
    const int64_t lead = s_lo - pbyte, cnt = s_hi - pbyte;
    const int nlead = lead <= 0 ? 0 : (lead >= 4 ? 4 : (int)lead);
    int nval = cnt <= 0 ? 0 : (cnt >= 4 ? 4 : (int)cnt);
    if (4 * sd >= (32 >> sb_log)) nval = 0;
    const uint32_t hi_m = nval >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nval)) - 1u);
    const uint32_t lo_m = nlead >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nlead)) - 1u);
    const uint32_t keep = hi_m & ~lo_m;
    v = (v & keep) | (0x7F7F7F7Fu & ~keep);
    uint8_t *dst = sl_b ? &sSB[sbuf][0] : &sSA[sbuf][0];
    *reinterpret_cast<uint32_t *>(dst + (piece * 32 + sr) * 32 + 4 * sd) = v;
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
    for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(bbase + bt + boff[t][i]);
  };
  auto store_a = [&](int buf, bool masked) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int row = lr + RSTEP * i;
      *reinterpret_cast<u32x4 *>(&sA[buf][row * 128 + swz_a(row, lc)]) = (!masked || ain) ? ra[i] : zero4;
    }
  };
  auto store_b = [&](int buf, int t, bool masked) {
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int row = t * (BN / 2) + lr + RSTEP * i;
      *reinterpret_cast<u32x4 *>(&sB[buf][row * 128 + swz_a(row, lc)]) = (!masked || bin) ? rb[i] : zero4;
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
    const int buf = (int)(st & 1), sbuf = (int)((st >> 3) & 1), piece = (int)(st & 7);
    const int bbuf = B4 ? (int)((st >> 1) & 1) : buf;
    const int t = (int)(st & 1);
    const int64_t kb = kb0 + 4 * st;
    const int64_t kbn = B4 ? kb0 + 8 * ((st >> 1) + 1) : kb + 4;  // B's prefetch target
    // scale bytes of blocks kb + h (s = 0) and kb + 2 + h (s = 1)
    uint32_t csa[WM][2], csb[WN][2];
    {
      const int64_t ca = (kb0 + 32 * (st >> 3)) >> P.a_sb, cb = (kb0 + 32 * (st >> 3)) >> P.b_sb;
      const int qa0 = (int)(((kb + h) >> P.a_sb) - ca), qa1 = (int)(((kb + 2 + h) >> P.a_sb) - ca);
      const int qb0 = (int)(((kb + h) >> P.b_sb) - cb), qb1 = (int)(((kb + 2 + h) >> P.b_sb) - cb);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(&sSA[sbuf][(wr0 + 32 * i + l32) * 32 + (qa0 & ~3)]);
        csa[i][0] = (w >> (8 * (qa0 & 3))) & 0xFFu;
        csa[i][1] = (w >> (8 * (qa1 & 3))) & 0xFFu;
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(&sSB[sbuf][(wc0 + 32 * j + l32) * 32 + (qb0 & ~3)]);
        csb[j][0] = (w >> (8 * (qb0 & 3))) & 0xFFu;
        csb[j][1] = (w >> (8 * (qb1 & 3))) & 0xFFu;
      }
    }
    if (PA != 0) load_a(kb + 4, PA == 2);
    if (PB != 0) load_b(kbn, B4 ? t : 0, PB == 2);
    if (PA != 0) load_slice((st >> 3) + 1, piece);

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      v8i fa[WM], fb[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int r = wr0 + 32 * i + l32;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(&sA[buf][r * 128 + swz_a(r, 4 * s + h)]);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(&sA[buf][r * 128 + swz_a(r, 4 * s + 2 + h)]);
        fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if (B4) {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int n = wc0 + 32 * j + l32;
          const u32x4 v = *reinterpret_cast<const u32x4 *>(&sB[bbuf][n * 128 + swz_a(n, 4 * t + 2 * s + h)]);
          fb[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], AF, BF, 0,
                                                                        (int)csa[i][s], 0, (int)csb[j][s]);
      } else {
        // fp8 B fragments are 8 registers each: one at a time, so that the fp8 x
        // fp8 form stays close to the register budget
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const int n = wc0 + 32 * j + l32;
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(&sB[buf][n * 128 + swz_a(n, 4 * s + h)]);
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(&sB[buf][n * 128 + swz_a(n, 4 * s + 2 + h)]);
          fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
          for (int i = 0; i < WM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], AF, BF, 0,
                                                                        (int)csa[i][s], 0, (int)csb[j][s]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the waits for the prefetch after the MFMAs
    if (PA != 0) store_a(buf ^ 1, PA == 2);
    if (PB != 0) store_b(bbuf ^ 1, B4 ? t : 0, PB == 2);
    if (PA != 0 || PB != 0) {
      if (PA != 0) store_slice(sbuf ^ 1, piece);
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
    for (int piece = 0; piece < 8; ++piece) {
      load_slice(0, piece);
      store_slice(0, piece);
    }
    __syncthreads();
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
  if (mlen == BM && nlen == BN) {
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

template <int AF, int BF>
hipError_t gemm_launch(const GemmArgs &a0, hipStream_t st) {
  GemmArgs a = a0;
  const int64_t BM = kBM, BN = kBN;
  a.tiles_n = (a.N + BN - 1) / BN;
  if (a.group_type == 0) {
    // upper bound of the M tiles: every group adds at most one partial tile
    a.tiles_m = (a.M + BM - 1) / BM + (a.gl ? a.G : 0);
    a.total = a.tiles_m * a.tiles_n;
  } else {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.total = a.tiles_m * a.tiles_n * a.G;
  }
  if (a.total <= 0) return hipSuccess;
  if (a.total > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.s4)
    hipLaunchKernelGGL((mxgemm_kernel<AF, BF, true>), dim3((unsigned)a.total), dim3(kGemmThreads), 0, st, a);
  else
    hipLaunchKernelGGL((mxgemm_kernel<AF, BF, false>), dim3((unsigned)a.total), dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
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
  return L.a_fmt == kFmtE4M3 ? gemm_launch_b<kFmtE4M3>(L.b_fmt, a, st) : gemm_launch_b<kFmtE5M2>(L.b_fmt, a, st);
}

}  // namespace mxfp4
