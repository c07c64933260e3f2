// kmajor_kernels.hip -- packed MXFP4 operands laid out along the reduction
// dimension, and decoding of packed codes back to values, on gfx950.
//
// K-major pack: column-wise (or per-expert grouped) blocks of x [rows, cols]
// are quantized and stored as the row-wise packed form of x^T: codes_t
// [cols, k_blocks * block / 2] (two FP4 codes per byte, the lower K position
// in the low nibble) and scales_t [cols, k_blocks] E8M0 bytes.  This is the
// column-direction operand (col_data / col_scale) of the hyper-parallel
// page's grouped W4A8 matmul, stored packed as on the sglang page, so an MX
// matrix product reads each column's blocks as contiguous 16-byte (block 32)
// or 64-byte (block 128) pieces along K.  K position t*block + o is x row
// start_t + o of block-row t while o < len_t, else a padding code 0.
//
// Tiling: a workgroup (8 waves) owns 256 K positions x 16 CPL columns, CPL
// = 8 columns per lane for bf16 and 4 for fp32 (one 16-byte piece per row
// either way).  Lane (cg, rq), with cg = lane & 15 and rq = 4*wave + (lane >>
// 4), holds K positions 8rq .. 8rq+7 (8 consecutive rows of x, inside one
// block-row) of columns CPL*cg .. CPL*cg + CPL-1, loaded as one 16-byte piece
// per row, so 16 lanes read a 256-byte row segment.  Then
//   - a 32-row block is one wave (lanes at distance 16): column max by
//     ds_swizzle xor 16 and ds_bpermute xor 32; a 128-row block spans 4 waves,
//     which combine their maxima through LDS;
//   - the 8 nibbles of one column in one lane form one 32-bit word at byte
//     4*rq of the column's 128-byte line of codes (CPL words per lane); the words are staged in LDS
//     and each line of codes_t is written whole, by 8 lanes with 16-byte
//     stores.
//
// Decode: codes [rows, ceil(cols/2)] + scales [rows, ceil(cols/block)] ->
// values [rows, cols] in bf16 or fp32; K-major codes decode with rows = the
// columns of x and cols = k_blocks * block.
#include "mxfp4_device.h"
#include "mxfp4_groups.h"
#include "mxfp4_kernels.h"

namespace mxfp4 {
namespace {

constexpr int kKTile = 256;      // K positions per workgroup
// Workgroup = 256 K positions x 128 columns per half (8 waves per half, each
// 32 K positions x 128 columns); bf16 block 32 takes two halves (256-byte
// row segments read as 512-byte ones: +2-5 % measured on MI355X), the other
// forms one (block 128 measured equal or slower with two).
template <int DT, int B>
struct KmShape {
  static constexpr int cpl = DT == kBF16 ? 8 : 4;     // columns per lane (16 bytes of a row)
  static constexpr int lcpl = DT == kBF16 ? 3 : 2;    // log2(cpl)
  static constexpr int halves = DT == kBF16 && B == 32 ? 2 : 1;
  static constexpr int chalf = 16 * cpl;              // columns per half
  static constexpr int ctile = chalf * halves;        // columns per workgroup
  static constexpr int threads = 512 * halves;
};
// A lane's row piece: 16 bytes = 4 words (two bf16 columns or one fp32
// column per word).
constexpr int kKmNW = 4;

// Columns c0 .. c0 + n - 1 of one row (n <= CPL) into 4 words; zeros past n.
// VEC (16-byte aligned pieces, whole column groups): n is CPL or 0.
template <int DT, bool VEC>
__device__ __forceinline__ void load_row16(uint32_t (&w)[kKmNW], const uint8_t *p, int n) {
  constexpr int CPL = DT == kBF16 ? 8 : 4;
  if (VEC && n == CPL) {
    const uint4 v = ld16(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    return;
  }
#pragma unroll
  for (int k = 0; k < kKmNW; ++k) w[k] = 0;
  if (!VEC) {
    for (int j = 0; j < n; ++j) {
      if (DT == kBF16) w[j >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(p)[j] << (16 * (j & 1));
      else w[j] = reinterpret_cast<const uint32_t *>(p)[j];
    }
  }
}
// Minimum waves per SIMD requested from the compiler: 8 (64 VGPRs, four
// 8-wave workgroups per CU) for bf16 FLOOR, whose common path fits in 64
// registers (only the generic snap of tiny blocks spills); 4 (128 VGPRs, two
// workgroups per CU) for the rest, whose common path would spill.  Measured
// on MI355X: +5-7 % for bf16 block 128 and grouped tokens, equal for block 32.
#ifndef MXFP4_KMAJOR_MINWG
#define MXFP4_KMAJOR_MINWG 4
#endif
#ifndef MXFP4_KMAJOR_MINWG_BF16_FLOOR
#define MXFP4_KMAJOR_MINWG_BF16_FLOOR 8
#endif
// 8-element chunks per lane of the flat decode kernel.
#ifndef MXFP4_DQ_U
#define MXFP4_DQ_U 2
#endif

struct KmArgs {
  const uint8_t *x;
  uint8_t *codes;   // [cols, ldk]
  uint8_t *scales;  // [cols, k_blocks]
  const int64_t *group_list;
  int64_t rows, cols, k_blocks, ldk;
  int64_t nct;     // column tiles
  int64_t ntiles;  // K tiles x column tiles
  int num_groups, list_type;
  float sf;
};

// Nibbles of a word of two bf16 columns, with the generic snap for a half
// whose column max needs it (FLOOR E8M0 byte 0..2).
__device__ __forceinline__ uint32_t fix_slow_nib(uint32_t w, uint32_t cm, uint32_t e8p, uint32_t n) {
  const uint32_t lo = cm & 0xFFFFu, hi = cm >> 16;
  if (lo != 0 && (lo >> 7) < 5) n = (n & 0xFFFF0000u) | half_bf16_slow(w & 0xFFFFu, e8p & 0xFFu).n;
  if (hi != 0 && (hi >> 7) < 5) n = (n & 0xFFFFu) | (half_bf16_slow(w >> 16, (e8p >> 16) & 0xFFu).n << 16);
  return n;
}

// Generic-snap nibbles of 8 fp32 rows of one column (E8M0 byte 0..2).  Out
// of line: inlined for all 64 elements of a lane it would spill; it runs
// only after every load of the lane has been consumed.
__device__ __noinline__ uint32_t slow_column_f32(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                 uint32_t a4, uint32_t a5, uint32_t a6, uint32_t a7,
                                                 uint32_t e8) {
  const uint32_t a[8] = {a0, a1, a2, a3, a4, a5, a6, a7};
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t idx;
    slow_snap<kF32>(a[i] & 0x7FFFFFFFu, e8, &idx);
    v |= (idx | (sign_f32(a[i], 0x7FFFFFFFu) >> 28)) << (4 * i);  // FLOOR sign rule
  }
  return v;
}

// The lane's code words (one per column: 8 for bf16, 4 for fp32; K position
// 8rq + i in bits 4i..4i+3).  SLOW = true only when some lane of the wave
// holds a column that needs the generic snap.
template <int DT, int RULE, bool SLOW>
__device__ __forceinline__ void code_words(const uint32_t (&w)[8][kKmNW], const uint32_t *pt,
                                           const uint32_t *pz, const uint32_t *pe, const uint32_t *cm,
                                           const BlockParams *cbp, uint32_t (&out)[8]) {
  if (DT == kBF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t t31 = pt[k] - 0x001F001Fu;
      uint32_t acc[2];  // rows 0-3 / 4-7; column 2k in bits 0-15, 2k+1 in 16-31
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        // nibble of row 4g + r at bits 12-15 / 28-31, shifted into place below
        uint32_t t[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t x = w[4 * g + r][k];
          if (SLOW && RULE == kFloor)
            t[r] = fix_slow_nib(x, cm[k], pe[k], n_bf16(x, pt[k], pz[k])) << 12;
          else
            t[r] = (snap_idx_bf16_tab(x & 0x7FFF7FFFu, t31) << 12) |
                   (RULE == kFloor ? sign_bf16_floor(x) : sign_bf16(x, pz[k]));
        }
        acc[g] = (t[0] >> 12) | (t[1] >> 8) | (t[2] >> 4) | t[3];
      }
      out[2 * k] = perm_b32(acc[1], acc[0], 0x05040100u);      // low halves
      out[2 * k + 1] = perm_b32(acc[1], acc[0], 0x07060302u);  // high halves
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      BlockParams q = cbp[k];
      q.slow = false;
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) v |= n_f32(w[i][k], q) << (4 * i);
      if (SLOW && cbp[k].slow)
        v = slow_column_f32(w[0][k], w[1][k], w[2][k], w[3][k], w[4][k], w[5][k], w[6][k], w[7][k],
                            cbp[k].e8);
      out[k] = v;
    }
  }
}

template <int DT>
__device__ __forceinline__ uint32_t colmax_step(uint32_t a, uint32_t b) {
  return DT == kBF16 ? pk_max(a, b) : max32(a, b);
}

// Where one lane's piece of a tile lives.
struct KmTile {
  const uint8_t *src;  // first of its 8 rows at its first column
  int64_t kt, col0;    // tile: K tile and first column
  int64_t kpos;        // first K position of the lane
  int64_t bt;          // its block-row
  int64_t c0;          // its first column
  int o0;              // offset of kpos inside the block
  int nrow, ncol;      // rows / columns of the 8 x 8 piece inside the tensor
  bool live;           // the block-row exists (every lane of it writes)
  bool full;           // wave-uniform: all rows and the whole column tile inside
};

template <int DT, int B, bool GROUPED, bool VEC>
__device__ __forceinline__ KmTile km_tile(const KmArgs &A, int64_t tile, int wave, int chalf, int rql, int cg) {
  constexpr int ES = PieceT<DT>::ES;
  constexpr int kCTile = KmShape<DT, B>::ctile;
  constexpr int LB = B == 32 ? 5 : 7;
  KmTile T;
  T.kt = tile / A.nct;
  T.col0 = (tile - T.kt * A.nct) * kCTile;
  T.kpos = T.kt * kKTile + 8 * (4 * wave + rql);
  T.bt = T.kpos >> LB;
  T.o0 = (int)(T.kpos & (B - 1));
  int64_t start, len;
  if (GROUPED) {
    // a wave covers 32 K positions: one block-row, the same for every lane
    block_row_uniform(A.group_list, A.num_groups, A.list_type, A.rows, LB, T.bt, &start, &len);
    if (T.bt >= A.k_blocks) len = 0;
  } else {
    start = T.bt << LB;
    const int64_t rem = A.rows - start;
    len = rem <= 0 ? 0 : (rem < B ? rem : B);
  }
  constexpr int CPL = KmShape<DT, B>::cpl;
  T.c0 = T.col0 + KmShape<DT, B>::chalf * chalf + CPL * cg;
  const int64_t crem = A.cols - T.c0;
  T.ncol = crem >= CPL ? CPL : (crem > 0 ? (int)crem : 0);
  const int64_t rrem = len - T.o0;
  T.nrow = rrem >= 8 ? 8 : (rrem > 0 ? (int)rrem : 0);
  T.live = len > 0;
  T.src = A.x + ((start + T.o0) * A.cols + T.c0) * ES;
  T.full = VEC && T.col0 + kCTile <= A.cols && __all(T.nrow == 8);
  return T;
}

// LDS staging of one tile's outputs.  With g = c >> LC the column group of
// column c (LC = log2 of the columns per lane), the 16-byte chunk q (K words
// 4q .. 4q + 3) of column c's row sits at chunk slot q ^ (g & 7) of the row,
// and inside the chunk word i sits at i ^ (2 * ((g >> 3) & 1)).  A staging
// write stores one word per lane for lanes (cg = column group 0..15, K word
// 4 * wave + rql): the XOR with the group's low three bits spreads the eight
// groups of a half-wave over the eight chunk slots, the XOR with its fourth
// bit puts groups cg and cg + 8 on different words of the chunk, so each
// half-wave's 32 words fall in 32 different banks.  The 8 lanes that read
// one column's row (ds_read_b128) cover its 32 words, so all banks, and swap
// the halves back where bit 3 of the group is set.  Scale bytes are staged
// block-row major ([block-row][column]): a lane writes its columns' bytes
// with one 8-byte (bf16) or 4-byte (fp32) store, 16 lanes consecutive bytes.
template <int CT>
struct KmStage {
  uint32_t codes[CT][kKTile / 8] __attribute__((aligned(16)));
  uint8_t scales[kKTile / 32][CT] __attribute__((aligned(16)));
  uint8_t live[kKTile / 32];
};

template <int LC>
__device__ __forceinline__ int km_chunk(int c, int q) { return c * (kKTile / 8) + 4 * (q ^ ((c >> LC) & 7)); }
template <int LC>
__device__ __forceinline__ int km_slot(int c, int kw) {
  return km_chunk<LC>(c, kw >> 2) + ((kw & 3) ^ (((c >> (LC + 3)) & 1) << 1));
}

// One workgroup per tile: load, column maxima, nibbles; then the tile's
// outputs go through LDS so that 8 lanes store each column's 128-byte line of
// codes with 16-byte stores and one lane its scale bytes (8 for block 32) in
// one store, instead of 4-byte and 1-byte pieces scattered by row lanes.
template <int DT, int B, int RULE, bool GROUPED, bool VEC>
__global__ __launch_bounds__((KmShape<DT, B>::threads),
                             (DT == kBF16 && RULE == kFloor ? MXFP4_KMAJOR_MINWG_BF16_FLOOR : MXFP4_KMAJOR_MINWG))
void kmajor_pack_kernel(KmArgs A) {
  constexpr int kCTile = KmShape<DT, B>::ctile;
  constexpr int kKmThreads = KmShape<DT, B>::threads;
  constexpr int NW = kKmNW;
  constexpr int ES = PieceT<DT>::ES;
  constexpr int CPL = KmShape<DT, B>::cpl, LC = KmShape<DT, B>::lcpl;
  constexpr uint32_t ABS = DT == kBF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
  constexpr int NBT_TILE = kKTile / B;  // block-rows per tile
  __shared__ uint32_t s_cm[kKmThreads / 64][NW][16];  // [wave][word][column group]: no bank conflicts
  __shared__ KmStage<kCTile> st;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int kwave = wave & 7;   // K slice of the wave (32 positions)
  const int chalf = wave >> 3;  // its 128-column half of the tile
  const int lane = tid & 63;
  const int cg = lane & 15;
  const int rql = lane >> 4;
  const KmTile T = km_tile<DT, B, GROUPED, VEC>(A, blockIdx.x, kwave, chalf, rql, cg);

  // ---- load 8 rows x 8 columns --------------------------------------------
  // A wave whose piece is all inside the tensor issues its eight loads
  // unconditionally, so they are all in flight together; 16 lanes read one
  // 256-byte (bf16) row segment.
  const int64_t rstride = A.cols * ES;
  uint32_t w[8][NW];
  if (T.full) {
#pragma unroll
    for (int i = 0; i < 8; ++i) load_row16<DT, true>(w[i], T.src + i * rstride, CPL);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) load_row16<DT, VEC>(w[i], T.src + i * rstride, i < T.nrow ? T.ncol : 0);
  }

  // ---- column maxima (padding rows read as +0 and never raise them) -------
  // a 32-row block is the wave's 4 lane rows (lanes cg, cg+16, cg+32, cg+48);
  // a 128-row block is 4 consecutive waves, combined through LDS
  uint32_t cm[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = colmax_step<DT>(m, w[i][k] & ABS);
    m = colmax_step<DT>(m, lane_xor16(m));
    m = colmax_step<DT>(m, lane_xor32(m));
    cm[k] = m;
  }
  if (B == 128) {
    if (rql == 0) {
#pragma unroll
      for (int k = 0; k < NW; ++k) s_cm[wave][k][cg] = cm[k];
    }
    __syncthreads();
    const int w0 = wave & ~3;
#pragma unroll
    for (int k = 0; k < NW; ++k)
      cm[k] = colmax_step<DT>(colmax_step<DT>(s_cm[w0][k][cg], s_cm[w0 + 1][k][cg]),
                              colmax_step<DT>(s_cm[w0 + 2][k][cg], s_cm[w0 + 3][k][cg]));
  }

  // ---- per-column parameters ---------------------------------------------
  uint32_t pt[NW], pz[NW], pe[NW];
  BlockParams cbp[DT == kF32 ? 4 : 1];
  bool slow_any = false;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (DT == kBF16 && RULE == kFloor) {
      const PackedParams q = floor_params_pk(cm[k]);
      pt[k] = q.t2;
      pz[k] = 0x7FFF7FFFu;
      pe[k] = q.e8;
      slow_any = slow_any || q.slow;
    } else if (DT == kBF16) {
      const BlockParams lo = block_params<DT, RULE>(cm[k] & 0xFFFFu, A.sf);
      const BlockParams hi = block_params<DT, RULE>(cm[k] >> 16, A.sf);
      pt[k] = lo.t025 | (hi.t025 << 16);
      pz[k] = lo.zc | (hi.zc << 16);
      pe[k] = lo.e8 | (hi.e8 << 16);
    } else {
      cbp[DT == kF32 ? k : 0] = block_params<DT, RULE>(cm[k], A.sf);
      pe[k] = cbp[DT == kF32 ? k : 0].e8;
      slow_any = slow_any || cbp[DT == kF32 ? k : 0].slow;
    }
  }

  // the E8M0 bytes of the lane's 8 columns, in column order (packed before
  // the code words so the per-column bytes need no registers meanwhile)
  uint32_t sc_lo, sc_hi = 0;
  if (DT == kBF16) {
    sc_lo = perm_b32(pe[1], pe[0], 0x06040200u);  // bytes 0 and 2 of each packed word
    sc_hi = perm_b32(pe[3], pe[2], 0x06040200u);
  } else {
    sc_lo = pe[0] | (pe[1] << 8) | (pe[2] << 16) | (pe[3] << 24);
  }

  uint32_t cw[8];
  if (__builtin_expect(__any(slow_any), 0)) code_words<DT, RULE, true>(w, pt, pz, pe, cm, cbp, cw);
  else code_words<DT, RULE, false>(w, pt, pz, pe, cm, cbp, cw);

  // ---- stage in LDS ----------------------------------------------------------
  const int kw = 4 * kwave + rql;  // K word of the lane inside the tile
  const int bl = (8 * kw) / B;    // block-row of the lane inside the tile
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    (&st.codes[0][0])[km_slot<LC>(KmShape<DT, B>::chalf * chalf + CPL * cg + j, kw)] = cw[j];
  if (T.o0 == 0) {
    uint8_t *sp = &st.scales[bl][KmShape<DT, B>::chalf * chalf + CPL * cg];
    if (DT == kBF16) *reinterpret_cast<uint2 *>(sp) = make_uint2(sc_lo, sc_hi);
    else *reinterpret_cast<uint32_t *>(sp) = sc_lo;
    if (cg == 0) st.live[bl] = T.live;
  }
  __syncthreads();

  // ---- stores ------------------------------------------------------------------
  // 8 consecutive lanes write one column's 128 bytes of codes (a 16-byte chunk
  // is 32 K positions, inside one block-row); a block-row past the blocking's
  // end is not written.
  const int64_t kbyte = T.kt * (kKTile / 2);
#pragma unroll
  for (int r = 0; r < (kCTile * kKTile / 32) / kKmThreads; ++r) {
    const int chunk = tid + r * kKmThreads;
    const int c = chunk >> 3, q = chunk & 7;
    const int64_t col = T.col0 + c;
    if (col < A.cols && st.live[(32 * q) / B]) {
      uint4 v = *reinterpret_cast<const uint4 *>(&(&st.codes[0][0])[km_chunk<LC>(c, q)]);
      if ((c >> (LC + 3)) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
      st16(A.codes + col * A.ldk + kbyte + 16 * q, v);
    }
  }
  if (tid < kCTile && T.col0 + tid < A.cols) {
    uint8_t *sd = A.scales + (T.col0 + tid) * A.k_blocks + T.kt * NBT_TILE;
    bool all_live = true;
#pragma unroll
    for (int b = 0; b < NBT_TILE; ++b) all_live = all_live && st.live[b];
    if (NBT_TILE == 8 && all_live && ((uintptr_t)sd & 7) == 0) {
      uint64_t v = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) v |= (uint64_t)st.scales[b][tid] << (8 * b);
      *reinterpret_cast<uint64_t *>(sd) = v;
    } else {
#pragma unroll
      for (int b = 0; b < NBT_TILE; ++b)
        if (st.live[b]) sd[b] = st.scales[b][tid];
    }
  }
}

template <int DT, int B, int RULE, bool GROUPED>
hipError_t km_launch(bool vec, const KmArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)a.ntiles);
  if (vec)
    hipLaunchKernelGGL((kmajor_pack_kernel<DT, B, RULE, GROUPED, true>), grid, dim3(KmShape<DT, B>::threads), 0, st, a);
  else
    hipLaunchKernelGGL((kmajor_pack_kernel<DT, B, RULE, GROUPED, false>), grid, dim3(KmShape<DT, B>::threads), 0, st, a);
  return hipGetLastError();
}

template <int DT, int B>
hipError_t km_rule(int rule, bool grouped, bool vec, const KmArgs &a, hipStream_t st) {
  if (rule == kFloor)
    return grouped ? km_launch<DT, B, kFloor, true>(vec, a, st) : km_launch<DT, B, kFloor, false>(vec, a, st);
  return grouped ? km_launch<DT, B, kAmct, true>(vec, a, st) : km_launch<DT, B, kAmct, false>(vec, a, st);
}

// ---- decode ------------------------------------------------------------------

struct DqArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  uint8_t *y;
  int64_t rows, cols;
  int64_t half;     // code bytes per row, ceil(cols / 2)
  int64_t nb;       // scale bytes per row, ceil(cols / block)
  int64_t nchunks;  // flat kernel: rows * cols / 8
  int64_t nxr;      // row kernel: workgroups per row
};

// Eight values (four words; element 2d in the low half of word d) of the code
// word c (element j in bits 4j..4j+3), E8M0 byte e8.  Closed form for
// 2 <= e8 <= 252, where every code times 2^(e8-127) is a normal bf16: for
// code index i >= 1 the magnitude bits are (e8-1)*128 + 64*t(i), t = [-, 0, 2,
// 3, 4, 5, 6, 7] (one byte-table lookup by v_perm), and 0 for i = 0.
// SLOW: lanes with other bytes recompute with the generic form.
template <bool SLOW>
__device__ __forceinline__ void decode8(uint32_t c, uint32_t e8, uint32_t (&y)[4]) {
  const uint32_t ev = c & 0x0F0F0F0Fu;         // elements 0 2 4 6
  const uint32_t od = (c >> 4) & 0x0F0F0F0Fu;  // elements 1 3 5 7
  const uint32_t e2 = splat16(((e8 - 1u) & 0x1FFu) << 7);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // byte d of ev -> low half, byte d of od -> high half
    const uint32_t n2 = __builtin_amdgcn_perm(od, ev, (0x0Cu << 24) | ((4u + d) << 16) | (0x0Cu << 8) | d);
    const uint32_t i2 = n2 & 0x00070007u;
    const uint32_t q2 = __builtin_amdgcn_perm(0x07060504u, 0x03020000u, i2);
    const uint32_t ze = pk_mad(pk_min1(i2), e2, 0u);
    y[d] = pk_mad(q2, 0x00400040u, ze) | ((n2 << 12) & 0x80008000u);
  }
  if (SLOW && (e8 - 2u) > 250u) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t b = (c >> (8 * d)) & 0xFFu;
      y[d] = decode_bf16_generic(b & 15u, e8) | (decode_bf16_generic(b >> 4, e8) << 16);
    }
  }
}

template <int DT>
__device__ __forceinline__ void store_chunk(uint8_t *p, const uint32_t (&y)[4]) {
  if (DT == kBF16) {
    st16(p, make_uint4(y[0], y[1], y[2], y[3]));
  } else {
    st16(p, make_uint4(y[0] << 16, y[0] & 0xFFFF0000u, y[1] << 16, y[1] & 0xFFFF0000u));
    st16(p + 16, make_uint4(y[2] << 16, y[2] & 0xFFFF0000u, y[3] << 16, y[3] & 0xFFFF0000u));
  }
}

// cols % block == 0: code word ch covers elements 8ch .. 8ch+7 of the flat
// tensor, whose block is 8ch / block.
template <int DT, int LB, int U>
__global__ __launch_bounds__(kThreads) void dequant_flat_kernel(DqArgs A) {
  constexpr int ES = PieceT<DT>::ES;
  const int64_t base = (int64_t)blockIdx.x * (U * kThreads) + threadIdx.x;
  const bool full = (int64_t)(blockIdx.x + 1) * (U * kThreads) <= A.nchunks;  // workgroup-uniform
  const uint32_t *cw = reinterpret_cast<const uint32_t *>(A.codes);
  uint32_t c[U], e[U];
  bool slow = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t ch = base + u * kThreads;
    c[u] = 0;
    e[u] = 127;
    if (full || ch < A.nchunks) {
      c[u] = __builtin_nontemporal_load(cw + ch);
      e[u] = A.scales[(ch << 3) >> LB];
    }
    slow = slow || (e[u] - 2u) > 250u;
  }
  const bool any_slow = __any(slow);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t ch = base + u * kThreads;
    uint32_t y[4];
    if (__builtin_expect(any_slow, 0)) decode8<true>(c[u], e[u], y);
    else decode8<false>(c[u], e[u], y);
    if (full || ch < A.nchunks) store_chunk<DT>(A.y + ch * (8 * ES), y);
  }
}

// Any cols: workgroup = one row segment of 256 chunks of 8 elements (a chunk
// never straddles a block: blocks are multiples of 8 within the row).
template <int DT, int LB, bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(DqArgs A) {
  constexpr int ES = PieceT<DT>::ES;
  const int64_t row = blockIdx.x / A.nxr;
  const int64_t col = ((blockIdx.x - row * A.nxr) * kThreads + threadIdx.x) * 8;
  if (col >= A.cols) return;
  const uint8_t *crow = A.codes + row * A.half;
  const uint32_t e8 = A.scales[row * A.nb + (col >> LB)];
  uint8_t *yrow = A.y + row * A.cols * ES;
  if (VEC) {  // cols % 8 == 0: a whole aligned chunk
    uint32_t y[4];
    decode8<true>(*reinterpret_cast<const uint32_t *>(crow + (col >> 1)), e8, y);
    store_chunk<DT>(yrow + col * ES, y);
  } else {
    for (int j = 0; j < 8 && col + j < A.cols; ++j) {
      const uint32_t b = crow[(col + j) >> 1];
      const uint32_t v = decode_bf16_generic(((col + j) & 1) ? b >> 4 : b & 15u, e8);
      if (DT == kBF16) reinterpret_cast<uint16_t *>(yrow)[col + j] = (uint16_t)v;
      else reinterpret_cast<uint32_t *>(yrow)[col + j] = v << 16;
    }
  }
}

template <int DT, int LB>
hipError_t dq_launch(const DqArgs &a0, hipStream_t st) {
  DqArgs a = a0;
  constexpr int U = MXFP4_DQ_U;
  if (a.cols % (1 << LB) == 0) {
    a.nchunks = a.rows * a.cols / 8;
    const int64_t nwg = (a.nchunks + U * kThreads - 1) / (U * kThreads);
    if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dequant_flat_kernel<DT, LB, U>), dim3((unsigned)nwg), dim3(kThreads), 0, st, a);
  } else {
    a.nxr = (a.cols + 8 * kThreads - 1) / (8 * kThreads);
    const int64_t nwg = a.rows * a.nxr;
    if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.cols % 8 == 0)
      hipLaunchKernelGGL((dequant_rows_kernel<DT, LB, true>), dim3((unsigned)nwg), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((dequant_rows_kernel<DT, LB, false>), dim3((unsigned)nwg), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kmajor_pack(const KmLaunch &L, hipStream_t st) {
  KmArgs a;
  a.x = static_cast<const uint8_t *>(L.x);
  a.codes = L.codes;
  a.scales = L.scales;
  a.group_list = L.group_list;
  a.rows = L.rows;
  a.cols = L.cols;
  a.k_blocks = L.k_blocks;
  a.ldk = L.k_blocks * L.block / 2;
  const int ct = L.dtype == kBF16 ? (L.block == 32 ? KmShape<kBF16, 32>::ctile : KmShape<kBF16, 128>::ctile)
                                   : (L.block == 32 ? KmShape<kF32, 32>::ctile : KmShape<kF32, 128>::ctile);
  a.nct = (L.cols + ct - 1) / ct;
  a.num_groups = L.num_groups;
  a.list_type = L.list_type;
  a.sf = L.sf;
  const bool grouped = L.group_list != nullptr;
  // block-rows the grid covers: all that can exist
  const int64_t nbt = grouped ? L.k_blocks : (L.rows + L.block - 1) / L.block;
  const int64_t nkt = (nbt * L.block + kKTile - 1) / kKTile;
  a.ntiles = nkt * a.nct;
  if (a.ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.ntiles == 0) return hipSuccess;
  const bool vec = L.cols % (L.dtype == kBF16 ? 8 : 4) == 0;  // 16-byte aligned row pieces
  if (L.dtype == kBF16)
    return L.block == 32 ? km_rule<kBF16, 32>(L.rule, grouped, vec, a, st)
                         : km_rule<kBF16, 128>(L.rule, grouped, vec, a, st);
  return L.block == 32 ? km_rule<kF32, 32>(L.rule, grouped, vec, a, st)
                       : km_rule<kF32, 128>(L.rule, grouped, vec, a, st);
}

hipError_t launch_dequant(const DqLaunch &L, hipStream_t st) {
  DqArgs a;
  a.codes = L.codes;
  a.scales = L.scales;
  a.y = static_cast<uint8_t *>(L.y);
  a.rows = L.rows;
  a.cols = L.cols;
  a.half = (L.cols + 1) / 2;
  a.nb = (L.cols + L.block - 1) / L.block;
  a.nchunks = 0;
  a.nxr = 0;
  if (L.dtype == kBF16) return L.block == 32 ? dq_launch<kBF16, 5>(a, st) : dq_launch<kBF16, 7>(a, st);
  return L.block == 32 ? dq_launch<kF32, 5>(a, st) : dq_launch<kF32, 7>(a, st);
}

}  // namespace mxfp4
