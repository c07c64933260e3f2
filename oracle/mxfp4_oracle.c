/*
 * mxfp4_oracle.c -- plain, slow, single-threaded CPU oracle for MXFP4 fake
 * quantization.  TEST INFRASTRUCTURE ONLY: nothing on the product path may
 * link, load or call it; only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py use it.  It shares no code with the HIP
 * library (mxfp4_fake_quantization_amd/csrc).
 *
 * What it computes follows the pages of the "MXFP4 QAT fake-quant Linear (with
 * STE)" pull request (gitcode cann/amct #264):
 *   - README "1. MXFP4 and STE": per-block power-of-two scale, E2M1 codebook
 *     {0, .5, 1, 1.5, 2, 3, 4, 6}, plain and clipped STE formulas;
 *   - fake_quant.py _block_view/_unpad (zero padding of the last dim per row,
 *     so blocks never straddle rows), _block_scale, _round_to_e2m1 (midpoint
 *     thresholds), _quant_dequant_torch (divide, snap, sign, multiply, cast),
 *     mxfp4_saturation_mask (|x| > 6*scale) and _MXFP4FakeQuantSTE.backward
 *     (masked_fill of the gradient with 0).
 * The grouped (per-expert) column-wise blocking follows the MindSpore
 * hyper-parallel page "fake_w4a8_gmm_func.py" (normalize_group_list: counts
 * -> cumulative sums), and the packed form follows the sglang "mxfp4_npu.py"
 * page (two FP4 codes per byte); oracle_pack_kmajor stores the column-wise /
 * grouped operand in that packed form with the reduction dimension contiguous.
 * oracle_grouped_matmul is the grouped matrix product that consumes these
 * operands (the hyper-parallel page's grouped_matmul, NN / NT / TN), computed
 * from decoded values with exact products and extended-precision sums.
 *
 * Two scale rules ("profiles"):
 *   FLOOR (default): k = floor(log2 amax) - 2, clamped below at -127; an
 *                    all-zero block takes k = -127.  Midpoint ties go to the
 *                    lower-magnitude code (a value is snapped by counting the
 *                    midpoints it strictly exceeds).
 *   AMCT:            the pages' executed arithmetic on binary32 tensors
 *                    (fake_quant.py _block_scale, _quant_dequant_torch):
 *                    r = fl32(amax / scale_factor), r = max(r, 2^-30),
 *                    L = fl32(log2 r), k = round(L) with halves to even
 *                    (torch.round); y = fl32(x / 2^k); the code follows
 *                    from |y| with ties to the higher-magnitude code
 *                    (torch.bucketize(..., right=True)); the sign is
 *                    torch.sign(y).
 *
 * Arithmetic.  FLOOR is exact: every input element is widened exactly to
 * double, division by 2^k, the midpoint comparisons and code*2^k are exact,
 * and every produced value is exactly representable in the output dtype, so
 * the final narrowing cast does not round.  AMCT repeats the pages' binary32
 * steps: the quotient amax/scale_factor, log2 of it (correctly rounded to
 * binary32; it is exactly a half-integer for some r near sqrt(2)*2^e, and
 * torch.round then picks the even neighbour), and the element quotient
 * x/2^k, which is exact unless it is below the normal range.  Built without
 * fast-math and with the default rounding mode (see build.py).
 *
 * Signs.  The pages multiply torch.sign(y) by the code, and sign(+-0) is 0,
 * so an output is negative only if its quotient is.  FLOOR reads the
 * quotient exactly: a zero input (of either sign) gives +0.0 and a negative
 * input that snaps to code 0 gives -0.0.  AMCT takes the binary32 quotient
 * as the pages do: where fl32(x / 2^k) underflows to zero (|x| <= 2^(k-150))
 * the output is +0.0 even for a negative x.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2 /* decoded operand values for the matrix product */
#define OR_FLOOR 0
#define OR_AMCT 1

/* E2M1 codebook and the midpoints between adjacent entries (fake_quant.py
 * module constants; README section 1). */
static const double kCodes[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
static const double kMids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
/* Largest E2M1 magnitude: the clip limit is 6*scale (MXFP4_E2M1_MAX). */
static const double kE2M1Max = 6.0;
/* Smallest raw scale of the AMCT rule (_MIN_SCALE_RAW = 2^-30). */
static const float kMinScaleRaw = 0x1p-30f;

/* ---- element access ------------------------------------------------------ */

static double get_elem(int dtype, const void *p, int64_t i) {
  if (dtype == OR_F64) return ((const double *)p)[i];
  if (dtype == OR_F32) return (double)((const float *)p)[i];
  /* bf16 is the upper half of an IEEE binary32: widening is exact. */
  uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static void put_elem(int dtype, void *p, int64_t i, double v) {
  if (dtype == OR_F64) {
    ((double *)p)[i] = v;
    return;
  }
  float f = (float)v; /* exact for every value this oracle produces */
  if (dtype == OR_F32) {
    ((float *)p)[i] = f;
    return;
  }
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  /* binary32 -> bf16 with round-to-nearest-even (exact here as well). */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
}

/* ---- the per-block method ------------------------------------------------ */

/* FLOOR: the shared exponent is floor(log2 amax) minus E2M1's emax (2). */
static int scale_exp_floor(double amax) {
  if (amax == 0.0) return -127;
  int e;
  (void)frexp(amax, &e); /* amax = f * 2^e with f in [0.5, 1): floor(log2) = e-1 */
  int k = (e - 1) - 2;
  return k < -127 ? -127 : k;
}

/* AMCT: the pages round log2 of the binary32 raw scale as binary32 tensors
 * do: log2 rounded to the nearest binary32 (log2l carries 64 significant
 * bits, far more than that rounding needs), then rounded to an integer with
 * halves going to the even one (rintf in the default rounding mode, as
 * torch.round does). */
static int scale_exp_amct(double amax, float sf) {
  float r = (float)amax / sf; /* amax is a binary32 value: the cast is exact */
  if (r < kMinScaleRaw) r = kMinScaleRaw;
  float l = (float)log2l((long double)r);
  return (int)rintf(l);
}

/*
 * Quantize-dequantize one block.  idx[] lists the n element positions of the
 * block in x/y (row-wise: consecutive columns; column-wise: consecutive rows).
 * Outputs (each optional): y (same dtype), clip (1 byte per element, the
 * saturation mask), nib (E2M1 nibble per element: sign<<3 | magnitude code).
 * Returns k, the block's scale exponent (scale = 2^k).
 */
static int qdq_block(int dtype, int rule, float sf, const void *x,
                     const int64_t *idx, int n, void *y, uint8_t *clip,
                     uint8_t *nib) {
  double amax = 0.0;
  for (int j = 0; j < n; ++j) {
    double a = fabs(get_elem(dtype, x, idx[j]));
    if (a > amax) amax = a;
  }
  int k = (rule == OR_FLOOR) ? scale_exp_floor(amax) : scale_exp_amct(amax, sf);
  double scale = ldexp(1.0, k);
  for (int j = 0; j < n; ++j) {
    double v = get_elem(dtype, x, idx[j]);
    double q_in;
    if (rule == OR_FLOOR)
      q_in = v / scale; /* exact: division by a power of two */
    else /* binary32 quotient, as y = x_blocked / scale on float32 tensors */
      q_in = (double)((float)v / (float)scale);
    double mag = fabs(q_in);
    int code = 0; /* number of midpoints passed = index of the E2M1 code */
    for (int i = 0; i < 7; ++i) {
      int passed = (rule == OR_FLOOR) ? (mag > kMids[i]) : (mag >= kMids[i]);
      code += passed;
    }
    double sgn = q_in > 0.0 ? 1.0 : (q_in < 0.0 ? -1.0 : 0.0); /* torch.sign */
    double q = sgn * kCodes[code];
    if (sgn == 0.0) q = 0.0; /* sign(+-0) * 0 is +0 */
    double out = q * scale;
    if (y) put_elem(dtype, y, idx[j], out);
    if (clip) clip[idx[j]] = (uint8_t)(fabs(v) > kE2M1Max * scale);
    if (nib) nib[idx[j]] = (uint8_t)((signbit(out) ? 8 : 0) | code);
  }
  return k;
}

/* ---- exported drivers ---------------------------------------------------- */

/* Row-wise: blocks of `block` consecutive elements along each row of the
 * rows x cols row-major tensor; the last block of a row may be shorter.
 * e8m0 (optional) is [rows, ceil(cols/block)] with byte = k + 127. */
int oracle_qdq_rows(int dtype, int64_t rows, int64_t cols, int block, int rule,
                    float sf, const void *x, void *y, uint8_t *clip,
                    uint8_t *e8m0) {
  if (block <= 0 || rows < 0 || cols < 0) return 1;
  int64_t nb = (cols + block - 1) / block;
  int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)block);
  if (!idx) return 2;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      int64_t c0 = b * block;
      int n = (int)((cols - c0) < block ? (cols - c0) : block);
      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;
      int k = qdq_block(dtype, rule, sf, x, idx, n, y, clip, NULL);
      if (e8m0) e8m0[r * nb + b] = (uint8_t)(k + 127);
    }
  }
  free(idx);
  return 0;
}

/* Column-wise: blocks of `block` consecutive rows of one column.  y keeps the
 * row-major rows x cols layout; e8m0 (optional) is [ceil(rows/block), cols]. */
int oracle_qdq_cols(int dtype, int64_t rows, int64_t cols, int block, int rule,
                    float sf, const void *x, void *y, uint8_t *clip,
                    uint8_t *e8m0) {
  if (block <= 0 || rows < 0 || cols < 0) return 1;
  int64_t nb = (rows + block - 1) / block;
  int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)block);
  if (!idx) return 2;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t r0 = b * block;
    int n = (int)((rows - r0) < block ? (rows - r0) : block);
    for (int64_t c = 0; c < cols; ++c) {
      for (int j = 0; j < n; ++j) idx[j] = (r0 + j) * cols + c;
      int k = qdq_block(dtype, rule, sf, x, idx, n, y, clip, NULL);
      if (e8m0) e8m0[b * cols + c] = (uint8_t)(k + 127);
    }
  }
  free(idx);
  return 0;
}

/* Grouped column-wise: the rows are split into num_groups consecutive groups
 * given by group_list (list_type 1: row counts; 0: cumulative row ends, as
 * normalize_group_list accepts).  Column-wise blocks restart at every group
 * start and never cross a group boundary; a group's last block may be short.
 * e8m0 (optional) has one row per block-row: block-rows are numbered group by
 * group, block by block, i.e. [sum_g ceil(c_g/block), cols].
 * Rows past the last group's end are not touched.  Returns 1 when the groups
 * are inconsistent (negative count, decreasing ends, or past `rows`). */
int oracle_grouped_cols(int dtype, int64_t rows, int64_t cols, int block,
                        int rule, float sf, const void *x,
                        const int64_t *group_list, int num_groups,
                        int list_type, void *y, uint8_t *clip, uint8_t *e8m0) {
  if (block <= 0 || rows < 0 || cols < 0 || num_groups < 1) return 1;
  int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)block);
  if (!idx) return 2;
  int64_t start = 0, brow = 0;
  for (int g = 0; g < num_groups; ++g) {
    int64_t end = list_type == 1 ? start + group_list[g] : group_list[g];
    if (end < start || end > rows) {
      free(idx);
      return 1;
    }
    for (int64_t r0 = start; r0 < end; r0 += block, ++brow) {
      int n = (int)((end - r0) < block ? (end - r0) : block);
      for (int64_t c = 0; c < cols; ++c) {
        for (int j = 0; j < n; ++j) idx[j] = (r0 + j) * cols + c;
        int k = qdq_block(dtype, rule, sf, x, idx, n, y, clip, NULL);
        if (e8m0) e8m0[brow * cols + c] = (uint8_t)(k + 127);
      }
    }
    start = end;
  }
  free(idx);
  return 0;
}

/* Straight-through estimator backward: clipped (clip != NULL) zeroes the
 * gradient where the forward saturated (masked_fill with 0.0, i.e. +0);
 * plain (clip == NULL) passes the gradient through unchanged. */
int oracle_ste_bwd(int dtype, int64_t n, const void *grad_out,
                   const uint8_t *clip, void *grad_in) {
  for (int64_t i = 0; i < n; ++i) {
    double g = get_elem(dtype, grad_out, i);
    if (clip && clip[i]) g = 0.0;
    put_elem(dtype, grad_in, i, g);
  }
  return 0;
}

/* Real (packed) row-wise quantization: codes is [rows, ceil(cols/2)] bytes,
 * element 2t in the low nibble and 2t+1 in the high nibble (an odd row's last
 * high nibble is 0); a nibble is sign<<3 | E2M1 magnitude code.  scales is
 * [rows, ceil(cols/block)] E8M0 bytes (k + 127). */
int oracle_pack_rows(int dtype, int64_t rows, int64_t cols, int block, int rule,
                     float sf, const void *x, uint8_t *codes, uint8_t *scales) {
  if (block <= 0 || rows < 0 || cols < 0) return 1;
  int64_t nb = (cols + block - 1) / block;
  int64_t half = (cols + 1) / 2;
  uint8_t *nib = (uint8_t *)calloc((size_t)(rows * cols) + 1, 1);
  int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)block);
  if (!nib || !idx) {
    free(nib);
    free(idx);
    return 2;
  }
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      int64_t c0 = b * block;
      int n = (int)((cols - c0) < block ? (cols - c0) : block);
      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;
      int k = qdq_block(dtype, rule, sf, x, idx, n, NULL, NULL, nib);
      scales[r * nb + b] = (uint8_t)(k + 127);
    }
    for (int64_t t = 0; t < half; ++t) {
      uint8_t lo = nib[r * cols + 2 * t];
      uint8_t hi = (2 * t + 1 < cols) ? nib[r * cols + 2 * t + 1] : 0;
      codes[r * half + t] = (uint8_t)(lo | (hi << 4));
    }
  }
  free(nib);
  free(idx);
  return 0;
}

/* Decode the packed form: value = (-1)^s * code[m] * 2^(e8m0 - 127). */
int oracle_unpack_rows(int dtype, int64_t rows, int64_t cols, int block,
                       const uint8_t *codes, const uint8_t *scales, void *y) {
  if (block <= 0 || rows < 0 || cols < 0) return 1;
  int64_t nb = (cols + block - 1) / block;
  int64_t half = (cols + 1) / 2;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      uint8_t byte = codes[r * half + c / 2];
      uint8_t nibble = (c & 1) ? (byte >> 4) : (byte & 15);
      int k = (int)scales[r * nb + c / block] - 127;
      double v = kCodes[nibble & 7] * ldexp(1.0, k);
      if (nibble & 8) v = -v;
      put_elem(dtype, y, r * cols + c, v);
    }
  }
  return 0;
}

/* K-major ("transposed") packed form of column-wise or grouped blocks: the
 * operand layout an MX matrix product reads along its reduction dimension
 * (the hyper-parallel page's col_data / col_scale directional operand, stored
 * packed two codes per byte as on the sglang page).  Column c of x becomes
 * row c of codes_t: K-position p = t*block + o holds x row start_t + o of
 * block-row t when o < len_t, else a padding code 0; bytes pair K-positions
 * (2j, 2j+1) with 2j in the low nibble.  Block-rows are those of
 * oracle_qdq_cols (group_list NULL: block t is rows t*block .. t*block +
 * block - 1, the last one possibly short) or of oracle_grouped_cols (blocks
 * restart at every group start).
 *   codes_t  [cols, k_blocks * block / 2] bytes,
 *   scales_t [cols, k_blocks] E8M0 bytes (k + 127).
 * Block-rows t >= NBT (the number the blocking yields) are not touched.
 * Returns 1 for bad sizes (k_blocks < NBT, odd block) or an inconsistent
 * group list, as oracle_grouped_cols does. */
int oracle_pack_kmajor(int dtype, int64_t rows, int64_t cols, int block, int rule,
                       float sf, const void *x, const int64_t *group_list,
                       int num_groups, int list_type, int64_t k_blocks,
                       uint8_t *codes_t, uint8_t *scales_t) {
  if (block <= 0 || (block & 1) || rows < 0 || cols < 0 || k_blocks < 0) return 1;
  if (group_list && num_groups < 1) return 1;
  int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)block);
  uint8_t *nib = (uint8_t *)calloc((size_t)(rows * cols) + 1, 1);
  if (!idx || !nib) {
    free(idx);
    free(nib);
    return 2;
  }
  /* block-row list: (start, len) per block-row, in order */
  int64_t nbt = 0, start = 0;
  int ng = group_list ? num_groups : 1;
  int64_t *bstart = (int64_t *)malloc(sizeof(int64_t) * (size_t)(rows / block + ng + 1));
  int64_t *blen = (int64_t *)malloc(sizeof(int64_t) * (size_t)(rows / block + ng + 1));
  if (!bstart || !blen) {
    free(idx); free(nib); free(bstart); free(blen);
    return 2;
  }
  for (int g = 0; g < ng; ++g) {
    int64_t end = !group_list ? rows : (list_type == 1 ? start + group_list[g] : group_list[g]);
    if (end < start || end > rows) {
      free(idx); free(nib); free(bstart); free(blen);
      return 1;
    }
    for (int64_t r0 = start; r0 < end; r0 += block) {
      bstart[nbt] = r0;
      blen[nbt] = (end - r0) < block ? (end - r0) : block;
      ++nbt;
    }
    start = end;
  }
  if (nbt > k_blocks) {
    free(idx); free(nib); free(bstart); free(blen);
    return 1;
  }
  int64_t ldk = k_blocks * block / 2; /* bytes per row of codes_t */
  for (int64_t t = 0; t < nbt; ++t) {
    int n = (int)blen[t];
    for (int64_t c = 0; c < cols; ++c) {
      for (int j = 0; j < n; ++j) idx[j] = (bstart[t] + j) * cols + c;
      int k = qdq_block(dtype, rule, sf, x, idx, n, NULL, NULL, nib);
      scales_t[c * k_blocks + t] = (uint8_t)(k + 127);
      for (int o = 0; o < block; o += 2) {
        uint8_t lo = o < n ? nib[idx[o]] : 0;
        uint8_t hi = o + 1 < n ? nib[idx[o + 1]] : 0;
        codes_t[c * ldk + (t * block + o) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
  free(idx);
  free(nib);
  free(bstart);
  free(blen);
  return 0;
}

/* ---- MXFP8 (the grad_output operand of the W4A8 grouped matmul) ------------
 * The hyper-parallel page quantizes grad_output with npu_dynamic_mx_quant for
 * the NN / NT products but does not define it; this follows the OCP
 * Microscaling (MX) v1.0 conversion: blocks of 32 along the last dimension,
 * shared scale X = 2^k with k = floor(log2 amax) - emax (emax = exponent of
 * the element format's largest normal: E4M3 8, E5M2 15; the same rule with
 * emax = 2 is this file's FLOOR rule for E2M1), clamped below at -127
 * (amax = 0 gives k = -127); every element is x / X rounded to the nearest
 * value of the element format, ties to even, saturating at the largest normal
 * (E4M3 448, E5M2 57344).  Signs follow IEEE conversion: a negative value
 * that rounds to zero, and -0.0, give -0 (byte 0x80).
 * fmt 0: E4M3 (bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN);
 * fmt 1: E5M2 (bias 15, 2 mantissa bits). */
static void fp8_params(int fmt, int *mb, int *bias, double *maxn, int *emax) {
  if (fmt == 0) {
    *mb = 3; *bias = 7; *maxn = 448.0; *emax = 8;
  } else {
    *mb = 2; *bias = 15; *maxn = 57344.0; *emax = 15;
  }
}

/* Encode |v| (already divided by the scale) as a sign-less fp8 code. */
static uint8_t fp8_encode_mag(int fmt, double a) {
  int mb, bias, emax;
  double maxn;
  fp8_params(fmt, &mb, &bias, &maxn, &emax);
  const int emin = 1 - bias; /* exponent of the smallest normal */
  if (a >= maxn) a = maxn;   /* saturation */
  if (a == 0.0) return 0;
  int e;
  (void)frexp(a, &e);
  e -= 1; /* a = m * 2^e, 1 <= m < 2 */
  const int eq = e < emin ? emin : e;
  const double quantum = ldexp(1.0, eq - mb);
  double q = rint(a / quantum) * quantum; /* exact division; rint = ties to even */
  if (q > maxn) q = maxn;
  if (q == 0.0) return 0;
  (void)frexp(q, &e);
  e -= 1;
  if (e < emin) /* subnormal: exponent field 0 */
    return (uint8_t)(q / ldexp(1.0, emin - mb));
  return (uint8_t)(((e + bias) << mb) | (int)((q / ldexp(1.0, e) - 1.0) * (1 << mb)));
}

/* One MXFP8 block of the n elements x[idx[0..n-1]] (OCP MX): scale 2^k with
 * k = floor(log2 amax) - emax, clamped below at -127 (an all-zero block takes
 * -127); each element x / 2^k (exact) rounded to the nearest fp8 value, ties
 * to even, saturating; the sign bit is the input's (so -0.0 gives 0x80).
 * Writes the n codes and returns the E8M0 byte k + 127. */
static uint8_t mx8_block(int dtype, int fmt, const void *x, const int64_t *idx, int n, uint8_t *codes) {
  int mb, bias, emax;
  double maxn;
  fp8_params(fmt, &mb, &bias, &maxn, &emax);
  double amax = 0.0;
  for (int j = 0; j < n; ++j) {
    const double a = fabs(get_elem(dtype, x, idx[j]));
    if (a > amax) amax = a;
  }
  int k = -127;
  if (amax > 0.0) {
    int e;
    (void)frexp(amax, &e);
    k = (e - 1) - emax;
    if (k < -127) k = -127;
  }
  const double scale = ldexp(1.0, k);
  for (int j = 0; j < n; ++j) {
    const double v = get_elem(dtype, x, idx[j]) / scale; /* exact */
    const uint8_t m = fp8_encode_mag(fmt, fabs(v));
    codes[j] = (uint8_t)(m | (signbit(v) ? 0x80 : 0));
  }
  return (uint8_t)(k + 127);
}

/* Row-wise MXFP8 with blocks of `block` elements (32, the OCP MX block, or
 * 128: the hyper-parallel page's block-128 mode quantizes activations and
 * grad_output with its quantizer's block size): q [rows, cols] bytes,
 * scales [rows, ceil(cols/block)] E8M0. */
int oracle_mxfp8_rows(int dtype, int64_t rows, int64_t cols, int fmt, int block, const void *x,
                      uint8_t *q, uint8_t *scales) {
  if (rows < 0 || cols < 0 || (fmt != 0 && fmt != 1) || (block != 32 && block != 128)) return 1;
  const int64_t nb = (cols + block - 1) / block;
  int64_t idx[128];
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t c0 = b * block;
      const int n = (int)((cols - c0) < block ? (cols - c0) : block);
      for (int j = 0; j < n; ++j) idx[j] = r * cols + c0 + j;
      scales[r * nb + b] = mx8_block(dtype, fmt, x, idx, n, q + r * cols + c0);
    }
  }
  return 0;
}

/* MXFP8 of column-wise blocks of 32 rows (group_list NULL) or of grouped
 * blocks that restart at every group start (the hyper-parallel page's
 * grouped quantization for block 32, which feeds the TN weight-gradient
 * product), stored K-major for that product: column c of x becomes row c of
 * q_t, K-position 32 t + o holds the code of row start_t + o of block-row t
 * when o < len_t and 0 otherwise.
 *   q_t      [cols, k_blocks * 32] fp8 bytes,
 *   scales_t [cols, k_blocks] E8M0 bytes.
 * Block-rows t >= NBT (the number the blocking yields) are not touched.
 * Returns 1 for bad sizes (k_blocks < NBT) or an inconsistent group list
 * (negative count, decreasing ends, or past rows). */
int oracle_mxfp8_kmajor(int dtype, int64_t rows, int64_t cols, int fmt, const void *x,
                        const int64_t *group_list, int num_groups, int list_type, int64_t k_blocks,
                        uint8_t *q_t, uint8_t *scales_t) {
  if (rows < 0 || cols < 0 || k_blocks < 0 || (fmt != 0 && fmt != 1)) return 1;
  if (group_list && num_groups < 1) return 1;
  /* block-rows: (start, len) */
  int64_t nbt = 0, cap = rows / 32 + (group_list ? num_groups : 1) + 1;
  int64_t *bs = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
  int *bl = (int *)malloc(sizeof(int) * (size_t)cap);
  if (!bs || !bl) {
    free(bs);
    free(bl);
    return 2;
  }
  const int ng = group_list ? num_groups : 1;
  int64_t start = 0;
  for (int g = 0; g < ng; ++g) {
    const int64_t end = !group_list ? rows : (list_type == 1 ? start + group_list[g] : group_list[g]);
    if (end < start || end > rows) {
      free(bs);
      free(bl);
      return 1;
    }
    for (int64_t r0 = start; r0 < end; r0 += 32) {
      bs[nbt] = r0;
      bl[nbt] = (int)((end - r0) < 32 ? (end - r0) : 32);
      ++nbt;
    }
    start = end;
  }
  if (nbt > k_blocks) {
    free(bs);
    free(bl);
    return 1;
  }
  const int64_t ldq = k_blocks * 32;
  int64_t idx[32];
  uint8_t codes[32];
  for (int64_t t = 0; t < nbt; ++t) {
    for (int64_t c = 0; c < cols; ++c) {
      for (int j = 0; j < bl[t]; ++j) idx[j] = (bs[t] + j) * cols + c;
      scales_t[c * k_blocks + t] = mx8_block(dtype, fmt, x, idx, bl[t], codes);
      for (int o = 0; o < 32; ++o) q_t[c * ldq + t * 32 + o] = o < bl[t] ? codes[o] : 0;
    }
  }
  free(bs);
  free(bl);
  return 0;
}

/* Decode MXFP8 back to values: (-1)^s * element(code) * 2^(e8 - 127), one
 * E8M0 byte per `block` elements of a row. */
int oracle_mxfp8_decode(int dtype, int64_t rows, int64_t cols, int fmt, int block, const uint8_t *q,
                        const uint8_t *scales, void *y) {
  if (rows < 0 || cols < 0 || (fmt != 0 && fmt != 1) || block <= 0) return 1;
  int mb, bias, emax;
  double maxn;
  fp8_params(fmt, &mb, &bias, &maxn, &emax);
  const int64_t nb = (cols + block - 1) / block;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const uint8_t b = q[r * cols + c];
      const int ef = (b & 0x7F) >> mb, m = b & ((1 << mb) - 1);
      double v = ef == 0 ? ldexp((double)m, 1 - bias - mb)
                         : ldexp(1.0 + (double)m / (1 << mb), ef - bias);
      v *= ldexp(1.0, (int)scales[r * nb + c / block] - 127);
      if (b & 0x80) v = -v;
      put_elem(dtype, y, r * cols + c, v);
    }
  return 0;
}

/* ---- grouped MX matrix product ------------------------------------------- */

/* The grouped matmul that consumes the directional operands (hyper-parallel
 * page, FakeW4A8GroupedLinear: grouped_matmul hands the operands chosen by
 * _select_operands to the NPU grouped matmul together with group_list and
 * group_type).  It is computed from the decoded operand values (the MX
 * decoders above, output type OR_F64): every product of two decoded elements
 * is exact in double, and the sums run in long double, so the result is the
 * exact sum to well below fp32 rounding.
 *
 *   group_type 0 -- groups split the rows (the NN forward and the NT input
 *     gradient: tokens of expert g times expert g's weight):
 *       left [M, K], right [G, K, N], out [M, N];
 *       out[m, n] = sum_k left[m, k] * right[g(m), k, n] for every row m of
 *       group g; rows past the last group end are not touched.
 *   group_type 2 -- groups split the reduction dimension (the TN weight
 *     gradient: expert g's tokens of x^T times the same tokens of dy):
 *       left [M, K], right [K, N], out [G, M, N];
 *       out[g, m, n] = sum over k in group g of left[m, k] * right[k, n].
 *
 * group_list holds per-group counts (list_type 1, normalize_group_list turns
 * them into cumulative sums) or cumulative ends (list_type 0) along the split
 * dimension.  Returns 1 for bad sizes, a group_type other than 0 or 2, or an
 * inconsistent list (negative count, decreasing ends, or past the split
 * dimension). */
int oracle_grouped_matmul(int group_type, int64_t M, int64_t N, int64_t K,
                          const double *left, const double *right,
                          const int64_t *group_list, int num_groups, int list_type,
                          double *out) {
  if (M < 0 || N < 0 || K < 0 || num_groups < 1) return 1;
  if (group_type != 0 && group_type != 2) return 1;
  const int64_t split = group_type == 0 ? M : K;
  int64_t start = 0;
  for (int g = 0; g < num_groups; ++g) {
    const int64_t end = list_type == 1 ? start + group_list[g] : group_list[g];
    if (end < start || end > split) return 1;
    if (group_type == 0) {
      const double *w = right + (int64_t)g * K * N;
      for (int64_t m = start; m < end; ++m)
        for (int64_t n = 0; n < N; ++n) {
          long double acc = 0.0L;
          for (int64_t k = 0; k < K; ++k)
            acc += (long double)left[m * K + k] * (long double)w[k * N + n];
          out[m * N + n] = (double)acc;
        }
    } else {
      double *o = out + (int64_t)g * M * N;
      for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
          long double acc = 0.0L;
          for (int64_t k = start; k < end; ++k)
            acc += (long double)left[m * K + k] * (long double)right[k * N + n];
          o[m * N + n] = (double)acc;
        }
    }
    start = end;
  }
  return 0;
}
