/*
 * mxfp4.h -- C ABI of libmxfp4, MXFP4 fake quantization on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (amct PR "feat: add MXFP4 QAT fake-quant Linear (with STE)",
 * README section "1. MXFP4 and STE", fake_quant.py):  a tensor is cut into
 * blocks of `block` consecutive elements along a chosen axis; every block
 * shares one power-of-two scale 2^k (stored as an E8M0 byte k + 127); each
 * element x is replaced by sign(x) * c * 2^k where c is the E2M1 code
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} nearest to |x| / 2^k (decided by the midpoints
 * 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), so the block is clipped at 6 * 2^k.
 * The backward pass is the straight-through estimator: the gradient passes
 * unchanged (plain) or is zeroed where |x| > 6 * 2^k (clipped STE,
 * _MXFP4FakeQuantSTE.backward / mxfp4_saturation_mask).
 *
 * Scale rules (mxfp4_desc_t.rule):
 *   MXFP4_RULE_FLOOR (default) -- k = floor(log2 amax) - 2, clamped below at
 *       -127 (an all-zero block gets k = -127, E8M0 byte 0); a magnitude
 *       exactly on a midpoint goes to the lower code.
 *   MXFP4_RULE_AMCT -- the pages' _block_scale: r = fl32(amax / scale_factor)
 *       (IEEE binary32 division), r = max(r, 2^-30), k = the integer nearest
 *       to log2(r); a magnitude exactly on a midpoint goes to the higher code
 *       (torch.bucketize(..., right=True)).  Results are specified while
 *       k <= 127 (always true for scale_factor >= 6 and finite input).
 * Zeros: x = -0.0 gives +0.0; a negative x that snaps to code 0 gives -0.0
 * (torch.sign(x/scale) * code; torch.sign(-0.0) is +0).  NaN and Inf inputs
 * are outside the contract (the kernels still run and do not fault).
 *
 * Tensors are 2-D, `rows` x `cols`, row-major and contiguous (leading
 * dimension = cols); higher-rank tensors are flattened to rows = prod(leading
 * dims).  Element dtype: MXFP4_BF16 (bf16 bit patterns) or MXFP4_F32.
 * Output values have the input's dtype and are exact (every produced value is
 * representable), so results are bit-for-bit reproducible.
 *
 * Memory and streams: every pointer is caller-owned device memory.  The
 * library allocates nothing, keeps no state between calls, never
 * synchronizes, and enqueues its kernels on `stream` (a hipStream_t; NULL is
 * the null stream).  Outputs are fully written inside their documented
 * shapes; no byte past a shape is touched.  Element arrays (x, y, grads),
 * packed codes and COL / GROUPED bitmaps must be 16-byte aligned, ROW bitmaps
 * 4-byte aligned, group_list 8-byte aligned; scale arrays need no alignment.
 *
 * Errors: every call validates its arguments on the host before launching
 * anything.  MXFP4_EINVAL: NULL where a pointer is required, misalignment,
 * negative sizes, rows*cols overflow, unknown axis/layout/rule, scale_factor
 * <= 0 (AMCT), num_groups < 1, unknown group_list_type, or an output that
 * aliases another argument where that is not allowed.  MXFP4_EUNSUPPORTED:
 * block not 32 or 128, dtype not bf16/f32, or an axis combination a call
 * does not offer.  MXFP4_EHIP: a launch failed (the HIP error text is kept).
 * mxfp4_last_error() returns a message for the calling thread's last failed
 * call.  rows*cols == 0 returns MXFP4_OK without launching.
 *
 * Bitmap layouts (uint32 words; the saturation mask |x| > 6 * 2^k, one bit
 * per element, replacing the pages' bool tensor):
 *   ROW      [rows, ceil(cols/32)]: bit b of word (r, w) is column 32w + b.
 *   COL      [ceil(rows/32), cols]: bit b of word (w, c) is row 32w + b.
 *   GROUPED  [NBT * block/32, cols]: word (t*block/32 + q, c) bit b is row
 *            start_t + 32q + b of block-row t (see mxfp4_grouped_qdq).
 * Bits for positions outside the tensor (or outside a short block) are 0.
 * E8M0 scale layouts (one byte per block, k + 127):
 *   ROW [rows, ceil(cols/block)];  COL [ceil(rows/block), cols];
 *   GROUPED [NBT, cols].
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP4_OK = 0,
  MXFP4_EINVAL = 1,
  MXFP4_EUNSUPPORTED = 2,
  MXFP4_EHIP = 3
} mxfp4_status_t;

enum { MXFP4_F32 = 0, MXFP4_BF16 = 1 };                 /* element dtype      */
enum { MXFP4_ROW = 1, MXFP4_COL = 2, MXFP4_GROUPED = 4 }; /* axis / layout bits */
enum { MXFP4_RULE_FLOOR = 0, MXFP4_RULE_AMCT = 1 };      /* scale + tie rule   */
enum { MXFP8_E4M3 = 0, MXFP8_E5M2 = 1 };                 /* MXFP8 element type */
/* element formats of the grouped matmul operands, group split, output type */
enum { MXGEMM_E4M3 = 0, MXGEMM_E5M2 = 1, MXGEMM_E2M1 = 4 };
enum { MXGEMM_GROUP_ROWS = 0, MXGEMM_GROUP_K = 2 };
enum { MXGEMM_OUT_BF16 = 0, MXGEMM_OUT_F32 = 1 };

typedef struct mxfp4_desc {
  int32_t dtype;        /* MXFP4_BF16 or MXFP4_F32                             */
  int32_t block;        /* 32 or 128 elements per shared scale                 */
  int32_t rule;         /* MXFP4_RULE_FLOOR or MXFP4_RULE_AMCT                 */
  int32_t reserved0;    /* must be 0                                           */
  int64_t rows;         /* x is rows x cols, row-major, contiguous             */
  int64_t cols;
  float scale_factor;   /* AMCT only (the pages' default 6.0); must be > 0     */
  int32_t reserved1;    /* must be 0                                           */
} mxfp4_desc_t;

/*
 * Quantize-dequantize (fake quant) forward: fake_quant.py
 * mxfp4_quant_dequant + mxfp4_saturation_mask, fused in one pass over x.
 *
 * axis = MXFP4_ROW: blocks along each row (the pages' last-dim blocking,
 *   _block_view: the last block of a row is short when cols % block != 0).
 * axis = MXFP4_COL: blocks along each column (rows 0..block-1, ...), the
 *   hyper-parallel page's column-wise operand direction; y_col keeps x's
 *   row-major layout.
 * axis = MXFP4_ROW | MXFP4_COL: both views from one read of x.
 * For each direction in `axis`, at least one of its outputs must be
 * non-NULL; outputs of a direction not in `axis` must be NULL.
 *   y_*      dequantized values, x's dtype and layout (NULL: not written);
 *   mask_*   saturation bitmap, ROW / COL layout (NULL: clip off);
 *   scales_* E8M0 bytes, ROW / COL layout (NULL: not written).
 * y_row may equal x when axis == MXFP4_ROW and y_col may equal x when
 * axis == MXFP4_COL (in place); no other aliasing is allowed.
 */
mxfp4_status_t mxfp4_qdq_fwd(const mxfp4_desc_t *desc, int32_t axis,
                             const void *x, void *y_row, uint32_t *mask_row,
                             uint8_t *scales_row, void *y_col,
                             uint32_t *mask_col, uint8_t *scales_col,
                             void *stream);

/*
 * Straight-through-estimator backward (_MXFP4FakeQuantSTE.backward):
 * grad_in = grad_out where the mask bit is 0 and +0.0 where it is 1 (clipped
 * STE).  mask == NULL is the plain STE: grad_in = grad_out (a copy, or
 * nothing when grad_in == grad_out).  `layout` names the bitmap layout the
 * forward wrote: MXFP4_ROW, MXFP4_COL, or MXFP4_GROUPED (then group_list,
 * num_groups and group_list_type are those given to mxfp4_grouped_qdq and
 * desc->block must match it; they are ignored for ROW and COL).
 * grad_out / grad_in are rows x cols of desc->dtype; grad_in may equal
 * grad_out.  desc->rule and scale_factor are ignored.
 */
mxfp4_status_t mxfp4_ste_bwd(const mxfp4_desc_t *desc, int32_t layout,
                             const void *grad_out, const uint32_t *mask,
                             void *grad_in, const int64_t *group_list,
                             int32_t num_groups, int32_t group_list_type,
                             void *stream);

/*
 * Several small tensors in one launch.  A QAT layer fake-quantizes its
 * weight and its input in the same forward (the amct PR page's
 * MXFP4QATLinear.forward: Q(x), then Q(W), then F.linear) and runs the STE
 * of both in its backward; for small layers each of those launches costs
 * more than its bytes.  These two calls take up to MXFP4_BATCH_MAX row-wise
 * tensors per launch with the single-tensor calls' semantics, layouts and
 * checks, tensor by tensor.  desc->dtype, block, rule and scale_factor are
 * shared by all items; desc->rows and cols are ignored (each item carries
 * its own).  items is a host array of n items, read during the call.  Items
 * with rows * cols == 0 are skipped without looking at their pointers.
 * Outputs of different items must not overlap (distinct pointers are
 * checked).
 */
#define MXFP4_BATCH_MAX 8

typedef struct mxfp4_row_item {
  const void *x;      /* rows x cols of desc->dtype                          */
  void *y;            /* QDQ values (may equal x) or NULL                     */
  uint32_t *mask;     /* ROW bitmap or NULL                                    */
  uint8_t *scales;    /* ROW E8M0 bytes or NULL (at least one output)          */
  int64_t rows;
  int64_t cols;
} mxfp4_row_item_t;

/* mxfp4_qdq_fwd with axis = MXFP4_ROW for each item. */
mxfp4_status_t mxfp4_qdq_fwd_rows_batch(const mxfp4_desc_t *desc, int32_t n,
                                        const mxfp4_row_item_t *items,
                                        void *stream);

typedef struct mxfp4_ste_item {
  const void *grad_out;  /* rows x cols of desc->dtype                       */
  const uint32_t *mask;  /* ROW bitmap, or NULL for the plain STE            */
  void *grad_in;         /* may equal grad_out                               */
  int64_t rows;
  int64_t cols;
} mxfp4_ste_item_t;

/* mxfp4_ste_bwd with layout = MXFP4_ROW for each item (desc->rule and
 * scale_factor are ignored; a plain in-place item does nothing). */
mxfp4_status_t mxfp4_ste_bwd_rows_batch(const mxfp4_desc_t *desc, int32_t n,
                                        const mxfp4_ste_item_t *items,
                                        void *stream);

/*
 * The saturation mask as the pages give it (fake_quant.py
 * mxfp4_saturation_mask: a bool tensor of x's shape, true where |x| > 6 * 2^k
 * of the element's block): expands a ROW or COL bitmap written by
 * mxfp4_qdq_fwd / mxfp4_quant_pack into rows x cols bytes, row-major,
 * 1 where the bit is set and 0 elsewhere (the byte values of a torch.bool
 * tensor).  layout: MXFP4_ROW (mask [rows, ceil(cols/32)] words, 4-byte
 * aligned) or MXFP4_COL (mask [ceil(rows/32), cols] words).  out: rows * cols
 * bytes, any alignment, must not overlap mask.
 */
mxfp4_status_t mxfp4_mask_to_bool(int32_t layout, int64_t rows, int64_t cols,
                                  const uint32_t *mask, uint8_t *out,
                                  void *stream);

/*
 * Real quantization to the packed MXFP4 form (the sglang page's
 * "float4_e2m1fn_x2": two FP4 codes per byte), row-wise blocks.
 *   codes  [rows, ceil(cols/2)] bytes: element 2t in the low nibble, 2t+1 in
 *          the high nibble (the last high nibble of an odd row is 0); a
 *          nibble is sign << 3 | E2M1 magnitude code (0..7 in codebook order).
 *   scales [rows, ceil(cols/block)] E8M0 bytes.
 * Optional in the same pass: y_opt (the QDQ values, may equal x) and
 * mask_opt (ROW bitmap).  Decoding codes with scales gives y exactly.
 */
mxfp4_status_t mxfp4_quant_pack(const mxfp4_desc_t *desc, const void *x,
                                uint8_t *codes, uint8_t *scales, void *y_opt,
                                uint32_t *mask_opt, void *stream);

/*
 * Grouped column-wise QDQ (the hyper-parallel page's per-expert operand:
 * rows are tokens split into num_groups consecutive expert groups).
 * group_list is a device array of num_groups int64: row counts
 * (group_list_type = 1, the default on the pages) or cumulative row ends
 * (group_list_type = 0), as normalize_group_list accepts.  Column blocks of
 * desc->block rows start at every group start and never cross a group
 * boundary; a group's last block is short when its count is not a multiple
 * of block; empty groups are allowed.
 * Block-rows are numbered group by group: group g owns ceil(c_g / block)
 * block-rows.  NBT = sum_g ceil(c_g / block) <= ceil(rows/block) + num_groups
 * - 1; size the mask to (ceil(rows/block) + num_groups) * block/32 word-rows
 * and scales to ceil(rows/block) + num_groups byte-rows; rows past NBT are
 * not touched.  The counts must be >= 0 and sum to rows (the caller's
 * contract: the device cannot check it without a host sync); the kernel
 * clamps group ends into [previous end, rows], so an inconsistent list never
 * causes out-of-bounds access, and rows past the last end are not touched.
 * y (required, may equal x), mask_opt (GROUPED bitmap), scales_opt (GROUPED
 * E8M0 bytes).
 */
mxfp4_status_t mxfp4_grouped_qdq(const mxfp4_desc_t *desc, const void *x,
                                 const int64_t *group_list, int32_t num_groups,
                                 int32_t group_list_type, void *y,
                                 uint32_t *mask_opt, uint8_t *scales_opt,
                                 void *stream);

/*
 * K-major packed operand of column-wise or grouped blocks: the hyper-parallel
 * page's column-direction operand (col_data / col_scale of the grouped W4A8
 * matmul), stored packed as on the sglang page (float4_e2m1fn_x2: two FP4
 * codes per byte), with the reduction dimension (the rows of x) contiguous,
 * i.e. the row-wise packed form of x^T with K padded to whole blocks.
 *   group_list NULL: dense column-wise blocks (rows t*block .. t*block +
 *     block - 1, the last one possibly short), NBT = ceil(rows/block);
 *   group_list non-NULL: grouped blocks exactly as mxfp4_grouped_qdq numbers
 *     them (same group_list / num_groups / group_list_type contract).
 *   codes_t  [cols, k_blocks * block / 2] bytes: byte j of row c holds K
 *            positions 2j (low nibble) and 2j+1 (high nibble); K position
 *            t*block + o is x[start_t + o, c] for o < len_t and a padding code
 *            0 otherwise.  Row c starts at c * k_blocks * block / 2 bytes.
 *   scales_t [cols, k_blocks] E8M0 bytes, scale of block-row t of column c at
 *            c * k_blocks + t.
 * k_blocks (the K extent in blocks, >= NBT) must be >= ceil(rows/block)
 * (dense) or >= ceil(rows/block) + num_groups - 1, the most block-rows any
 * group split can produce (grouped); block-rows t >= NBT are not touched.
 * Values and scales are those of mxfp4_qdq_fwd(axis = MXFP4_COL) /
 * mxfp4_grouped_qdq: decoding codes_t with mxfp4_dequant (rows = cols of x,
 * cols = k_blocks * block) gives their y transposed, with zeros at padding.
 * codes_t 16-byte aligned; scales_t any alignment; no aliasing.
 */
mxfp4_status_t mxfp4_quant_pack_kmajor(const mxfp4_desc_t *desc, const void *x,
                                       const int64_t *group_list,
                                       int32_t num_groups,
                                       int32_t group_list_type,
                                       int64_t k_blocks, uint8_t *codes_t,
                                       uint8_t *scales_t, void *stream);

/*
 * Decode (dequantize) the packed form back to values: y[r, c] =
 * (-1)^s * code * 2^(e8 - 127) with the nibble of element c of row r and the
 * E8M0 byte of its block (the sglang page's packed storage read back; the
 * inverse of mxfp4_quant_pack).  desc->rows x desc->cols is y's shape,
 * desc->dtype its dtype (MXFP4_BF16 or MXFP4_F32), desc->block the block of
 * the scales; desc->rule and scale_factor are ignored.
 *   codes  [rows, ceil(cols/2)] (mxfp4_quant_pack layout; K-major codes_t
 *          with rows = cols of x and cols = k_blocks * block),
 *   scales [rows, ceil(cols/block)].
 * Every byte pattern decodes: results are exact (all such values, subnormals
 * included, fit bf16 and fp32) except that values above the largest finite
 * become +-inf (E8M0 >= 253 with large codes); 0xFF is decoded by the same
 * formula.  A sign bit on code 0 gives -0.0.
 * codes and y 16-byte aligned; scales any alignment; no aliasing.
 */
mxfp4_status_t mxfp4_dequant(const mxfp4_desc_t *desc, const uint8_t *codes,
                             const uint8_t *scales, void *y, void *stream);

/*
 * MXFP8 quantization of the grad_output operand of the W4A8 grouped matmul
 * (the hyper-parallel page's npu_dynamic_mx_quant for the NN / NT products,
 * which it does not define; this is the OCP Microscaling v1.0 conversion):
 * blocks of desc->block elements along each row -- 32, the MX block, or 128,
 * the block of the page's block-128 mode, whose quantizer quantizes
 * activations and grad_output in blocks of 128 --, E8M0 scale byte
 * e8 = max(floor(log2 amax) - emax + 127, 0) with emax 8 (MXFP8_E4M3) or 15
 * (MXFP8_E5M2), an all-zero block giving 0; each element is x / 2^(e8-127)
 * rounded to the nearest fp8 value, ties to even, saturating at 448 (E4M3) /
 * 57344 (E5M2), so no NaN / infinity code is produced; -0.0 and negative
 * values that round to zero give -0 (0x80).
 *   q      [rows, cols] fp8 bytes (OCP E4M3 bias 7 / E5M2 bias 15),
 *   scales [rows, ceil(cols/block)] E8M0 bytes.
 * desc->rule and scale_factor are ignored.  x and q 16-byte aligned, scales
 * any alignment, no aliasing.
 */
mxfp4_status_t mxfp8_quant(const mxfp4_desc_t *desc, int32_t fmt, const void *x,
                           uint8_t *q, uint8_t *scales, void *stream);

/*
 * MXFP8 of column-wise (group_list NULL) or grouped blocks of 32 rows, stored
 * K-major: the operands of the TN weight-gradient product (the hyper-parallel
 * page quantizes x and grad_output for it with grouped dynamic quantization
 * for block 32: blocks run down each column and restart at every expert's
 * first token, a group's last block may be short).  Element rule as
 * mxfp8_quant (OCP MX, ties to even, saturating).  Column c of x becomes row
 * c of q_t; block-row t (numbered group by group) fills K positions
 * 32 t .. 32 t + 31 of it, positions past a short block's length hold code 0.
 *   q_t      [cols, k_blocks * 32] fp8 bytes,
 *   scales_t [cols, k_blocks] E8M0 bytes.
 * desc->rows x desc->cols is x's shape (rows = tokens), desc->block must be
 * 32; rule and scale_factor are ignored.  k_blocks >= ceil(rows / 32)
 * (dense) or ceil(rows / 32) + num_groups - 1 (grouped: the most block-rows
 * any list yields); block-rows past the ones the list yields are not
 * written.  group_list: device int64 counts (type 1) or cumulative ends
 * (type 0), clamped as in mxfp4_grouped_qdq.  x and q_t 16-byte aligned; no
 * aliasing.  These operands feed mxfp4_grouped_matmul with MXGEMM_GROUP_K.
 */
mxfp4_status_t mxfp8_quant_kmajor(const mxfp4_desc_t *desc, int32_t fmt, const void *x,
                                  const int64_t *group_list, int32_t num_groups,
                                  int32_t group_list_type, int64_t k_blocks, uint8_t *q_t,
                                  uint8_t *scales_t, void *stream);

/*
 * One MX operand of the grouped matmul: element codes stored with the
 * reduction dimension K contiguous, and E8M0 scales (value of element k of
 * row r = decode(code) * 2^(scale[r, k / block] - 127)).
 */
typedef struct mxfp4_mx_operand {
  const void *data;        /* device, 16-byte aligned: [rows, ld] bytes.  MXGEMM_E4M3 /
                              MXGEMM_E5M2: one OCP fp8 code per byte; MXGEMM_E2M1: two
                              codes per byte, low nibble = even K (mxfp4_quant_pack /
                              mxfp4_quant_pack_kmajor layout)                          */
  const uint8_t *scales;   /* device: [rows, ld_scales] E8M0 bytes                     */
  int32_t fmt;             /* MXGEMM_E4M3, MXGEMM_E5M2 or MXGEMM_E2M1                  */
  int32_t block;           /* elements per scale along K: 32 or 128                    */
  int64_t ld;              /* bytes between rows of data, multiple of 16               */
  int64_t ld_scales;       /* bytes between rows of scales                             */
  int64_t group_stride;    /* MXGEMM_GROUP_ROWS right operand: bytes from group g's
                              data to group g+1's (0 for one shared matrix)           */
  int64_t group_stride_scales;  /* the same for the scales                           */
} mxfp4_mx_operand_t;

/*
 * Grouped MX matrix product, the consumer of the directional operands (the
 * hyper-parallel page's FakeW4A8GroupedLinear.grouped_matmul with the
 * operands _select_operands picks for the NN, NT and TN layouts).  Both
 * operands are K-contiguous, so every layout is, per group,
 *     C[m, n] = sum_k A[m, k] * B[n, k]
 * with A MXFP8 (a->fmt E4M3 or E5M2) and B MXFP4 (E2M1) or MXFP8, products
 * of decoded values summed in fp32 by the matrix cores and rounded once to
 * the output type (bf16 round-to-nearest-even, or fp32).
 *   group_type MXGEMM_GROUP_ROWS (NN forward: A = row-wise MXFP8 tokens, B_g =
 *     the K-major column-wise weight of expert g; NT input gradient: A =
 *     row-wise MXFP8 grad_output, B_g = the row-wise weight): group_list
 *     splits A's M rows; rows of group g use B_g = b->data + g *
 *     b->group_stride (scales likewise).  A [M, K], B [G][N, K], C [M, ldc];
 *     rows past the groups' total are not written.  group_list NULL: one
 *     group of all M rows.  K % 32 == 0.
 *   group_type MXGEMM_GROUP_K (TN weight gradient: A = x^T and B = dy^T,
 *     both column-wise grouped operands in the K-major layout of
 *     mxfp4_quant_pack_kmajor): group_list (required) splits the K tokens;
 *     group g occupies the 32-blocks starting at sum_{h<g} ceil(c_h / 32), in
 *     both operands, and positions past c_g in its last block hold zero
 *     codes.  A [M, k_blocks*32], B [N, k_blocks*32] (codes), C [G][M, ldc];
 *     an empty group writes zeros.  Both blocks 32; group spans are clamped
 *     to k_blocks.
 * group_list: device int64 counts (group_list_type 1) or cumulative ends
 * (type 0), clamped as in mxfp4_grouped_qdq.  out_dtype MXGEMM_OUT_BF16 /
 * MXGEMM_OUT_F32; c aligned to its element size, ldc >= N.  ld >= the bytes
 * of one row of K, ld_scales >= its blocks, and ld * 256 < 2^32.  Nothing is
 * allocated; the kernels run on `stream`.
 */
mxfp4_status_t mxfp4_grouped_matmul(int32_t group_type, int64_t M, int64_t N, int64_t K,
                                    const mxfp4_mx_operand_t *a, const mxfp4_mx_operand_t *b,
                                    const int64_t *group_list, int32_t num_groups,
                                    int32_t group_list_type, int64_t k_blocks,
                                    int32_t out_dtype, void *c, int64_t ldc, void *stream);

/* Message for the calling thread's most recent failed call ("" if none). */
const char *mxfp4_last_error(void);

/* Library ABI version (major * 100 + minor). */
int32_t mxfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
