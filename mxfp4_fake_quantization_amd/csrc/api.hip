// api.hip -- the extern "C" entry points declared in include/mxfp4.h.
// Arguments are validated on the host before anything is enqueued; the
// kernels run on the caller's stream; nothing is allocated or synchronized.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/mxfp4.h"
#include "mxfp4_kernels.h"

namespace {

thread_local std::string g_last_error;

mxfp4_status_t fail(mxfp4_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mxfp4_status_t ok() {
  g_last_error.clear();
  return MXFP4_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Common descriptor checks; sets *n to rows * cols.
mxfp4_status_t check_desc(const mxfp4_desc_t *d, bool need_rule, int64_t *n) {
  if (!d) return fail(MXFP4_EINVAL, "desc is NULL");
  if (d->dtype != MXFP4_BF16 && d->dtype != MXFP4_F32)
    return fail(MXFP4_EUNSUPPORTED, "dtype %d is not MXFP4_BF16 or MXFP4_F32", d->dtype);
  if (d->block != 32 && d->block != 128)
    return fail(MXFP4_EUNSUPPORTED, "block %d is not 32 or 128", d->block);
  if (d->reserved0 != 0 || d->reserved1 != 0) return fail(MXFP4_EINVAL, "reserved fields must be 0");
  if (d->rows < 0 || d->cols < 0) return fail(MXFP4_EINVAL, "negative shape %lld x %lld",
                                              (long long)d->rows, (long long)d->cols);
  if (d->cols > 0 && d->rows > INT64_MAX / 4 / d->cols)
    return fail(MXFP4_EINVAL, "rows * cols overflows");
  if (need_rule) {
    if (d->rule != MXFP4_RULE_FLOOR && d->rule != MXFP4_RULE_AMCT)
      return fail(MXFP4_EINVAL, "unknown rule %d", d->rule);
    if (d->rule == MXFP4_RULE_AMCT && !(d->scale_factor > 0.0f))
      return fail(MXFP4_EINVAL, "scale_factor must be > 0 (got %g)", (double)d->scale_factor);
  }
  *n = d->rows * d->cols;
  return MXFP4_OK;
}

mxfp4_status_t check_ptr(const void *p, uintptr_t align, const char *what) {
  if (!p) return fail(MXFP4_EINVAL, "%s is NULL", what);
  if (!aligned(p, align)) return fail(MXFP4_EINVAL, "%s is not %u-byte aligned", what, (unsigned)align);
  return MXFP4_OK;
}

mxfp4_status_t check_opt(const void *p, uintptr_t align, const char *what) {
  return p ? check_ptr(p, align, what) : MXFP4_OK;
}

mxfp4_status_t hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MXFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define MXFP4_TRY(expr)                      \
  do {                                       \
    mxfp4_status_t st_ = (expr);             \
    if (st_ != MXFP4_OK) return st_;         \
  } while (0)

// Distinct non-NULL pointers (NULL entries are skipped).
bool distinct(std::initializer_list<const void *> ps) {
  const void *seen[16];
  int n = 0;
  for (const void *p : ps) {
    if (!p) continue;
    for (int i = 0; i < n; ++i)
      if (seen[i] == p) return false;
    seen[n++] = p;
  }
  return true;
}

}  // namespace

extern "C" {

mxfp4_status_t mxfp4_qdq_fwd(const mxfp4_desc_t *desc, int32_t axis, const void *x, void *y_row,
                             uint32_t *mask_row, uint8_t *scales_row, void *y_col,
                             uint32_t *mask_col, uint8_t *scales_col, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, true, &n));
  if (axis != MXFP4_ROW && axis != MXFP4_COL && axis != (MXFP4_ROW | MXFP4_COL))
    return fail(MXFP4_EINVAL, "axis %d is not MXFP4_ROW, MXFP4_COL or both", axis);
  const bool row = axis & MXFP4_ROW, col = axis & MXFP4_COL;
  if (!row && (y_row || mask_row || scales_row))
    return fail(MXFP4_EINVAL, "row outputs given but axis has no MXFP4_ROW");
  if (!col && (y_col || mask_col || scales_col))
    return fail(MXFP4_EINVAL, "column outputs given but axis has no MXFP4_COL");
  if (row && !y_row && !mask_row && !scales_row) return fail(MXFP4_EINVAL, "no row output given");
  if (col && !y_col && !mask_col && !scales_col) return fail(MXFP4_EINVAL, "no column output given");
  MXFP4_TRY(check_ptr(x, 16, "x"));
  MXFP4_TRY(check_opt(y_row, 16, "y_row"));
  MXFP4_TRY(check_opt(y_col, 16, "y_col"));
  MXFP4_TRY(check_opt(mask_row, 4, "mask_row"));
  MXFP4_TRY(check_opt(mask_col, 16, "mask_col"));
  // in place is allowed for a single direction only
  const void *xin = (axis == MXFP4_ROW && y_row == x) || (axis == MXFP4_COL && y_col == x) ? nullptr : x;
  if (!distinct({xin, y_row, mask_row, scales_row, y_col, mask_col, scales_col}))
    return fail(MXFP4_EINVAL, "outputs alias each other or x");
  if (n == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (axis == MXFP4_ROW) {
    mxfp4::RowLaunch L{desc->dtype, desc->block, desc->rule, desc->rows, desc->cols,
                       desc->scale_factor, x, y_row, mask_row, scales_row, nullptr};
    return hip_status(mxfp4::launch_row_fwd(L, st), "row-wise forward launch");
  }
  mxfp4::ColLaunch L{desc->dtype, desc->block, desc->rule, desc->rows, desc->cols,
                     desc->scale_factor, x, y_col, mask_col, scales_col,
                     y_row, mask_row, scales_row, nullptr, 0, 1};
  return hip_status(mxfp4::launch_col_fwd(L, st), "column-wise forward launch");
}

mxfp4_status_t mxfp4_ste_bwd(const mxfp4_desc_t *desc, int32_t layout, const void *grad_out,
                             const uint32_t *mask, void *grad_in, const int64_t *group_list,
                             int32_t num_groups, int32_t group_list_type, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, false, &n));
  if (layout != MXFP4_ROW && layout != MXFP4_COL && layout != MXFP4_GROUPED)
    return fail(MXFP4_EINVAL, "layout %d is not MXFP4_ROW, MXFP4_COL or MXFP4_GROUPED", layout);
  MXFP4_TRY(check_ptr(grad_out, 16, "grad_out"));
  MXFP4_TRY(check_ptr(grad_in, 16, "grad_in"));
  MXFP4_TRY(check_opt(mask, layout == MXFP4_ROW ? 4 : 16, "mask"));
  if (mask && layout == MXFP4_GROUPED) {
    if (!group_list) return fail(MXFP4_EINVAL, "group_list is NULL");
    if (!aligned(group_list, 8)) return fail(MXFP4_EINVAL, "group_list is not 8-byte aligned");
    if (num_groups < 1) return fail(MXFP4_EINVAL, "num_groups must be >= 1 (got %d)", num_groups);
    if (group_list_type != 0 && group_list_type != 1)
      return fail(MXFP4_EINVAL, "group_list_type must be 0 or 1 (got %d)", group_list_type);
  }
  if (mask && (mask == grad_out || mask == grad_in)) return fail(MXFP4_EINVAL, "mask aliases a gradient");
  if (n == 0) return ok();
  if (!mask && grad_in == grad_out) return ok();  // plain STE in place: nothing to do
  mxfp4::SteLaunch L{desc->dtype, desc->block, layout, desc->rows, desc->cols, grad_out, mask,
                     grad_in, group_list, num_groups, group_list_type};
  return hip_status(mxfp4::launch_ste_bwd(L, static_cast<hipStream_t>(stream)), "STE backward launch");
}

mxfp4_status_t mxfp4_qdq_fwd_rows_batch(const mxfp4_desc_t *desc, int32_t n, const mxfp4_row_item_t *items,
                                        void *stream) {
  if (n < 1 || n > MXFP4_BATCH_MAX) return fail(MXFP4_EINVAL, "n %d is not in [1, %d]", n, MXFP4_BATCH_MAX);
  if (!items) return fail(MXFP4_EINVAL, "items is NULL");
  mxfp4_desc_t d0 = desc ? *desc : mxfp4_desc_t{};
  d0.rows = 0;
  d0.cols = 0;
  int64_t n0;
  MXFP4_TRY(check_desc(desc ? &d0 : nullptr, true, &n0));
  mxfp4::RowLaunch L[MXFP4_BATCH_MAX];
  const void *outs[3 * MXFP4_BATCH_MAX];
  int m = 0, no = 0;
  for (int i = 0; i < n; ++i) {
    const mxfp4_row_item_t &it = items[i];
    mxfp4_desc_t d = d0;
    d.rows = it.rows;
    d.cols = it.cols;
    int64_t ne;
    MXFP4_TRY(check_desc(&d, true, &ne));
    if (ne == 0) continue;  // an empty item is skipped whatever its pointers
    MXFP4_TRY(check_ptr(it.x, 16, "items[].x"));
    MXFP4_TRY(check_opt(it.y, 16, "items[].y"));
    MXFP4_TRY(check_opt(it.mask, 4, "items[].mask"));
    if (!it.y && !it.mask && !it.scales) return fail(MXFP4_EINVAL, "items[%d] has no output", i);
    if (!distinct({it.y == it.x ? nullptr : it.x, it.y, it.mask, it.scales}))
      return fail(MXFP4_EINVAL, "items[%d]: outputs alias each other or x", i);
    for (const void *o : {(const void *)it.y, (const void *)it.mask, (const void *)it.scales}) {
      if (!o) continue;
      for (int k = 0; k < no; ++k)
        if (outs[k] == o) return fail(MXFP4_EINVAL, "items[%d] shares an output with another item", i);
      outs[no++] = o;
    }
    L[m++] = mxfp4::RowLaunch{desc->dtype, desc->block, desc->rule, it.rows, it.cols, desc->scale_factor,
                              it.x, it.y, it.mask, it.scales, nullptr};
  }
  if (m == 0) return ok();
  return hip_status(mxfp4::launch_row_fwd_batch(L, m, static_cast<hipStream_t>(stream)), "batched forward launch");
}

mxfp4_status_t mxfp4_ste_bwd_rows_batch(const mxfp4_desc_t *desc, int32_t n, const mxfp4_ste_item_t *items,
                                        void *stream) {
  if (n < 1 || n > MXFP4_BATCH_MAX) return fail(MXFP4_EINVAL, "n %d is not in [1, %d]", n, MXFP4_BATCH_MAX);
  if (!items) return fail(MXFP4_EINVAL, "items is NULL");
  mxfp4_desc_t d0 = desc ? *desc : mxfp4_desc_t{};
  d0.rows = 0;
  d0.cols = 0;
  int64_t n0;
  MXFP4_TRY(check_desc(desc ? &d0 : nullptr, false, &n0));
  mxfp4::SteLaunch L[MXFP4_BATCH_MAX];
  const void *outs[MXFP4_BATCH_MAX];
  int m = 0, no = 0;
  for (int i = 0; i < n; ++i) {
    const mxfp4_ste_item_t &it = items[i];
    mxfp4_desc_t d = d0;
    d.rows = it.rows;
    d.cols = it.cols;
    int64_t ne;
    MXFP4_TRY(check_desc(&d, false, &ne));
    if (ne == 0) continue;  // an empty item is skipped whatever its pointers
    MXFP4_TRY(check_ptr(it.grad_out, 16, "items[].grad_out"));
    MXFP4_TRY(check_ptr(it.grad_in, 16, "items[].grad_in"));
    MXFP4_TRY(check_opt(it.mask, 4, "items[].mask"));
    if (it.mask && (it.mask == it.grad_out || it.mask == it.grad_in))
      return fail(MXFP4_EINVAL, "items[%d]: mask aliases a gradient", i);
    for (int k = 0; k < no; ++k)
      if (outs[k] == it.grad_in) return fail(MXFP4_EINVAL, "items[%d] shares grad_in with another item", i);
    outs[no++] = it.grad_in;
    if (!it.mask && it.grad_in == it.grad_out) continue;
    L[m++] = mxfp4::SteLaunch{desc->dtype, desc->block, MXFP4_ROW, it.rows, it.cols, it.grad_out, it.mask,
                              it.grad_in, nullptr, 0, 1};
  }
  if (m == 0) return ok();
  return hip_status(mxfp4::launch_ste_row_batch(L, m, static_cast<hipStream_t>(stream)), "batched STE launch");
}

mxfp4_status_t mxfp4_mask_to_bool(int32_t layout, int64_t rows, int64_t cols, const uint32_t *mask,
                                  uint8_t *out, void *stream) {
  if (layout != MXFP4_ROW && layout != MXFP4_COL)
    return fail(MXFP4_EINVAL, "layout %d is not MXFP4_ROW or MXFP4_COL", layout);
  if (rows < 0 || cols < 0) return fail(MXFP4_EINVAL, "negative shape %lld x %lld", (long long)rows,
                                        (long long)cols);
  if (cols > 0 && rows > INT64_MAX / 32 / cols) return fail(MXFP4_EINVAL, "rows * cols overflows");
  MXFP4_TRY(check_ptr(mask, 4, "mask"));
  if (!out) return fail(MXFP4_EINVAL, "out is NULL");
  if ((const void *)mask == (const void *)out) return fail(MXFP4_EINVAL, "out aliases mask");
  if (rows * cols == 0) return ok();
  return hip_status(mxfp4::launch_mask_bool(layout, rows, cols, mask, out, static_cast<hipStream_t>(stream)),
                    "mask expansion launch");
}

mxfp4_status_t mxfp4_quant_pack(const mxfp4_desc_t *desc, const void *x, uint8_t *codes,
                                uint8_t *scales, void *y_opt, uint32_t *mask_opt, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, true, &n));
  MXFP4_TRY(check_ptr(x, 16, "x"));
  MXFP4_TRY(check_ptr(codes, 16, "codes"));
  MXFP4_TRY(check_ptr(scales, 1, "scales"));
  MXFP4_TRY(check_opt(y_opt, 16, "y_opt"));
  MXFP4_TRY(check_opt(mask_opt, 4, "mask_opt"));
  if (!distinct({y_opt == x ? nullptr : x, codes, scales, y_opt, mask_opt}))
    return fail(MXFP4_EINVAL, "outputs alias each other or x");
  if (n == 0) return ok();
  mxfp4::RowLaunch L{desc->dtype, desc->block, desc->rule, desc->rows, desc->cols,
                     desc->scale_factor, x, y_opt, mask_opt, scales, codes};
  return hip_status(mxfp4::launch_row_fwd(L, static_cast<hipStream_t>(stream)), "pack launch");
}

mxfp4_status_t mxfp4_grouped_qdq(const mxfp4_desc_t *desc, const void *x,
                                 const int64_t *group_list, int32_t num_groups,
                                 int32_t group_list_type, void *y, uint32_t *mask_opt,
                                 uint8_t *scales_opt, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, true, &n));
  MXFP4_TRY(check_ptr(x, 16, "x"));
  MXFP4_TRY(check_ptr(y, 16, "y"));
  MXFP4_TRY(check_opt(mask_opt, 16, "mask_opt"));
  if (!group_list) return fail(MXFP4_EINVAL, "group_list is NULL");
  if (!aligned(group_list, 8)) return fail(MXFP4_EINVAL, "group_list is not 8-byte aligned");
  if (num_groups < 1) return fail(MXFP4_EINVAL, "num_groups must be >= 1 (got %d)", num_groups);
  if (group_list_type != 0 && group_list_type != 1)
    return fail(MXFP4_EINVAL, "group_list_type must be 0 or 1 (got %d)", group_list_type);
  if (!distinct({y == x ? nullptr : x, y, mask_opt, scales_opt, group_list}))
    return fail(MXFP4_EINVAL, "outputs alias each other, x or group_list");
  if (n == 0) return ok();
  mxfp4::ColLaunch L{desc->dtype, desc->block, desc->rule, desc->rows, desc->cols,
                     desc->scale_factor, x, y, mask_opt, scales_opt,
                     nullptr, nullptr, nullptr, group_list, num_groups, group_list_type};
  return hip_status(mxfp4::launch_col_fwd(L, static_cast<hipStream_t>(stream)), "grouped launch");
}

mxfp4_status_t mxfp4_quant_pack_kmajor(const mxfp4_desc_t *desc, const void *x,
                                       const int64_t *group_list, int32_t num_groups,
                                       int32_t group_list_type, int64_t k_blocks,
                                       uint8_t *codes_t, uint8_t *scales_t, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, true, &n));
  MXFP4_TRY(check_ptr(x, 16, "x"));
  MXFP4_TRY(check_ptr(codes_t, 16, "codes_t"));
  MXFP4_TRY(check_ptr(scales_t, 1, "scales_t"));
  const int64_t nb = (desc->rows + desc->block - 1) / desc->block;
  int64_t need = nb;
  if (group_list) {
    if (!aligned(group_list, 8)) return fail(MXFP4_EINVAL, "group_list is not 8-byte aligned");
    if (num_groups < 1) return fail(MXFP4_EINVAL, "num_groups must be >= 1 (got %d)", num_groups);
    if (group_list_type != 0 && group_list_type != 1)
      return fail(MXFP4_EINVAL, "group_list_type must be 0 or 1 (got %d)", group_list_type);
    need = desc->rows > 0 ? nb + num_groups - 1 : 0;
  }
  if (k_blocks < need)
    return fail(MXFP4_EINVAL, "k_blocks %lld is below the %lld block-rows the blocking can produce",
                (long long)k_blocks, (long long)need);
  if (desc->cols > 0 && k_blocks > INT64_MAX / 4 / desc->block / desc->cols)
    return fail(MXFP4_EINVAL, "cols * k_blocks * block overflows");
  if (!distinct({x, codes_t, scales_t, group_list}))
    return fail(MXFP4_EINVAL, "outputs alias each other, x or group_list");
  if (n == 0) return ok();
  mxfp4::KmLaunch L{desc->dtype, desc->block, desc->rule, desc->rows, desc->cols,
                    desc->scale_factor, x, group_list, num_groups, group_list_type,
                    k_blocks, codes_t, scales_t};
  return hip_status(mxfp4::launch_kmajor_pack(L, static_cast<hipStream_t>(stream)),
                    "K-major pack launch");
}

mxfp4_status_t mxfp4_dequant(const mxfp4_desc_t *desc, const uint8_t *codes,
                             const uint8_t *scales, void *y, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, false, &n));
  MXFP4_TRY(check_ptr(codes, 16, "codes"));
  MXFP4_TRY(check_ptr(scales, 1, "scales"));
  MXFP4_TRY(check_ptr(y, 16, "y"));
  if (!distinct({codes, scales, y})) return fail(MXFP4_EINVAL, "codes, scales and y must not alias");
  if (n == 0) return ok();
  mxfp4::DqLaunch L{desc->dtype, desc->block, desc->rows, desc->cols, codes, scales, y};
  return hip_status(mxfp4::launch_dequant(L, static_cast<hipStream_t>(stream)), "dequant launch");
}

mxfp4_status_t mxfp8_quant(const mxfp4_desc_t *desc, int32_t fmt, const void *x, uint8_t *q,
                           uint8_t *scales, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, false, &n));
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2)
    return fail(MXFP4_EINVAL, "fmt %d is not MXFP8_E4M3 or MXFP8_E5M2", fmt);
  MXFP4_TRY(check_ptr(x, 16, "x"));
  MXFP4_TRY(check_ptr(q, 16, "q"));
  MXFP4_TRY(check_ptr(scales, 1, "scales"));
  if (!distinct({x, q, scales})) return fail(MXFP4_EINVAL, "x, q and scales must not alias");
  if (n == 0) return ok();
  mxfp4::Mx8Launch L{desc->dtype, fmt, desc->rows, desc->cols, x, q, scales, desc->block};
  return hip_status(mxfp4::launch_mxfp8_rows(L, static_cast<hipStream_t>(stream)), "MXFP8 launch");
}

}  // extern "C"

namespace {

mxfp4_status_t check_operand(const mxfp4_mx_operand_t *o, const char *what, bool rows_split, int64_t K,
                             int64_t k_blocks, bool is_a) {
  if (!o) return fail(MXFP4_EINVAL, "%s is NULL", what);
  if (is_a ? (o->fmt != MXGEMM_E4M3 && o->fmt != MXGEMM_E5M2)
           : (o->fmt != MXGEMM_E4M3 && o->fmt != MXGEMM_E5M2 && o->fmt != MXGEMM_E2M1))
    return fail(MXFP4_EUNSUPPORTED, "%s->fmt %d is not supported", what, o->fmt);
  if (o->block != 32 && o->block != 128)
    return fail(MXFP4_EUNSUPPORTED, "%s->block %d is not 32 or 128", what, o->block);
  if (!rows_split && o->block != 32)
    return fail(MXFP4_EUNSUPPORTED, "%s->block must be 32 when groups split K", what);
  MXFP4_TRY(check_ptr(o->data, 16, what));
  if (!o->scales) return fail(MXFP4_EINVAL, "%s->scales is NULL", what);
  const int64_t kel = rows_split ? K : k_blocks * 32;  // K extent of a row
  const int64_t row_bytes = o->fmt == MXGEMM_E2M1 ? kel / 2 : kel;
  const int64_t nblk = (kel + o->block - 1) / o->block;
  if (o->ld % 16 != 0 || o->ld < row_bytes)
    return fail(MXFP4_EINVAL, "%s->ld %lld must be a multiple of 16 and >= %lld", what, (long long)o->ld,
                (long long)row_bytes);
  if (o->ld > (int64_t)1 << 24) return fail(MXFP4_EUNSUPPORTED, "%s->ld is above 2^24 bytes", what);
  if (o->ld_scales < nblk || o->ld_scales > (int64_t)1 << 24)
    return fail(MXFP4_EINVAL, "%s->ld_scales %lld must be >= %lld (and below 2^24)", what,
                (long long)o->ld_scales, (long long)nblk);
  if (o->group_stride < 0 || o->group_stride_scales < 0 || o->group_stride % 16 != 0)
    return fail(MXFP4_EINVAL, "%s group strides must be >= 0 (data: a multiple of 16)", what);
  return MXFP4_OK;
}

}  // namespace

extern "C" {

mxfp4_status_t mxfp4_grouped_matmul(int32_t group_type, int64_t M, int64_t N, int64_t K,
                                    const mxfp4_mx_operand_t *a, const mxfp4_mx_operand_t *b,
                                    const int64_t *group_list, int32_t num_groups,
                                    int32_t group_list_type, int64_t k_blocks, int32_t out_dtype,
                                    void *c, int64_t ldc, void *stream) {
  if (group_type != MXGEMM_GROUP_ROWS && group_type != MXGEMM_GROUP_K)
    return fail(MXFP4_EINVAL, "group_type %d is not MXGEMM_GROUP_ROWS or MXGEMM_GROUP_K", group_type);
  const bool rows = group_type == MXGEMM_GROUP_ROWS;
  if (M < 0 || N < 0 || K < 0) return fail(MXFP4_EINVAL, "negative shape");
  if (rows && K % 32 != 0) return fail(MXFP4_EINVAL, "K %lld is not a multiple of 32", (long long)K);
  if (!rows && (k_blocks < 0 || !group_list))
    return fail(MXFP4_EINVAL, "groups that split K need a group_list and k_blocks >= 0");
  if (group_list && (num_groups < 1 || (group_list_type != 0 && group_list_type != 1)))
    return fail(MXFP4_EINVAL, "num_groups must be >= 1 and group_list_type 0 or 1");
  MXFP4_TRY(check_opt(group_list, 8, "group_list"));
  MXFP4_TRY(check_operand(a, "a", rows, K, k_blocks, true));
  MXFP4_TRY(check_operand(b, "b", rows, K, k_blocks, false));
  if (out_dtype != MXGEMM_OUT_BF16 && out_dtype != MXGEMM_OUT_F32)
    return fail(MXFP4_EUNSUPPORTED, "out_dtype %d is not MXGEMM_OUT_BF16 or MXGEMM_OUT_F32", out_dtype);
  MXFP4_TRY(check_ptr(c, out_dtype == MXGEMM_OUT_F32 ? 4 : 2, "c"));
  if (ldc < N) return fail(MXFP4_EINVAL, "ldc %lld < N %lld", (long long)ldc, (long long)N);
  if (M == 0 || N == 0) return ok();
  if (rows && K == 0) return fail(MXFP4_EUNSUPPORTED, "K must be > 0 when groups split rows");
  mxfp4::GemmLaunch L{};
  L.group_type = group_type;
  L.a_fmt = a->fmt;
  L.b_fmt = b->fmt;
  L.a_block = a->block;
  L.b_block = b->block;
  L.out_f32 = out_dtype == MXGEMM_OUT_F32;
  L.M = M;
  L.N = N;
  L.K = K;
  L.k_blocks = k_blocks;
  L.a = static_cast<const uint8_t *>(a->data);
  L.as = a->scales;
  L.b = static_cast<const uint8_t *>(b->data);
  L.bs = b->scales;
  L.lda = a->ld;
  L.ldas = a->ld_scales;
  L.ldb = b->ld;
  L.ldbs = b->ld_scales;
  L.b_gs = rows ? b->group_stride : 0;
  L.b_gss = rows ? b->group_stride_scales : 0;
  L.ldc = ldc;
  L.c = c;
  L.group_list = group_list;
  L.num_groups = group_list ? num_groups : 1;
  L.list_type = group_list_type;
  return hip_status(mxfp4::launch_mx_gemm(L, static_cast<hipStream_t>(stream)), "grouped matmul launch");
}

mxfp4_status_t mxfp8_quant_kmajor(const mxfp4_desc_t *desc, int32_t fmt, const void *x,
                                  const int64_t *group_list, int32_t num_groups,
                                  int32_t group_list_type, int64_t k_blocks, uint8_t *q_t,
                                  uint8_t *scales_t, void *stream) {
  int64_t n;
  MXFP4_TRY(check_desc(desc, false, &n));
  if (desc->block != 32)
    return fail(MXFP4_EUNSUPPORTED, "MXFP8 blocks are 32 elements (got block %d)", desc->block);
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2)
    return fail(MXFP4_EINVAL, "fmt %d is not MXFP8_E4M3 or MXFP8_E5M2", fmt);
  MXFP4_TRY(check_ptr(x, 16, "x"));
  MXFP4_TRY(check_ptr(q_t, 16, "q_t"));
  MXFP4_TRY(check_ptr(scales_t, 1, "scales_t"));
  const int64_t nb = (desc->rows + 31) / 32;
  int64_t need = nb;
  if (group_list) {
    if (!aligned(group_list, 8)) return fail(MXFP4_EINVAL, "group_list is not 8-byte aligned");
    if (num_groups < 1) return fail(MXFP4_EINVAL, "num_groups must be >= 1 (got %d)", num_groups);
    if (group_list_type != 0 && group_list_type != 1)
      return fail(MXFP4_EINVAL, "group_list_type must be 0 or 1 (got %d)", group_list_type);
    need = desc->rows > 0 ? nb + num_groups - 1 : 0;
  }
  if (k_blocks < need)
    return fail(MXFP4_EINVAL, "k_blocks %lld is below the %lld block-rows the blocking can produce",
                (long long)k_blocks, (long long)need);
  if (desc->cols > 0 && k_blocks > INT64_MAX / 64 / desc->cols)
    return fail(MXFP4_EINVAL, "cols * k_blocks * 32 overflows");
  if (!distinct({x, q_t, scales_t, group_list}))
    return fail(MXFP4_EINVAL, "outputs alias each other, x or group_list");
  if (n == 0) return ok();
  mxfp4::Km8Launch L{desc->dtype, fmt, desc->rows, desc->cols, x, group_list, num_groups,
                     group_list_type, k_blocks, q_t, scales_t};
  return hip_status(mxfp4::launch_mxfp8_kmajor(L, static_cast<hipStream_t>(stream)),
                    "K-major MXFP8 launch");
}

const char *mxfp4_last_error(void) { return g_last_error.c_str(); }

int32_t mxfp4_version(void) { return 105; }

}  // extern "C"
