// mxfp4_groups.h -- device-side decoding of a grouped (per-expert) row split.
//
// The hyper-parallel page's grouped operand passes a group_list of per-group
// row counts (group_list_type 1) or cumulative row ends (type 0;
// normalize_group_list turns counts into cumulative sums).  Column blocks
// restart at every group start, so block-row t (numbered group by group,
// ceil(c_g / block) per group) covers rows [start, start + len) with
// len <= block.  One wave scans the list (64 groups per step) and the result
// is shared through LDS; no host synchronisation is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

template <typename T>
__device__ __forceinline__ T wave_incl_scan_add(T v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}
__device__ __forceinline__ int64_t wave_incl_scan_max(int64_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int64_t u = __shfl_up(v, off, 64);
    if (lane >= off) v = v > u ? v : u;
  }
  return v;
}

// Group ends are clamped into [previous end, rows]: an inconsistent list
// (negative counts, decreasing ends, a total above rows) never leads to an
// out-of-range row.  Called by all 64 lanes of one wave; lane 0 writes
// out[0] = start, out[1] = len (len 0: t is past the last block-row).
__device__ __forceinline__ void find_block_row(const int64_t *gl, int num_groups, int list_type,
                                               int64_t rows, int block_log2, int64_t t,
                                               int64_t *out) {
  const int lane = (int)__lane_id();
  const int64_t block = (int64_t)1 << block_log2;
  int64_t carry_cum = 0, carry_end = 0, carry_b = 0;
  int64_t start = 0, len = 0;
  bool found = false;
  for (int base = 0; base < num_groups && !found; base += 64) {
    const int g = base + lane;
    const bool valid = g < num_groups;
    const int64_t raw = valid ? gl[g] : 0;
    int64_t top;
    if (list_type == 1) {
      const int64_t inc = valid && raw > 0 ? raw : 0;
      top = carry_cum + wave_incl_scan_add<int64_t>(inc, lane);
      carry_cum = __shfl(top, 63, 64);
    } else {
      top = wave_incl_scan_max(valid ? raw : INT64_MIN, lane);
    }
    int64_t end = top > carry_end ? top : carry_end;
    end = end < rows ? end : rows;
    int64_t prev = __shfl_up(end, 1, 64);
    if (lane == 0) prev = carry_end;
    const int64_t nb = valid ? (end - prev + block - 1) >> block_log2 : 0;
    const int64_t bend = carry_b + wave_incl_scan_add<int64_t>(nb, lane);
    const int64_t bstart = bend - nb;
    const bool hit = valid && nb > 0 && t >= bstart && t < bend;
    if (hit) {
      start = prev + ((t - bstart) << block_log2);
      len = end - start < block ? end - start : block;
    }
    const uint64_t any = __ballot(hit);
    if (any) {
      const int src = __ffsll((unsigned long long)any) - 1;
      start = __shfl(start, src, 64);
      len = __shfl(len, src, 64);
      found = true;
    }
    carry_end = __shfl(end, 63, 64);
    carry_b = __shfl(bend, 63, 64);
  }
  if (lane == 0) {
    out[0] = start;
    out[1] = found ? len : 0;
  }
}

}  // namespace mxfp4
