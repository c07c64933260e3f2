// mxfp4_groups.h -- device-side decoding of a grouped (per-expert) row split.
//
// The hyper-parallel page's grouped operand passes a group_list of per-group
// row counts (group_list_type 1) or cumulative row ends (type 0;
// normalize_group_list turns counts into cumulative sums).  Column blocks
// restart at every group start, so block-row t (numbered group by group,
// ceil(c_g / block) per group) covers rows [start, start + len) with
// len <= block.  Every wave decodes the list itself: one vector load brings
// 64 entries into the lanes, then a wave-uniform loop walks them in scalar
// registers (v_readlane), so no LDS, no barrier and no host synchronisation
// are involved.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

__device__ __forceinline__ int64_t lane_i64(int64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave-uniform result: *start and *len of block-row t (len 0 past the end).
// Group ends are clamped into [previous end, rows].
__device__ __forceinline__ void block_row_uniform(const int64_t *gl, int num_groups, int list_type,
                                                  int64_t rows, int block_log2, int64_t t,
                                                  int64_t *start, int64_t *len) {
  const int lane = (int)__lane_id();
  int64_t prev_end = 0, cum = 0, brow = 0;
  *start = 0;
  *len = 0;
  for (int base = 0; base < num_groups; base += 64) {
    const int g = base + lane;
    const int64_t mine = g < num_groups ? gl[g] : 0;
    const int n = num_groups - base < 64 ? num_groups - base : 64;
    for (int j = 0; j < n; ++j) {
      const int64_t raw = lane_i64(mine, j);
      int64_t end;
      if (list_type == 1) {
        cum += raw > 0 ? raw : 0;
        end = cum;
      } else {
        end = raw;
      }
      end = end > prev_end ? end : prev_end;
      end = end < rows ? end : rows;
      const int64_t nb = (end - prev_end + ((int64_t)1 << block_log2) - 1) >> block_log2;
      if (t < brow + nb) {
        *start = prev_end + ((t - brow) << block_log2);
        const int64_t rem = end - *start;
        *len = rem < ((int64_t)1 << block_log2) ? rem : ((int64_t)1 << block_log2);
        return;
      }
      brow += nb;
      prev_end = end;
    }
  }
}

}  // namespace mxfp4
