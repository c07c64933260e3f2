// mxfp4_groups.h -- device-side decoding of a grouped (per-expert) row split.
//
// The hyper-parallel page's grouped operand passes a group_list of per-group
// row counts (group_list_type 1) or cumulative row ends (type 0;
// normalize_group_list turns counts into cumulative sums).  Column blocks
// restart at every group start, so block-row t (numbered group by group,
// ceil(c_g / block) per group) covers rows [start, start + len) with
// len <= block.
//
// Every wave decodes the list itself, without LDS, barriers or host
// synchronisation.  Short lists are read by scalar loads and walked in
// scalar registers.  Long ones are
// scanned 64 groups per step: one vector load puts group g in lane g, 64-bit
// prefix scans over the wave give each group's end row and its cumulative
// block-row count, and a ballot of "cumulative count <= t" counts the groups
// that end before block-row t, i.e. names the group holding it, at a cost
// that does not grow with t's position.  Group ends are clamped into
// [previous end, rows] (negative counts count as 0), so any list gives
// in-range block-rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

__device__ __forceinline__ int64_t lane_i64(int64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t shfl_up_i64(int64_t v, int d) {
  const int lo = __shfl_up((int)(uint32_t)v, d);
  const int hi = __shfl_up((int)(uint32_t)((uint64_t)v >> 32), d);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Inclusive prefix sum / max over the 64 lanes of the wave.
__device__ __forceinline__ int64_t scan_add_i64(int64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = shfl_up_i64(v, d);
    if (lane >= d) v += u;
  }
  return v;
}
__device__ __forceinline__ int64_t scan_max_i64(int64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = shfl_up_i64(v, d);
    if (lane >= d) v = u > v ? u : v;
  }
  return v;
}

// Up to this many groups the list is walked in scalar registers (latency
// grows with the group count but starts low); longer lists use the scan.
#ifndef MXFP4_GROUP_WALK_MAX
#define MXFP4_GROUP_WALK_MAX 32
#endif

// Scalar walk: the entries are read 8 at a time into scalar registers and a
// wave-uniform loop resolves every requested block-row in one pass.
//
// The entries come in by scalar loads (s_load_dwordx16 / x8 / x4 / x2 for
// 8 / 4 / 2 / 1 entries, never past the list's end).  They travel through the
// scalar cache, which the streaming kernels leave idle: a vector load of the
// list waits behind the workgroup's (and the CU's) queued tensor loads, and
// every load of the tensor that depends on a block-row's start waits for it.
// Each load waits for its data inside its own asm statement.  The scalar cache
// is invalidated at every dispatch, so the list may be written by any earlier
// work on the stream.  SLOAD = false reads the list with one vector load per
// 64 entries instead (lane g holds entry g, read back with v_readlane): for
// the matrix product, whose lookup is off the streaming path and whose
// scalar registers are already full.

template <int N>  // 8, 4, 2 or 1 entries from p (p: wave-uniform, 4-byte aligned)
__device__ __forceinline__ void sload_entries(const int64_t *p, int64_t (&e)[8]) {
  typedef int i32x16 __attribute__((ext_vector_type(16)));
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  uint32_t w[16];
  if constexpr (N == 8) {
    i32x16 r;
    asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = (uint32_t)r[i];
  } else if constexpr (N == 4) {
    i32x8 r;
    asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (uint32_t)r[i];
  } else if constexpr (N == 2) {
    i32x4 r;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)r[i];
  } else {
    i32x2 r;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p) : "memory");
    w[0] = (uint32_t)r[0];
    w[1] = (uint32_t)r[1];
  }
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = (int64_t)(((uint64_t)w[2 * i + 1] << 32) | w[2 * i]);
}

template <int NT, bool SLOAD>
__device__ __forceinline__ void block_rows_walk(const int64_t *gl, int num_groups, int list_type,
                                                int64_t rows, int block_log2, const int64_t (&t)[NT],
                                                int64_t (&start)[NT], int64_t (&len)[NT],
                                                int (&grp)[NT]) {
  const int64_t B = (int64_t)1 << block_log2;
  int64_t prev_end = 0, cum = 0, brow = 0;
  int left = NT;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    start[i] = 0;
    len[i] = 0;
    grp[i] = 0;
  }
  // entry j of the current chunk -> block-rows it holds
  auto step = [&](int64_t raw, int g) {
    int64_t end;
    if (list_type == 1) {
      cum += raw > 0 ? raw : 0;
      end = cum;
    } else {
      end = raw;
    }
    end = end > prev_end ? end : prev_end;
    end = end < rows ? end : rows;
    const int64_t nb = (end - prev_end + B - 1) >> block_log2;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (len[i] == 0 && t[i] >= brow && t[i] < brow + nb) {  // wave-uniform
        start[i] = prev_end + ((t[i] - brow) << block_log2);
        const int64_t rem = end - start[i];
        len[i] = rem < B ? rem : B;
        grp[i] = g;
        --left;
      }
    }
    brow += nb;
    prev_end = end;
  };
  if (SLOAD) {
    for (int base = 0; base < num_groups && left > 0;) {
      const int r = num_groups - base;
      const int n = r >= 8 ? 8 : r >= 4 ? 4 : r >= 2 ? 2 : 1;
      int64_t e[8];
      if (n == 8) sload_entries<8>(gl + base, e);
      else if (n == 4) sload_entries<4>(gl + base, e);
      else if (n == 2) sload_entries<2>(gl + base, e);
      else sload_entries<1>(gl + base, e);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < n && left > 0) step(e[j], base + j);
      base += n;
    }
    return;
  }
  const int lane = (int)__lane_id();
  for (int base = 0; base < num_groups && left > 0; base += 64) {
    const int g = base + lane;
    const int64_t mine = g < num_groups ? gl[g] : 0;
    const int n = num_groups - base < 64 ? num_groups - base : 64;
    for (int j = 0; j < n && left > 0; ++j) step(lane_i64(mine, j), base + j);
  }
}

// Wave-uniform lookup of NT block-rows t[0..NT-1] (wave-uniform values):
// start[i], len[i] (len 0 past the last block-row) and the group grp[i]
// holding it.
template <int NT, bool SLOAD = true>
__device__ __forceinline__ void block_rows_lookup(const int64_t *gl, int num_groups, int list_type,
                                                  int64_t rows, int block_log2, const int64_t (&t)[NT],
                                                  int64_t (&start)[NT], int64_t (&len)[NT],
                                                  int (&grp)[NT]) {
  if (num_groups <= MXFP4_GROUP_WALK_MAX) {
    block_rows_walk<NT, SLOAD>(gl, num_groups, list_type, rows, block_log2, t, start, len, grp);
    return;
  }
  const int lane = (int)__lane_id();
  const int64_t B = (int64_t)1 << block_log2;
  int64_t carry_end = 0, carry_blk = 0;
  bool done[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    start[i] = 0;
    len[i] = 0;
    grp[i] = 0;
    done[i] = false;
  }
  for (int base = 0; base < num_groups; base += 64) {
    const int g = base + lane;
    const bool valid = g < num_groups;
    const int64_t raw = valid ? gl[g] : 0;
    // end row of group g, clamped into [previous end, rows]
    int64_t end;
    if (list_type == 1) {
      end = carry_end + scan_add_i64(valid && raw > 0 ? raw : 0, lane);
    } else {
      end = scan_max_i64(valid ? raw : 0, lane);
      end = end > carry_end ? end : carry_end;
    }
    end = end < rows ? end : rows;
    int64_t prev = shfl_up_i64(end, 1);
    if (lane == 0) prev = carry_end;
    const int64_t nb = valid ? (end - prev + B - 1) >> block_log2 : 0;
    const int64_t cum = carry_blk + scan_add_i64(nb, lane);  // block-rows through group g
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (done[i]) continue;  // wave-uniform
      const uint64_t before = __ballot(valid && cum <= t[i]);
      const int gi = (int)__popcll(before);  // first group whose blocks reach past t
      if (gi < 64 && base + gi < num_groups) {
        const int64_t gprev = lane_i64(prev, gi);
        const int64_t gend = lane_i64(end, gi);
        const int64_t gfirst = lane_i64(cum - nb, gi);
        start[i] = gprev + ((t[i] - gfirst) << block_log2);
        const int64_t rem = gend - start[i];
        len[i] = rem < B ? rem : B;
        grp[i] = base + gi;
        done[i] = true;
      }
    }
    carry_end = lane_i64(end, 63);
    carry_blk = lane_i64(cum, 63);
  }
}

// One block-row (and optionally the group holding it).
template <bool SLOAD = true>
__device__ __forceinline__ void block_row_uniform(const int64_t *gl, int num_groups, int list_type,
                                                  int64_t rows, int block_log2, int64_t t,
                                                  int64_t *start, int64_t *len, int *group = nullptr) {
  const int64_t tt[1] = {t};
  int64_t s[1], l[1];
  int g[1];
  block_rows_lookup<1, SLOAD>(gl, num_groups, list_type, rows, block_log2, tt, s, l, g);
  *start = s[0];
  *len = l[0];
  if (group) *group = g[0];
}

// Span of group g in a layout where every group starts on a block boundary
// (ceil(c_h / block) blocks per group h, numbered group by group): first
// block *kb_start and block count *nb (0 for an empty group or g past the
// list).  Ends are clamped as above; wave-uniform.
__device__ __forceinline__ void group_block_span(const int64_t *gl, int num_groups, int list_type,
                                                 int64_t rows, int block_log2, int g,
                                                 int64_t *kb_start, int64_t *nb_out) {
  const int lane = (int)__lane_id();
  const int64_t B = (int64_t)1 << block_log2;
  int64_t carry_end = 0, carry_blk = 0;
  *kb_start = 0;
  *nb_out = 0;
  for (int base = 0; base < num_groups && base <= g; base += 64) {
    const int gg = base + lane;
    const bool valid = gg < num_groups;
    const int64_t raw = valid ? gl[gg] : 0;
    int64_t end;
    if (list_type == 1) {
      end = carry_end + scan_add_i64(valid && raw > 0 ? raw : 0, lane);
    } else {
      end = scan_max_i64(valid ? raw : 0, lane);
      end = end > carry_end ? end : carry_end;
    }
    end = end < rows ? end : rows;
    int64_t prev = shfl_up_i64(end, 1);
    if (lane == 0) prev = carry_end;
    const int64_t nb = valid ? (end - prev + B - 1) >> block_log2 : 0;
    const int64_t cum = carry_blk + scan_add_i64(nb, lane);
    if (g < base + 64) {
      *kb_start = lane_i64(cum - nb, g - base);
      *nb_out = lane_i64(nb, g - base);
      return;
    }
    carry_end = lane_i64(end, 63);
    carry_blk = lane_i64(cum, 63);
  }
}

}  // namespace mxfp4
