// probe_kernels.hip -- streaming probes for measurement (libmxfp4_probe.so).
//
// Not part of the method or of the C ABI in include/mxfp4.h: these kernels
// move bytes with the access pattern of the quantization kernels and do no
// arithmetic, so their time is what the memory system gives that pattern.
// bench.py reports them as the achievable bandwidth next to the kernels.
//
// Per 16-byte piece (a lane's chunk of 8 bf16 elements in the row-wise
// forward):
//   kind 0 "fwd"   read 16 B, write 16 B (y) and 1 B (one bitmap byte)
//   kind 1 "copy"  read 16 B, write 16 B
//   kind 2 "read"  read 16 B (a word of the sum is stored only if it equals
//                  a value no input here produces, so nothing is written)
//   kind 3 "write" write 16 B
//   kind 4 "dual"  read 16 B, write 16 B to dst and 16 B to side (the dual
//                  launch's two y views, without its bitmaps)
//   kind 5 "pack"  read 16 B, write 4 B (the packed codes of 8 elements)
// with non-temporal 16-byte accesses (the quantization kernels' ld16/st16),
// `per_lane` pieces per lane in workgroups of `threads` lanes (the row-wise
// forward: one piece, 64 lanes).  With a stamps
// buffer, the first lane of every workgroup records the 100 MHz wall clock
// (s_memrealtime) when the workgroup starts and when its stores have been
// issued: stamps[2 * wg] and stamps[2 * wg + 1].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// U pieces per lane: piece (blockIdx.x * U + u) * blockDim.x + threadIdx.x, so
// each of the lane's U accesses is part of one contiguous stretch of
// 16 * blockDim.x bytes; all U loads are issued before any store.
template <int KIND, bool STAMP, int U>
__global__ void probe_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                             uint8_t *__restrict__ side, int64_t npieces, uint64_t *stamps) {
  uint64_t t0 = 0;
  if (STAMP) t0 = wall_clock64();
  const int64_t base = (int64_t)blockIdx.x * U * blockDim.x + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * blockDim.x;
    const u32x4 z = {0u, 0u, 0u, 0u};
    v[u] = (KIND != 3 && i < npieces) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src) + i) : z;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * blockDim.x;
    if (i < npieces) {
      if (KIND == 3) {
        const u32x4 w = {(uint32_t)i, 1u, 2u, 3u};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(dst) + i);
      } else if (KIND == 5) {
        reinterpret_cast<uint32_t *>(dst)[i] = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      } else {
        if (KIND == 0 || KIND == 1 || KIND == 4)
          __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4 *>(dst) + i);
        if (KIND == 4) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4 *>(side) + i);
        if (KIND == 0) side[i] = (uint8_t)v[u].x;
        if (KIND == 2) {
          const uint32_t s = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
          if (s == 0x9E3779B9u && v[u].x == 0x7F7F7F7Fu) side[i] = 1;
        }
      }
    }
  }
  if (STAMP && threadIdx.x == 0) {
    stamps[2 * (int64_t)blockIdx.x] = t0;
    stamps[2 * (int64_t)blockIdx.x + 1] = wall_clock64();
  }
}

template <int KIND, int U>
hipError_t launch(const void *src, void *dst, void *side, int64_t npieces, int threads, uint64_t *stamps,
                  hipStream_t st) {
  const int64_t per_wg = (int64_t)threads * U;
  const int64_t nwg = (npieces + per_wg - 1) / per_wg;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg), block((unsigned)threads);
  auto s = static_cast<const uint8_t *>(src);
  auto d = static_cast<uint8_t *>(dst);
  auto m = static_cast<uint8_t *>(side);
  if (stamps)
    hipLaunchKernelGGL((probe_kernel<KIND, true, U>), grid, block, 0, st, s, d, m, npieces, stamps);
  else
    hipLaunchKernelGGL((probe_kernel<KIND, false, U>), grid, block, 0, st, s, d, m, npieces, stamps);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_u(int per_lane, const void *src, void *dst, void *side, int64_t npieces, int threads,
                    uint64_t *stamps, hipStream_t st) {
  switch (per_lane) {
    case 1: return launch<KIND, 1>(src, dst, side, npieces, threads, stamps, st);
    case 2: return launch<KIND, 2>(src, dst, side, npieces, threads, stamps, st);
    case 4: return launch<KIND, 4>(src, dst, side, npieces, threads, stamps, st);
    case 8: return launch<KIND, 8>(src, dst, side, npieces, threads, stamps, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// npieces 16-byte pieces: src and dst hold 16 * npieces bytes (16-byte
// aligned; dst 4 * npieces for kind 5), side npieces bytes (kinds 0 and 2) or
// 16 * npieces (kind 4, 16-byte aligned), stamps 2 * ceil(npieces /
// (threads * per_lane)) words when not NULL.  threads: 64, 128, 256, 512 or
// 1024; per_lane: 1, 2, 4 or 8.  Returns a hipError_t value (0 on success).
extern "C" int probe_stream(int kind, const void *src, void *dst, void *side, int64_t npieces, int threads,
                            int per_lane, uint64_t *stamps, void *stream) {
  if (threads != 64 && threads != 128 && threads != 256 && threads != 512 && threads != 1024)
    return (int)hipErrorInvalidValue;
  if (npieces < 0) return (int)hipErrorInvalidValue;
  if (kind != 3 && !src) return (int)hipErrorInvalidValue;
  if (kind != 2 && !dst) return (int)hipErrorInvalidValue;
  if ((kind == 0 || kind == 2 || kind == 4) && !side) return (int)hipErrorInvalidValue;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return (int)hipErrorInvalidValue;
  if (kind == 4 && (reinterpret_cast<uintptr_t>(side) & 15)) return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0: return (int)launch_u<0>(per_lane, src, dst, side, npieces, threads, stamps, st);
    case 1: return (int)launch_u<1>(per_lane, src, dst, side, npieces, threads, stamps, st);
    case 2: return (int)launch_u<2>(per_lane, src, dst, side, npieces, threads, stamps, st);
    case 3: return (int)launch_u<3>(per_lane, src, dst, side, npieces, threads, stamps, st);
    case 4: return (int)launch_u<4>(per_lane, src, dst, side, npieces, threads, stamps, st);
    case 5: return (int)launch_u<5>(per_lane, src, dst, side, npieces, threads, stamps, st);
    default: return (int)hipErrorInvalidValue;
  }
}

// Frequency of the clock behind wall_clock64(), in kHz.
extern "C" int probe_wall_clock_khz(int device) {
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return -1;
  return khz;
}

// ---- per-CU rates ------------------------------------------------------------
// 512-thread workgroups holding 96 KiB (kind 0) or 160 KiB (kinds 1-3) of LDS,
// so one runs per CU.
//   kind 0 "load": each workgroup reads `passes` times a window of `win`
//          16-byte pieces starting at piece (blockIdx.x % nwin) * win, U = 4
//          loads per lane in flight; one XOR per lane to out.  A window
//          shared by all workgroups stays in L2 (per-CU rate from L2); a
//          window per workgroup over a large buffer streams from HBM.
//   kind 1 "lds_read_swizzled": per wave `passes` x 8 ds_read_b128 in the
//          grouped matmul's fragment pattern (row l % 32 of a 32-row tile,
//          XOR-swizzled 16-byte slot), rotating over 16 KiB windows.
//   kind 2 "lds_read_linear": the same with 16 lanes reading 256 contiguous
//          bytes.
//   kind 3 "lds_write": 8 ds_write_b128 per wave and pass in the matmul's
//          staging pattern (8 lanes per 128-byte row, swizzled slots).
// All offsets stay inside the buffer / the LDS array; out holds
// gridDim.x * 512 16-byte pieces.
namespace {

__device__ __forceinline__ int swz16(int r, int c) { return (c ^ ((r ^ (r >> 3)) & 7)) << 4; }

__global__ __launch_bounds__(512, 1) void cu_load_kernel(const u32x4 *__restrict__ buf, int64_t win, int64_t nwin,
                                                         int passes, u32x4 *__restrict__ out) {
  extern __shared__ uint8_t dyn[];
  const int t = threadIdx.x;
  const u32x4 *w = buf + (int64_t)(blockIdx.x % nwin) * win;
  u32x4 acc = {0u, 0u, 0u, 0u};
  constexpr int U = 4;
  for (int p = 0; p < passes; ++p) {
    for (int64_t b = 0; b + 512 * U <= win; b += 512 * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = w[b + u * 512 + t];
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u];
    }
  }
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F7F7F7Fu) dyn[t] = 1;  // keeps the LDS allocation
  out[(int64_t)blockIdx.x * 512 + t] = acc;
}

template <int KIND>
__global__ __launch_bounds__(512, 1) void cu_lds_kernel(int passes, u32x4 *__restrict__ out) {
  __shared__ __align__(16) uint8_t s[160 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  for (int i = tid; i < 160 * 1024 / 16; i += 512) reinterpret_cast<u32x4 *>(s)[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < passes; ++it) {
    const int base = ((it + wave) & 7) * 16384;
    if (KIND == 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = (k & 3) * 32 + l32;
        acc ^= *reinterpret_cast<const u32x4 *>(&s[base + r * 128 + swz16(r, (k >> 2) * 4 + h)]);
      }
    } else if (KIND == 2) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= *reinterpret_cast<const u32x4 *>(&s[base + k * 1024 + lane * 16]);
    } else {
      const int lr = tid >> 3, lc = tid & 7;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = (lr + 64 * (k & 1)) & 127;
        *reinterpret_cast<u32x4 *>(&s[base + row * 128 + swz16(row, lc)]) = acc + u32x4{(unsigned)k, 0u, 0u, 0u};
        acc.x += 1u;
      }
    }
  }
  __syncthreads();
  if (KIND == 3) acc ^= reinterpret_cast<const u32x4 *>(s)[tid];
  out[(int64_t)blockIdx.x * 512 + tid] = acc;
}

}  // namespace

// kind 0: buf holds nwin * win 16-byte pieces (16-byte aligned); kinds 1-3
// ignore buf, win and nwin.  Returns a hipError_t value (0 on success).
extern "C" int probe_cu_rate(int kind, const void *buf, int64_t win, int64_t nwin, int passes, int nwg, void *out,
                             void *stream) {
  if (nwg <= 0 || passes < 0 || !out || (kind == 0 && (!buf || win <= 0 || nwin <= 0)))
    return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  u32x4 *o = static_cast<u32x4 *>(out);
  switch (kind) {
    case 0:
      hipLaunchKernelGGL(cu_load_kernel, dim3(nwg), dim3(512), 96 * 1024, st, static_cast<const u32x4 *>(buf), win,
                         nwin, passes, o);
      break;
    case 1: hipLaunchKernelGGL(cu_lds_kernel<1>, dim3(nwg), dim3(512), 0, st, passes, o); break;
    case 2: hipLaunchKernelGGL(cu_lds_kernel<2>, dim3(nwg), dim3(512), 0, st, passes, o); break;
    case 3: hipLaunchKernelGGL(cu_lds_kernel<3>, dim3(nwg), dim3(512), 0, st, passes, o); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// ---- matrix-core rate and shader clock ---------------------------------------
// 512-thread workgroups (two waves per SIMD, one workgroup per CU), each wave
// issuing `iters` rounds of 8 independent v_mfma_scale_f32_32x32x64_f8f6f4
// (fp8 A; fp8 or E2M1 B as fmt_b 0 / 4; operands in registers, E8M0 scales
// 2^0), so the matrix cores stay busy with no memory traffic.  Thread 0 of
// each workgroup writes its shader-clock cycles (s_memtime) and 100 MHz
// ticks (s_memrealtime) from start to end, and the start tick, to
// clocks[3 * blockIdx.x ...]; every lane adds its accumulators to out so that
// no MFMA is dead.  The values stay finite: products of codes below 2 in
// magnitude, at most 2^31 of them per accumulator.
namespace {

typedef int v8i_p __attribute__((ext_vector_type(8)));
typedef float v16f_p __attribute__((ext_vector_type(16)));

template <int BF>
__global__ __launch_bounds__(512, 1) void mfma_rate_kernel(int iters, float *__restrict__ out,
                                                          unsigned long long *__restrict__ clocks) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int tid = threadIdx.x;
  // E4M3 codes 0x30..0x37 (0.5 .. 0.94) and E2M1 codes 1..3 (0.5 .. 1.5), by lane
  const int av = 0x30303030 + 0x01010101 * (tid & 7);
  const int bv = BF == 4 ? 0x21212121 + 0x01010101 * ((tid >> 3) & 1) : av;
  v8i_p a = {av, av, av, av, av, av, av, av};
  v8i_p b = {bv, bv, bv, bv, bv, bv, bv, bv};
  v16f_p acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, BF, 0, 127, 0, 127);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) sum += acc[j][v];
  out[(int64_t)blockIdx.x * 512 + tid] = sum;
  if (tid == 0) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    clocks[3 * blockIdx.x] = c1 - c0;
    clocks[3 * blockIdx.x + 1] = r1 - r0;
    clocks[3 * blockIdx.x + 2] = r0;
  }
}

}  // namespace

// fmt_b 0 (fp8 B) or 4 (E2M1 B); out: nwg * 512 floats; clocks: 3 * nwg
// 64-bit words.  Returns a hipError_t value (0 on success).
extern "C" int probe_mfma_rate(int fmt_b, int iters, int nwg, void *out, void *clocks, void *stream) {
  if (nwg <= 0 || iters < 0 || !out || !clocks || (fmt_b != 0 && fmt_b != 4)) return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float *o = static_cast<float *>(out);
  unsigned long long *c = static_cast<unsigned long long *>(clocks);
  if (fmt_b == 4) hipLaunchKernelGGL(mfma_rate_kernel<4>, dim3(nwg), dim3(512), 0, st, iters, o, c);
  else hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(nwg), dim3(512), 0, st, iters, o, c);
  return (int)hipGetLastError();
}
