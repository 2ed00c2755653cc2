// Bandwidth probe kernels used by the benchmark, not by the attention path:
//  - da_probe_read: stream a buffer once with 16-byte loads (the HBM read
//    ceiling the attention kernel is compared with);
//  - da_probe_copy: copy a buffer of known size (its FETCH_SIZE / WRITE_SIZE
//    counter readings calibrate the counters to bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ src, size_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  // Four independent loads in flight per thread per trip.
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // One store per thread keeps the loads live; the sink holds gridDim.x * kThreads words.
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// Each work-group streams its own contiguous chunk, UNROLL 16-byte loads per
// thread in flight per trip.
template <int UNROLL>
__global__ __launch_bounds__(kThreads) void read_chunk_kernel(const uint4* __restrict__ src, size_t n16,
                                                              uint32_t* sink) {
  const size_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = static_cast<size_t>(blockIdx.x) * per_block;
  const size_t hi = lo + per_block < n16 ? lo + per_block : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (UNROLL - 1) * kThreads < hi; i += UNROLL * kThreads) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kThreads) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// Gather pattern of a shuffled page pool: work-group w reads blocks
// perm[w * per_wg + i] (UNITS x 4 KiB each) for i < per_wg, one wave per
// 4 KiB piece per trip, 4 x 16-byte loads per lane per piece.
template <bool NT, int UNITS>
__global__ __launch_bounds__(kThreads) void read_blocks_kernel(const u32x4* __restrict__ src, const int* perm,
                                                               int per_wg, int nblocks, uint32_t* sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (int i = wave; i < per_wg * UNITS; i += 4) {
    const int idx = blockIdx.x * per_wg + i / UNITS;
    if (idx >= nblocks) break;
    const u32x4* blk = src + (static_cast<size_t>(perm[idx]) * UNITS + i % UNITS) * 256;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = NT ? __builtin_nontemporal_load(blk + u * 64 + lane) : blk[u * 64 + lane];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Work-groups the probes launch; the read sink must hold blocks * 256 uint32.
int da_probe_blocks(void) { return 256 * 16; }

// Read `bytes` (a multiple of 16, 16-byte aligned) from `src`; 0 on success.
int da_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_kernel, dim3(da_probe_blocks()), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Read with a chosen shape: mode 0 = grid-stride (4 loads per trip), mode 1
// = contiguous chunk per work-group with 8 nontemporal loads per trip, mode 2
// = the same with 16. `blocks` work-groups (the sink must hold blocks * 256
// uint32). 0 on success.
int da_probe_read_cfg(const void* src, size_t bytes, uint32_t* sink, int blocks, int mode, void* stream) {
  if (!src || !sink || blocks < 1 || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint4* p = static_cast<const uint4*>(src);
  if (mode == 0)
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, st, p, bytes / 16, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(read_chunk_kernel<8>, dim3(blocks), dim3(kThreads), 0, st, p, bytes / 16, sink);
  else if (mode == 2)
    hipLaunchKernelGGL(read_chunk_kernel<16>, dim3(blocks), dim3(kThreads), 0, st, p, bytes / 16, sink);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// As da_probe_read_blocks with blocks of `units` x 4 KiB (units 1, 2, 4 or 8);
// perm values < bytes / (units * 4096).
int da_probe_read_blocks_ex(const void* src, const int* perm, int nblocks, int per_wg, int nt, int units,
                            uint32_t* sink, void* stream) {
  if (!src || !perm || !sink || nblocks < 1 || per_wg < 1) return 1;
  (void)hipGetLastError();
  const int grid = (nblocks + per_wg - 1) / per_wg;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(src);
#define DA_PROBE_LAUNCH(NTV, U) \
  hipLaunchKernelGGL((read_blocks_kernel<NTV, U>), dim3(grid), dim3(kThreads), 0, st, p, perm, per_wg, nblocks, sink)
  if (nt) {
    switch (units) {
      case 1: DA_PROBE_LAUNCH(true, 1); break;
      case 2: DA_PROBE_LAUNCH(true, 2); break;
      case 4: DA_PROBE_LAUNCH(true, 4); break;
      case 8: DA_PROBE_LAUNCH(true, 8); break;
      default: return 1;
    }
  } else {
    switch (units) {
      case 1: DA_PROBE_LAUNCH(false, 1); break;
      case 2: DA_PROBE_LAUNCH(false, 2); break;
      case 4: DA_PROBE_LAUNCH(false, 4); break;
      case 8: DA_PROBE_LAUNCH(false, 8); break;
      default: return 1;
    }
  }
#undef DA_PROBE_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Read `nblocks` 4 KiB blocks of `src` in the order of `perm` (device int32,
// values < bytes / 4096), `per_wg` blocks per work-group; nt != 0 uses
// nontemporal loads. The sink must hold ceil(nblocks / per_wg) * 256 uint32.
int da_probe_read_blocks(const void* src, const int* perm, int nblocks, int per_wg, int nt, uint32_t* sink,
                         void* stream) {
  return da_probe_read_blocks_ex(src, perm, nblocks, per_wg, nt, 1, sink, stream);
}

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned); 0 on success.
int da_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!src || !dst || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_kernel, dim3(da_probe_blocks()), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
