// Bandwidth probe kernels used by the benchmark, not by the attention path:
//  - da_probe_read_stream: every work-group streams one contiguous chunk of a
//    buffer with non-temporal 16-byte loads (the plain HBM read ceiling);
//  - da_probe_read_blocks: 4 KiB blocks read in a given order (the access
//    pattern of a shuffled page pool: the gather ceiling);
//  - da_probe_copy: copy a buffer of known size (its FETCH_SIZE / WRITE_SIZE
//    counter readings calibrate the counters to bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread per trip
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Work-group w streams elements [w * per_block, (w + 1) * per_block).
__global__ __launch_bounds__(kThreads) void read_chunk_kernel(const u32x4* __restrict__ src, size_t n16,
                                                              uint32_t* sink) {
  const size_t per_block = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = static_cast<size_t>(blockIdx.x) * per_block;
  const size_t hi = lo + per_block < n16 ? lo + per_block : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kThreads) {
    const u32x4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // One store per thread keeps the loads live.
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

// Work-group w reads blocks perm[w * per_wg + i] (4 KiB each) for i <
// per_wg, one wave per block per trip, four non-temporal 16-byte loads per
// lane.
__global__ __launch_bounds__(kThreads) void read_blocks_kernel(const u32x4* __restrict__ src, const int* perm,
                                                               int per_wg, int nblocks, uint32_t* sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (int i = wave; i < per_wg; i += 4) {
    const int idx = blockIdx.x * per_wg + i;
    if (idx >= nblocks) break;
    const u32x4* blk = src + static_cast<size_t>(perm[idx]) * 256;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(blk + u * 64 + lane);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                        size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from `src` with `blocks`
// work-groups, each streaming one contiguous chunk. The sink must hold
// blocks * 256 uint32. 0 on success, 1 on a bad argument, 2 on a launch error.
int da_probe_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || blocks < 1 || (bytes % 16) != 0 || misaligned(src)) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_chunk_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Read `nblocks` 4 KiB blocks of `src` in the order of `perm` (device int32,
// every value < the buffer's size / 4096), `per_wg` blocks per work-group.
// The sink must hold ceil(nblocks / per_wg) * 256 uint32. 0 on success.
int da_probe_read_blocks(const void* src, const int* perm, int nblocks, int per_wg, uint32_t* sink, void* stream) {
  if (!src || !perm || !sink || nblocks < 1 || per_wg < 1 || misaligned(src)) return 1;
  (void)hipGetLastError();
  const int grid = (nblocks + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(read_blocks_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), perm, per_wg, nblocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned); 0 on success.
int da_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!src || !dst || (bytes % 16) != 0 || misaligned(src) || misaligned(dst)) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_kernel, dim3(256 * 16), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
