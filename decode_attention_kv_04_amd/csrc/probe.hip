// Bandwidth probe kernels used by the benchmark, not by the attention path:
//  - da_probe_read: stream a buffer once with 16-byte loads (the HBM read
//    ceiling the attention kernel is compared with);
//  - da_probe_copy: copy a buffer of known size (its FETCH_SIZE / WRITE_SIZE
//    counter readings calibrate the counters to bytes).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

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
