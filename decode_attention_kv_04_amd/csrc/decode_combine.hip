// Combine pass of paged decode attention for gfx950.
//
// Merges the per-split online-softmax states (m_s, l_s, O_s) of one
// (sequence, query head) into the output row (TVM pull 20426, sharded-nest
// commit message: the per-shard online-softmax states are merged; mlx-runner
// pull 3, GQA-shared split attention commit: a combine kernel merges the
// split partials in a fixed order):
//     M = max_s m_s,  w_s = 2^(m_s - M),  out = sum_s w_s O_s / sum_s w_s l_s
// A split with no attended key (m_s = -inf) gets weight 0 (never -inf minus
// -inf). The order of the sums is fixed, so results are identical run to run.
//
// One wave64 per (query head, sequence); lane i owns elements i, i+64, ... of
// the row, so every load of O_s is one contiguous 256-byte-per-64-lane read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "kernels.h"

namespace da {
namespace {

__device__ __forceinline__ void store_out(void* base, int64_t idx, int dtype, float x) {
  if (dtype == DA_F32) {
    static_cast<float*>(base)[idx] = x;
  } else if (dtype == DA_F16) {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
  } else {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (x != x) ? 0x7fc00000u : u + 0x7fffu + ((u >> 16) & 1u);
    static_cast<uint16_t*>(base)[idx] = static_cast<uint16_t>(r >> 16);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const KernelArgs a) {
  constexpr int N = D / 64;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;

  const int P = a.page_size;
  const int64_t L = a.seq_lens[b];
  const int64_t t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
  const int64_t pf = L > 0 ? t0 / P : 0;
  const int64_t pe = L > 0 ? (L + P - 1) / P : 0;
  int64_t nsplit = (pe - pf + a.pages_per_split - 1) / a.pages_per_split;
  if (nsplit > a.max_splits) nsplit = a.max_splits;
  if (nsplit <= 1) return;  // the split pass wrote this row

  const int64_t base = (static_cast<int64_t>(b) * a.num_q_heads + h) * a.max_splits;
  const float* ml = a.ws_ml + base * 2;
  const float* os = a.ws_o + base * D;

  float M = -INFINITY;
  for (int64_t s = lane; s < nsplit; s += 64) M = fmaxf(M, ml[s * 2]);
  M = wave_max(M);
  const float Mu = (M == -INFINITY) ? 0.0f : M;

  float lsum = 0.0f;
  for (int64_t s = lane; s < nsplit; s += 64) lsum += __builtin_amdgcn_exp2f(ml[s * 2] - Mu) * ml[s * 2 + 1];
  lsum = wave_sum(lsum);

  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.0f;
  for (int64_t s = 0; s < nsplit; ++s) {
    const float w = __builtin_amdgcn_exp2f(ml[s * 2] - Mu);
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = fmaf(w, os[s * D + lane + 64 * i], acc[i]);
  }
  const int64_t row = (static_cast<int64_t>(b) * a.num_q_heads + h) * D;
#pragma unroll
  for (int i = 0; i < N; ++i) store_out(a.out, row + lane + 64 * i, a.out_dtype, lsum > 0.0f ? acc[i] / lsum : 0.0f);
}

}  // namespace

hipError_t launch_combine(const KernelArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.batch);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace da
