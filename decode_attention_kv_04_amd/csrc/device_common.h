// Device helpers shared by the split kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "kernels.h"

#ifndef DA_NT_LOADS
#define DA_NT_LOADS 1
#endif

// Online softmax: the reference max of a state moves only when a score
// exceeds it by more than this (base-2 units). Probabilities then stay below
// 2^slack (finite, exact range for fp32 sums and 16-bit P) and the rescale
// of O happens rarely after the first keys. 0 = move on every increase.
#ifndef DA_RESCALE_SLACK
#define DA_RESCALE_SLACK 8.0f
#endif

namespace da {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR adjacent lanes of a row; every lane of the group receives
// the same bits (each step adds a value and its partner's, a commutative pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: pairs the two quads of each half-row
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: pairs the two half-rows
  if constexpr (LPR >= 32)
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));  // lane ^ 16
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Lane N of this lane's 16-lane DPP row, broadcast to the whole row
// (row_newbcast, gfx90a and later).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(N >= 0 && N < 16, "lane within a row");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, true));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders a wave's LDS accesses across its lanes: the LDS writes before this
// point happen before the reads after it (a lane reading what another lane
// of the wave wrote), and reads before it before later overwrites. A
// wavefront-scope release / acquire pair around a wave barrier: the LDS
// instructions of one wave execute in order, so it emits no wait and only
// keeps the compiler from moving those accesses across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi for packed 16-bit pairs, fp32 accumulation.
template <int KVT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (KVT == DA_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), acc,
                                           false);
}

// Low / high 16-bit element of a packed word as float (exact).
template <int KVT>
__device__ __forceinline__ float lo16_to_f32(uint32_t w) {
  if constexpr (KVT == DA_F16)
    return h2f(w & 0xffffu);
  else
    return __uint_as_float(w << 16);
}
template <int KVT>
__device__ __forceinline__ float hi16_to_f32(uint32_t w) {
  if constexpr (KVT == DA_F16)
    return h2f(w >> 16);
  else
    return __uint_as_float(w & 0xffff0000u);
}

// 16 bytes of KV elements -> E floats.
template <int KVT>
__device__ __forceinline__ void unpack(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (KVT == DA_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (KVT == DA_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = h2f(w[i] & 0xffffu);
      f[2 * i + 1] = h2f(w[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// N contiguous elements of dtype QT at p -> floats (vector loads).
template <int QT, int N>
__device__ __forceinline__ void load_row_f32(const void* p, float* f) {
  if constexpr (QT == DA_F32) {
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 x = static_cast<const float4*>(p)[i];
      f[4 * i] = x.x;
      f[4 * i + 1] = x.y;
      f[4 * i + 2] = x.z;
      f[4 * i + 3] = x.w;
    }
  } else {
    static_assert(N % 4 == 0, "");
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint2 x = static_cast<const uint2*>(p)[i];
      const uint32_t w[2] = {x.x, x.y};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if constexpr (QT == DA_F16) {
          f[4 * i + 2 * k] = h2f(w[k] & 0xffffu);
          f[4 * i + 2 * k + 1] = h2f(w[k] >> 16);
        } else {
          f[4 * i + 2 * k] = __uint_as_float(w[k] << 16);
          f[4 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
      }
    }
  }
}

__device__ __forceinline__ void store_elem(void* base, int64_t idx, int dtype, float x) {
  if (dtype == DA_F32) {
    static_cast<float*>(base)[idx] = x;
  } else if (dtype == DA_F16) {
    static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);  // round to nearest even
  } else {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (x != x) ? 0x7fc00000u : u + 0x7fffu + ((u >> 16) & 1u);  // round to nearest even
    static_cast<uint16_t*>(base)[idx] = static_cast<uint16_t>(r >> 16);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte K/V load (streamed once: optionally with the nontemporal hint).
__device__ __forceinline__ uint4 load16(const char* p) {
#if DA_NT_LOADS
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

// Merge state (m2, l2, o2) into (m, l, o); m in base-2 units, -inf = empty.
template <int N>
__device__ __forceinline__ void merge_into(float& m, float& l, float* o, float m2, float l2, const float* o2) {
  const float M = fmaxf(m, m2);
  const float Mu = (M == -INFINITY) ? 0.0f : M;
  const float a1 = exp2_fast(m - Mu);
  const float a2 = exp2_fast(m2 - Mu);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = M;
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

}  // namespace
}  // namespace da
