// Split pass of paged decode attention for gfx950.
//
// One work-group of four wave64s owns one (split s, KV head j, sequence b):
// the attended keys of pages [pf + s*c, pf + (s+1)*c) of sequence b. It reads
// each K/V row of that range once for all G query heads of the GQA group
// (mlx-runner pull 3, GQA-shared split attention commit: each K/V row is read
// once per group instead of once per head) and produces, per query head, the
// online-softmax state of its keys (TVM pull 20426, sharded-nest commit
// message: shards of the context, each an online-softmax state):
//     m = max_t s_t,  l = sum_t 2^(s_t - m),  O = sum_t 2^(s_t - m) v_t
// with scores s_t kept in base-2 units (s_t = scale*log2(e) * <q, k_t>). A
// sequence with one split writes O / l to the output directly; otherwise the
// state goes to the workspace for the combine pass.
//
// Lane layout. A key row of D elements (D * elt bytes) is read by LPR
// adjacent lanes, each holding DPL = D / LPR elements as VPL 16-byte vectors;
// a load instruction covers RPI = 64 / LPR consecutive rows, each lane group
// reading one contiguous LPR*16-byte segment of its row, so every wave-wide
// 1 KiB load touches whole 64-128 byte lines. q.k is a per-lane partial dot
// product finished by a sum over the LPR lanes of the row with DPP (no LDS,
// no barrier), which leaves the full score in every lane of the row (the
// 8-lanes-per-key layout of llm-web pull 8 is the same idea for WebGPU).
// Each lane then owns the rows of its row slot as a private online-softmax
// shard: its m, l and O slice live in VGPRs and the slots are merged once, at
// the end, first across the wave with lane shuffles and then across the four
// waves through LDS. No barrier is executed inside the key loop.
//
// Masking uses selects, never multiplication by zero, because rows outside
// the attended range may hold NaN: a score outside [t_lo, t_hi) becomes -inf
// and its value row is replaced by zeros before it is accumulated.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

template <int D, int KVT, int GT>
struct Layout {
  static constexpr int ELT = KVT == DA_F32 ? 4 : 2;
  static constexpr int ROWB = D * ELT;                       // bytes per key row
  static constexpr int E = 16 / ELT;                         // elements per 16-byte vector
  static constexpr int LPR_MIN = cmax(8, ROWB / 64);         // at most 4 vectors per lane
  static constexpr int LPR_MAX = ROWB / 16;                  // at least 1 vector per lane
  static constexpr int LPR = cmin(cmax(GT * D / 32, LPR_MIN), LPR_MAX);
  static constexpr int DPL = D / LPR;                        // elements per lane per row
  static constexpr int VPL = DPL / E;                        // vectors per lane per row
  static constexpr int RPI = 64 / LPR;                       // rows per load instruction
  static constexpr int NS = VPL >= 4 ? 1 : 4 / VPL;          // rows per lane per tile
  static constexpr int TR = NS * RPI;                        // rows per tile
  static constexpr int SEG = LPR * E;                        // elements per row segment
  static_assert(LPR >= 8 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lanes per row");
  static_assert(VPL >= 1 && VPL * E * LPR == D, "row split");
  static_assert(RPI <= 8, "a load group must stay inside a page of a multiple of 8 rows");
};

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

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
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

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == DA_F32) return static_cast<const float*>(base)[idx];
  const uint16_t bits = static_cast<const uint16_t*>(base)[idx];
  if (dtype == DA_F16) return h2f(bits);
  return __uint_as_float(static_cast<uint32_t>(bits) << 16);
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

template <int D, int KVT, int GT>
__global__ __launch_bounds__(kThreads) void split_kernel(const KernelArgs a) {
  using LY = Layout<D, KVT, GT>;
  constexpr int LPR = LY::LPR, DPL = LY::DPL, VPL = LY::VPL, RPI = LY::RPI, NS = LY::NS, TR = LY::TR,
                E = LY::E, SEG = LY::SEG;

  const int s = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane % LPR;  // lane within the row
  const int r = lane / LPR;  // row slot within a load instruction

  const int P = a.page_size;
  const int64_t L = a.seq_lens[b];
  const int64_t t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
  const int64_t pf = L > 0 ? t0 / P : 0;
  const int64_t pe = L > 0 ? (L + P - 1) / P : 0;
  const int64_t c_pages = a.pages_per_split;
  int64_t nsplit = (pe - pf + c_pages - 1) / c_pages;
  if (nsplit < 1) nsplit = 1;
  if (nsplit > a.max_splits) nsplit = a.max_splits;
  if (s >= nsplit) return;  // whole work-group, uniform

  const int64_t plo = pf + static_cast<int64_t>(s) * c_pages;
  const int64_t phi = (plo + c_pages < pe) ? plo + c_pages : pe;
  const int64_t t_lo = L > 0 ? (t0 > plo * P ? t0 : plo * P) : 0;
  const int64_t t_hi = L > 0 ? (L < phi * P ? L : phi * P) : 0;

  const int G = a.group;
  const int h0 = kvh * G;

  // q for the G heads of the group, this lane's elements, as float.
  float qf[GT][DPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = v * SEG + c * E + e;
        qf[g][v * E + e] =
            g < G ? load_elem(a.q, (static_cast<int64_t>(b) * a.num_q_heads + h0 + g) * D + d, a.q_dtype) : 0.0f;
      }
    }
  }

  float m[GT], l[GT], o[GT][DPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[g][i] = 0.0f;
  }

  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int64_t block_elems = static_cast<int64_t>(P) * D;             // one (page, head) block
  const int64_t page_elems = block_elems * a.num_kv_heads;
  const int32_t* table_row = a.page_table + static_cast<int64_t>(b) * a.max_pages;
  const uint32_t lane_off = static_cast<uint32_t>((r * D + c * E) * LY::ELT);

  const int64_t tile_first = t_lo / TR;
  const int64_t tile_end = (t_hi + TR - 1) / TR;

  struct Tile {
    uint4 k[NS][VPL];
    uint4 v[NS][VPL];
  };

  // Issue the loads of one tile. Load groups wholly outside [t_lo, t_hi) are
  // skipped (no page-table read, registers zeroed), so only pages holding
  // attended keys are touched.
  auto load_tile = [&](Tile& t, int64_t tile) {
    const int64_t tb = tile * TR;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int64_t gs = tb + ns * RPI;
      if (gs < t_hi && gs + RPI > t_lo) {
        const int64_t pi = gs / P;
        const int64_t phys = table_row[pi];
        const int64_t off = (phys * a.num_kv_heads + kvh) * block_elems + (gs - pi * P) * D;
        const char* kp = kbase + off * LY::ELT + lane_off;
        const char* vp = vbase + off * LY::ELT + lane_off;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          t.k[ns][v] = *reinterpret_cast<const uint4*>(kp + v * SEG * LY::ELT);
          t.v[ns][v] = *reinterpret_cast<const uint4*>(vp + v * SEG * LY::ELT);
        }
      } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          t.k[ns][v] = make_uint4(0, 0, 0, 0);
          t.v[ns][v] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto compute_tile = [&](const Tile& t, int64_t tile) {
    const int64_t tb = tile * TR;
    const bool full = tb >= t_lo && tb + TR <= t_hi;
    bool valid[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int64_t tok = tb + ns * RPI + r;
      valid[ns] = full || (tok >= t_lo && tok < t_hi);
    }
    float sc[NS][GT];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      float kf[DPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) unpack<KVT>(t.k[ns][v], kf + v * E);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc = fmaf(qf[g][i], kf[i], acc);
        sc[ns][g] = acc;
      }
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float x = row_sum<LPR>(sc[ns][g]) * a.scale_log2;
        sc[ns][g] = valid[ns] ? x : -INFINITY;
      }
    }
    float p[NS][GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mt = sc[0][g];
#pragma unroll
      for (int ns = 1; ns < NS; ++ns) mt = fmaxf(mt, sc[ns][g]);
      const float mn = fmaxf(m[g], mt);
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      const float alpha = exp2_fast(m[g] - mu);
      m[g] = mn;
      float ps = 0.0f;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        p[ns][g] = exp2_fast(sc[ns][g] - mu);
        ps += p[ns][g];
      }
      l[g] = l[g] * alpha + ps;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[g][i] *= alpha;
    }
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      float vf[DPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) unpack<KVT>(t.v[ns][v], vf + v * E);
      if (!full) {
#pragma unroll
        for (int i = 0; i < DPL; ++i) vf[i] = valid[ns] ? vf[i] : 0.0f;
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[g][i] = fmaf(p[ns][g], vf[i], o[g][i]);
      }
    }
  };

  // Tiles tile_first + wave, + kWaves, ... with the next tile's loads in
  // flight while the current one is computed.
  int64_t tile = tile_first + wave;
  if (tile < tile_end) {
    Tile ta, tb;
    load_tile(ta, tile);
    while (true) {
      const int64_t next = tile + kWaves;
      if (next < tile_end) load_tile(tb, next);
      compute_tile(ta, tile);
      if (next >= tile_end) break;
      tile = next;
      const int64_t next2 = tile + kWaves;
      if (next2 < tile_end) load_tile(ta, next2);
      compute_tile(tb, tile);
      if (next2 >= tile_end) break;
      tile = next2;
    }
  }

  // Merge the RPI row slots of the wave (lanes with the same c).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float m2 = __shfl_xor(m[g], off, 64);
      const float l2 = __shfl_xor(l[g], off, 64);
      float o2[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) o2[i] = __shfl_xor(o[g][i], off, 64);
      merge_into<DPL>(m[g], l[g], o[g], m2, l2, o2);
    }
  }

  // Merge the four waves through LDS and write the result.
  __shared__ float sh_o[kWaves][GT][D];
  __shared__ float sh_m[kWaves][GT];
  __shared__ float sh_l[kWaves][GT];
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
#pragma unroll
        for (int e = 0; e < E; ++e) sh_o[wave][g][v * SEG + c * E + e] = o[g][v * E + e];
      }
    }
    if (c == 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        sh_m[wave][g] = m[g];
        sh_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = sh_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh_m[w][g]);
    const float Mu = (M == -INFINITY) ? 0.0f : M;
    float lsum = 0.0f, osum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float aw = exp2_fast(sh_m[w][g] - Mu);
      lsum += aw * sh_l[w][g];
      osum += aw * sh_o[w][g][d];
    }
    const int64_t row = static_cast<int64_t>(b) * a.num_q_heads + h0 + g;
    if (nsplit == 1) {
      store_elem(a.out, row * D + d, a.out_dtype, lsum > 0.0f ? osum / lsum : 0.0f);
    } else {
      const int64_t srow = row * a.max_splits + s;
      a.ws_o[srow * D + d] = osum;
      if (d == 0) {
        a.ws_ml[srow * 2] = M;
        a.ws_ml[srow * 2 + 1] = lsum;
      }
    }
  }
}

template <int D, int KVT>
hipError_t launch_gt(const KernelArgs& a, int gt, dim3 grid, hipStream_t st) {
  switch (gt) {
    case 1: hipLaunchKernelGGL((split_kernel<D, KVT, 1>), grid, dim3(kThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((split_kernel<D, KVT, 2>), grid, dim3(kThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((split_kernel<D, KVT, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((split_kernel<D, KVT, 8>), grid, dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_kv(const KernelArgs& a, int kv, int gt, dim3 grid, hipStream_t st) {
  switch (kv) {
    case DA_F32: return launch_gt<D, DA_F32>(a, gt, grid, st);
    case DA_F16: return launch_gt<D, DA_F16>(a, gt, grid, st);
    case DA_BF16: return launch_gt<D, DA_BF16>(a, gt, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split(const KernelArgs& a, int head_dim, int kv_dtype, int group_tile, hipStream_t stream) {
  const dim3 grid(a.max_splits, a.num_kv_heads, a.batch);
  switch (head_dim) {
    case 64: return launch_kv<64>(a, kv_dtype, group_tile, grid, stream);
    case 128: return launch_kv<128>(a, kv_dtype, group_tile, grid, stream);
    case 256: return launch_kv<256>(a, kv_dtype, group_tile, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace da
