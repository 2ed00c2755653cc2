// Split pass of attention for several new tokens per sequence over the paged
// cache (suffix prefill, or checking several drafted tokens), for gfx950.
//
// llm-web pull 8, commit on the batched suffix prefill: the new tokens of a
// prompt whose prefix is already cached are processed together; their K/V are
// written after the resident prefix and their attention reads the cache. Here
// sequence b holds L_b keys of which the last T are the new tokens; new token
// t sits at position p = L_b - T + t and attends keys [max(0, p+1-W), p+1)
// (all keys up to itself, or the last W of them with a window).
//
// Query rows. The T*G (token, head) pairs that share KV head j form the rows
// r = t*G + g of one contraction; a work-group takes QB = 16*NQ consecutive
// rows (NQ wave64s, 16 rows each) and one split of the keys those rows see.
// Both products run on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16}):
//   S^T = K Q^T    A = 16 keys x 32 dims of K,  B = 32 dims x 16 rows of q
//   O^T += V^T P^T A = 16 dims x 32 keys of V,  B = 32 keys x 16 rows of P
// so a lane holds the scores of one query row (its column of S^T) and the
// output dims of that same row (its column of O^T): the online-softmax state
// of a row lives in the four lanes that share its column, and the rescale of
// O needs no data movement. The 32 keys of a tile enter the P.V contraction in
// the order that lets each lane pass its own eight probabilities as its B
// operand: contraction index 8*q + j is key 4q + j (j < 4) or 16 + 4q + j - 4.
//
// Staging. Each tile of 32 keys is read from HBM once per work-group with
// 16-byte loads into registers (the next tile's loads are in flight while the
// current tile is computed) and written to LDS: K row-major, V transposed
// (dims as rows, keys in contraction order) so both MFMA operands are single
// 16-byte LDS reads. V rows outside the split's attended keys are stored as
// zeros (they may hold NaN and would poison 0 * V), scores outside a row's own
// keys become -inf by select.
//
// Softmax precision: P enters the P.V product as f16 for f16 K/V and as a
// bf16 hi + lo pair (two products) for bf16 K/V, since one bf16 rounding of P
// alone costs more than the 1e-3 relative-L2 budget; scores, softmax state and
// accumulation are fp32.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "device_common.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int KT = 32;   // keys per tile
constexpr int KPAD = 8;  // LDS padding (16-bit elements) per K row
constexpr int VPAD = 8;  // LDS padding per transposed V row

typedef _Float16 mq_half8 __attribute__((ext_vector_type(8)));
typedef __bf16 mq_bf168 __attribute__((ext_vector_type(8)));
typedef float mq_float4 __attribute__((ext_vector_type(4)));

template <int KVT>
__device__ __forceinline__ mq_float4 mfma(const uint4& a, const uint4& b, mq_float4 c) {
  if constexpr (KVT == DA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mq_half8, a), __builtin_bit_cast(mq_half8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mq_bf168, a), __builtin_bit_cast(mq_bf168, b),
                                                   c, 0, 0, 0);
}

// Contraction position of key k (0..31) of a tile in the P.V product.
__device__ __forceinline__ int kpos(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }

// Round to nearest even: f32 -> f16 bits / bf16 bits.
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite inputs only (probabilities)
}

// LDS barrier that does not wait for outstanding global loads: the next
// tile's K/V loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int KVT, int NQ>
__global__ __launch_bounds__(64 * NQ) void multi_kernel(const KernelArgs a) {
  constexpr int NT = 64 * NQ;           // threads
  constexpr int QB = 16 * NQ;           // query rows per work-group
  constexpr int ROWB = D * 2;           // bytes per K/V row
  constexpr int ROWV = D / 8;           // 16-byte vectors per row
  constexpr int NV = KT * ROWV / NT;    // vectors per thread per tensor per tile
  constexpr int KSTEP = NT / ROWV;      // key distance between a thread's vectors
  constexpr int KS = D + KPAD;          // K row stride in LDS (elements)
  constexpr int VS = KT + VPAD;         // transposed-V row stride (elements)
  constexpr int NKS = D / 32;           // k-steps of q.K
  constexpr int NDB = D / 16;           // 16-dim blocks of P.V
  static_assert(NV >= 1 && NV * NT == KT * ROWV && NT % ROWV == 0, "staging split");
  __shared__ __align__(16) uint16_t sk[KT * KS];
  __shared__ __align__(16) uint16_t sv[D * VS];

  const int kvh = blockIdx.x;
  const int b = blockIdx.z;
  const int S = a.max_splits;
  const int rb = blockIdx.y / S;
  const int s = blockIdx.y - rb * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // query row within the wave's 16
  const int q4 = lane >> 4;   // k-group of the MFMA operands

  const int T = a.query_len;
  const int G = a.group;
  const int R = T * G;
  const int P = a.page_size;
  const int W = a.window;
  const int L = a.seq_lens[b];

  // Rows of this work-group and the keys any of them sees: [lo_blk, hi_blk).
  const int r_first = rb * QB;
  if (r_first >= R) return;
  const int r_last = (r_first + QB < R ? r_first + QB : R) - 1;
  const int t_min = r_first / G;
  const int t_max = r_last / G;
  int hi_blk = L - T + t_max + 1;
  hi_blk = hi_blk < 0 ? 0 : hi_blk;
  int lo_blk = W > 0 ? L - T + t_min + 1 - W : 0;
  lo_blk = lo_blk < 0 ? 0 : (lo_blk > hi_blk ? hi_blk : lo_blk);
  const int pf = lo_blk / P;
  const int pe = (hi_blk + P - 1) / P;
  const int cp = a.pages_per_split;
  int nsplit = (pe - pf + cp - 1) / cp;
  nsplit = nsplit < 1 ? 1 : (nsplit > S ? S : nsplit);
  if (s >= nsplit) return;  // whole work-group, uniform
  const int plo = pf + s * cp;
  const int phi = plo + cp < pe ? plo + cp : pe;
  const int t_lo = lo_blk > plo * P ? lo_blk : plo * P;
  const int t_hi = hi_blk < phi * P ? hi_blk : phi * P;

  // This lane's query row and its own keys within the split.
  const int r = r_first + wave * 16 + col;
  const bool row_ok = r <= r_last;
  const int t = row_ok ? r / G : 0;
  const int g = row_ok ? r - t * G : 0;
  const int p_r = L - T + t;
  int hi_r = p_r + 1 < t_hi ? p_r + 1 : t_hi;
  int lo_r = W > 0 ? p_r + 1 - W : 0;
  lo_r = lo_r > t_lo ? lo_r : t_lo;
  if (!row_ok) hi_r = lo_r;  // no keys
  const int64_t qrow = (static_cast<int64_t>(b) * T + t) * a.num_q_heads + kvh * G + g;

  // q as the B operand of S^T = K Q^T: dims 32*ks + 8*q4 .. +8 of this row.
  uint4 qb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qb[ks] = make_uint4(0, 0, 0, 0);
    if (row_ok)
      qb[ks] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + (qrow * D + ks * 32 + q4 * 8) * 2);
  }

  float m = -INFINITY, lpart = 0.0f;
  mq_float4 o[NDB];
#pragma unroll
  for (int nb = 0; nb < NDB; ++nb) o[nb] = mq_float4{0.0f, 0.0f, 0.0f, 0.0f};

  const int tile_first = t_lo / KT;
  const int ntiles = t_hi > t_lo ? (t_hi + KT - 1) / KT - tile_first : 0;

  // Staging: thread vector i covers key kk0 + i*KSTEP of the tile, 16-byte
  // segment `seg` of its row. Page cursor per vector, page ids fetched one
  // tile ahead, indices clamped to this split's pages.
  const int seg = tid % ROWV;
  const int kk0 = tid / ROWV;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int64_t block_bytes = static_cast<int64_t>(P) * ROWB;
  const int64_t page_bytes = block_bytes * a.num_kv_heads;
  const int64_t head_bytes = block_bytes * kvh + seg * 16;
  const int32_t* table_row = a.page_table + static_cast<int64_t>(b) * a.max_pages;
  const int pi_last = phi > plo ? phi - 1 : plo;
  int cpi[NV], coff[NV], cphys[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int pos = tile_first * KT + kk0 + i * KSTEP;
    cpi[i] = pos / P;
    coff[i] = pos - cpi[i] * P;
  }
  auto fetch_ids = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int pi = cpi[i] < plo ? plo : (cpi[i] > pi_last ? pi_last : cpi[i]);
      pi = pi < a.max_pages ? pi : a.max_pages - 1;
      cphys[i] = table_row[pi];
    }
  };
  auto advance = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      coff[i] += KT;
      while (coff[i] >= P) {
        coff[i] -= P;
        cpi[i] += 1;
      }
    }
  };
  uint4 rk[NV], rv[NV];
  auto issue = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int64_t off = static_cast<int64_t>(cphys[i]) * page_bytes + head_bytes +
                          static_cast<int64_t>(coff[i]) * ROWB;
      rk[i] = load16(kbase + off);
      rv[i] = load16(vbase + off);
    }
    advance();
    fetch_ids();
  };
  // Registers -> LDS: K row-major, V transposed into contraction order, V
  // rows outside [t_lo, t_hi) as zeros.
  auto stage = [&](int tb) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int kk = kk0 + i * KSTEP;
      *reinterpret_cast<uint4*>(&sk[kk * KS + seg * 8]) = rk[i];
      const int pos = tb + kk;
      const bool live = pos >= t_lo && pos < t_hi;
      const uint32_t w[4] = {live ? rv[i].x : 0u, live ? rv[i].y : 0u, live ? rv[i].z : 0u, live ? rv[i].w : 0u};
      const int kp = kpos(kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[(seg * 8 + 2 * e) * VS + kp] = static_cast<uint16_t>(w[e] & 0xFFFFu);
        sv[(seg * 8 + 2 * e + 1) * VS + kp] = static_cast<uint16_t>(w[e] >> 16);
      }
    }
  };

  const float sl2 = a.scale_log2;
  auto compute = [&](int tb) {
    // S^T for keys tb + 16*kb + 4*q4 + i of this lane's row.
    mq_float4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = mq_float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&sk[(kb * 16 + col) * KS + ks * 32 + q4 * 8]);
        sacc[kb] = mfma<KVT>(ka, qb[ks], sacc[kb]);
      }
    }
    float x[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = tb + kb * 16 + q4 * 4 + i;
        const float v = sacc[kb][i] * sl2;
        x[kb * 4 + i] = (key >= lo_r && key < hi_r) ? v : -INFINITY;
      }
    }
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    if (__any(mn > m)) {
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2_fast(m - mu);
      lpart *= alpha;
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) o[nb] *= alpha;
      m = mn;
    }
    const float mu = m == -INFINITY ? 0.0f : m;
    float pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = exp2_fast(x[j] - mu);
      lpart += pr[j];
    }
    // P^T as the B operand: contraction index 8*q4 + j holds pr[j].
    if constexpr (KVT == DA_F16) {
      uint4 pb;
      pb.x = f16_bits(pr[0]) | (f16_bits(pr[1]) << 16);
      pb.y = f16_bits(pr[2]) | (f16_bits(pr[3]) << 16);
      pb.z = f16_bits(pr[4]) | (f16_bits(pr[5]) << 16);
      pb.w = f16_bits(pr[6]) | (f16_bits(pr[7]) << 16);
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) {
        const uint4 va = *reinterpret_cast<const uint4*>(&sv[(nb * 16 + col) * VS + q4 * 8]);
        o[nb] = mfma<KVT>(va, pb, o[nb]);
      }
    } else {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hi[j] = bf16_bits(pr[j]);
        lo[j] = bf16_bits(pr[j] - __builtin_bit_cast(float, hi[j] << 16));
      }
      uint4 ph, pl;
      ph.x = hi[0] | (hi[1] << 16);
      ph.y = hi[2] | (hi[3] << 16);
      ph.z = hi[4] | (hi[5] << 16);
      ph.w = hi[6] | (hi[7] << 16);
      pl.x = lo[0] | (lo[1] << 16);
      pl.y = lo[2] | (lo[3] << 16);
      pl.z = lo[4] | (lo[5] << 16);
      pl.w = lo[6] | (lo[7] << 16);
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) {
        const uint4 va = *reinterpret_cast<const uint4*>(&sv[(nb * 16 + col) * VS + q4 * 8]);
        o[nb] = mfma<KVT>(va, ph, o[nb]);
        o[nb] = mfma<KVT>(va, pl, o[nb]);
      }
    }
  };

  if (ntiles > 0) {
    fetch_ids();
    issue();
    for (int n = 0; n < ntiles; ++n) {
      const int tb = (tile_first + n) * KT;
      lds_barrier();  // every wave is done reading the previous tile
      stage(tb);
      if (n + 1 < ntiles) issue();
      lds_barrier();  // the tile is in LDS
      compute(tb);
    }
  }

  // The row's l is split over its four lanes (one per key group).
  float l = lpart + __shfl_xor(lpart, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (!row_ok) return;
  if (nsplit == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_elem(a.out, qrow * D + nb * 16 + q4 * 4 + i, a.out_dtype, l > 0.0f ? o[nb][i] * inv : 0.0f);
    }
  } else {
    const int64_t srow = qrow * S + s;
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb)
      *reinterpret_cast<mq_float4*>(a.ws_o + srow * D + nb * 16 + q4 * 4) = o[nb];
    if (q4 == 0) {
      a.ws_ml[srow * 2] = m;
      a.ws_ml[srow * 2 + 1] = l;
    }
  }
}

template <int D, int KVT>
hipError_t launch_nq(const KernelArgs& a, int rows, dim3 grid, hipStream_t st) {
  switch (rows) {
    case 32: hipLaunchKernelGGL((multi_kernel<D, KVT, 2>), grid, dim3(128), 0, st, a); break;
    case 64: hipLaunchKernelGGL((multi_kernel<D, KVT, 4>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_kv(const KernelArgs& a, int kv, int rows, dim3 grid, hipStream_t st) {
  switch (kv) {
    case DA_F16: return launch_nq<D, DA_F16>(a, rows, grid, st);
    case DA_BF16: return launch_nq<D, DA_BF16>(a, rows, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_multi(const KernelArgs& a, int head_dim, int kv_dtype, int rows_per_group, hipStream_t stream) {
  const int R = a.query_len * a.group;
  const int nrb = (R + rows_per_group - 1) / rows_per_group;
  const dim3 grid(a.num_kv_heads, nrb * a.max_splits, a.batch);
  switch (head_dim) {
    case 64: return launch_kv<64>(a, kv_dtype, rows_per_group, grid, stream);
    case 128: return launch_kv<128>(a, kv_dtype, rows_per_group, grid, stream);
    case 256: return launch_kv<256>(a, kv_dtype, rows_per_group, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace da
