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
// r = t*G + g of one contraction. A work-group takes 64 or 128 consecutive
// rows (4 wave64s, one or two groups of 16 rows each), or 16 rows (a few
// drafted tokens: wave 0 computes them, the other three waves only copy),
// and one split of the keys those rows see, K/V staged through a ring of LDS
// buffers filled by direct global -> LDS loads.
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
// Staging is described at the kernel's definition. V rows outside the
// split's attended keys (possibly NaN) are cleared in the operand; scores
// outside a row's own keys become -inf by select.
//
// Softmax precision: P enters the P.V product as f16 for f16 K/V and as a
// bf16 hi + lo pair (two products) for bf16 K/V, since one bf16 rounding of P
// alone costs more than the 1e-3 relative-L2 budget; scores, softmax state and
// accumulation are fp32. The row sums l are taken on the matrix cores from
// the same rounded P (a ones operand), so numerator and denominator use
// identical weights.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "device_common.h"
#include "kernels.h"

namespace da {
namespace {

constexpr int KT = 32;          // keys per tile
constexpr float kSlack = 8.0f;  // rescale slack of the reference max, see tile_update

typedef _Float16 mq_half8 __attribute__((ext_vector_type(8)));
typedef __bf16 mq_bf168 __attribute__((ext_vector_type(8)));
typedef float mq_float4 __attribute__((ext_vector_type(4)));
typedef float mq_float2 __attribute__((ext_vector_type(2)));
typedef _Float16 mq_half2 __attribute__((ext_vector_type(2)));
typedef __bf16 mq_bf162 __attribute__((ext_vector_type(2)));

template <int KVT>
__device__ __forceinline__ mq_float4 mfma(const uint4& a, const uint4& b, mq_float4 c) {
  if constexpr (KVT == DA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mq_half8, a), __builtin_bit_cast(mq_half8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mq_bf168, a), __builtin_bit_cast(mq_bf168, b),
                                                   c, 0, 0, 0);
}

// LDS barrier that does not wait for outstanding global loads: the next
// tile's K/V loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One lane's share of 16 query rows of a wave: the row in column `col` of
// the MFMA tiles (its q as the B operand of S^T = K Q^T, its keys within the
// split, its online-softmax state and output dims 16*nb + 4*q4 + i).
// The scale applied to raw scores in the exponents below, always positive,
// so that masked keys (raw score -inf) get probability 0 and the largest raw
// score of a row is its largest scaled score. A negative scale is folded
// into q instead: negating a 16-bit value flips its sign bit, so the raw
// score of -q is exactly minus that of q, and scale * s = |scale| * (-s)
// exactly. A zero scale makes every scaled score 0: q is zeroed (every raw
// score 0) and the unit scale gives the same scores.
__device__ __forceinline__ float positive_scale(float sl2) {
  return sl2 > 0.0f ? sl2 : (sl2 < 0.0f ? -sl2 : 1.0f);
}

template <int D>
struct RowGroup {
  uint4 qb[D / 32];
  int lo, hi;     // keys [lo, hi) of the row within the split (empty if no row)
  int64_t qrow;   // flat (sequence, token, query head) index
  bool ok;        // a real row
  float m;
  mq_float4 lsum;  // row sum of P from the matrix cores: register 0 of lane (col, k-group 0)
  mq_float4 o[D / 16];
};

template <int D>
__device__ __forceinline__ void init_rows(RowGroup<D>& g, const KernelArgs& a, int r, int r_last, int b, int kvh,
                                          int L, int t_lo, int t_hi, int q4) {
  const int T = a.query_len, G = a.group;
  g.ok = r <= r_last;
  const int t = g.ok ? r / G : 0;
  const int gh = g.ok ? r - t * G : 0;
  const int p = L - T + t;
  g.hi = p + 1 < t_hi ? p + 1 : t_hi;
  g.lo = a.window > 0 ? p + 1 - a.window : 0;
  g.lo = g.lo > t_lo ? g.lo : t_lo;
  if (!g.ok) g.hi = g.lo;
  g.qrow = (static_cast<int64_t>(b) * T + t) * a.num_q_heads + kvh * G + gh;
  // The sign of the scale is folded into q (see positive_scale).
  const uint32_t qx = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  const uint32_t qa = a.scale_log2 == 0.0f ? 0u : 0xFFFFFFFFu;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    g.qb[ks] = make_uint4(0, 0, 0, 0);
    if (g.ok) {
      const uint4 v =
          *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + (g.qrow * D + ks * 32 + q4 * 8) * 2);
      g.qb[ks] = make_uint4((v.x ^ qx) & qa, (v.y ^ qx) & qa, (v.z ^ qx) & qa, (v.w ^ qx) & qa);
    }
  }
  // A lane of no row gets the reference +inf: every slack test below passes
  // for it and its probabilities are 0 (or NaN where K holds NaN), which
  // reach only its own column of S^T and O^T, never written out.
  g.m = g.ok ? -INFINITY : INFINITY;
  g.lsum = mq_float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) g.o[nb] = mq_float4{0.0f, 0.0f, 0.0f, 0.0f};
}

// S^T of a 32-key tile for NR row groups. kop(kb, ks) returns this lane's K
// operand (16 keys x 32 dims per MFMA): keys 16*kb + col, dims 32*ks + 8*q4.
template <int D, int KVT, int NR, class KOp>
__device__ __forceinline__ void tile_scores(KOp&& kop, const RowGroup<D> (&rg)[NR], mq_float4 (&sacc)[NR][2]) {
  constexpr int NKS = D / 32;
#pragma unroll
  for (int g = 0; g < NR; ++g)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[g][kb] = mq_float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 ka = kop(kb, ks);
#pragma unroll
      for (int g = 0; g < NR; ++g) sacc[g][kb] = mfma<KVT>(ka, rg[g].qb[ks], sacc[g][kb]);
    }
  }
}

// P of one row group from its eight raw scores x (probabilities
// exp2(x * sl2 + nmu)), as the B operand of the P.V products: pairs rounded
// to nearest even and packed by one conversion each; for bf16 a hi + lo
// pair of operands.
template <int KVT>
__device__ __forceinline__ void make_p(const float (&x)[8], float sl2, float nmu, uint4& ph, uint4& pl) {
  float pr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pr[j] = exp2_fast(fmaf(x[j], sl2, nmu));
  uint32_t w[4];
  if constexpr (KVT == DA_F16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(mq_float2{pr[2 * j], pr[2 * j + 1]}, mq_half2));
    ph = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint32_t wl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(mq_float2{pr[2 * j], pr[2 * j + 1]}, mq_bf162));
      const float h0 = __builtin_bit_cast(float, w[j] << 16);
      const float h1 = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
      wl[j] = __builtin_bit_cast(uint32_t,
                                 __builtin_convertvector(mq_float2{pr[2 * j] - h0, pr[2 * j + 1] - h1}, mq_bf162));
    }
    ph = make_uint4(w[0], w[1], w[2], w[3]);
    pl = make_uint4(wl[0], wl[1], wl[2], wl[3]);
  }
}


// O^T += V^T P^T and the row sums of P for NR row groups. The sums run on
// the matrix cores (one more product per row group instead of eight
// additions per lane): a 16 x 32 operand whose row 0 is ones gives
// sum_k P[k][row] in row 0 of the result, over the rounded P that also
// enters O. vop(nb) returns this lane's V^T operand: dim 16*nb + col, the
// eight keys of its contraction positions 8*q4 .. 8*q4 + 7.
template <int D, int KVT, int NR, class VOp>
__device__ __forceinline__ void pv_products(const uint4 (&ph)[NR], const uint4 (&pl)[NR], VOp&& vop,
                                            RowGroup<D> (&rg)[NR]) {
  constexpr uint32_t one2 = KVT == DA_F16 ? 0x3C003C00u : 0x3F803F80u;
  const uint32_t o = (threadIdx.x & 15) == 0 ? one2 : 0u;
  const uint4 ones = make_uint4(o, o, o, o);
#pragma unroll
  for (int g = 0; g < NR; ++g) {
    rg[g].lsum = mfma<KVT>(ones, ph[g], rg[g].lsum);
    if constexpr (KVT != DA_F16) rg[g].lsum = mfma<KVT>(ones, pl[g], rg[g].lsum);
  }
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const uint4 va = vop(nb);
#pragma unroll
    for (int g = 0; g < NR; ++g) {
      rg[g].o[nb] = mfma<KVT>(va, ph[g], rg[g].o[nb]);
      if constexpr (KVT != DA_F16) rg[g].o[nb] = mfma<KVT>(va, pl[g], rg[g].o[nb]);
    }
  }
}

// Masking, online-softmax update and O^T += V^T P^T of a 32-key tile whose
// scores are in sacc, for NR row groups. vop(nb, full) returns this lane's
// V^T operand (as for pv_products); `full` is true when every key of the
// tile is inside every row's keys.
template <int D, int KVT, int NR, class VOp>
__device__ __forceinline__ void tile_update(mq_float4 (&sacc)[NR][2], VOp&& vop, int tb, RowGroup<D> (&rg)[NR],
                                            float sl2, int q4) {
  constexpr int NDB = D / 16;
  // Tiles inside every row's keys (all but the causal diagonal and the
  // split and window edges) skip the per-key masks: a wave-uniform branch.
  bool inside = true;
#pragma unroll
  for (int g = 0; g < NR; ++g) inside = inside && tb >= rg[g].lo && tb + 32 <= rg[g].hi;
  const bool full = __all(inside);
  uint4 ph[NR], pl[NR];  // P^T as the B operand of each row group: contraction index 8*q4 + j
#pragma unroll
  for (int g = 0; g < NR; ++g) {
    // Raw scores (the scale is applied inside the exponent's fma); keys
    // outside the row's range become -inf by select, in place.
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = tb + kb * 16 + q4 * 4 + i;
          sacc[g][kb][i] = (key >= rg[g].lo && key < rg[g].hi) ? sacc[g][kb][i] : -INFINITY;
        }
      }
    }
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sacc[g][j >> 2][j & 3];
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
    mt *= sl2;  // = the largest scaled score (sl2 > 0, see positive_scale)
    // The reference max moves only when a score exceeds it by more than
    // kSlack (base-2 units): probabilities stay below 2^kSlack, exactly
    // representable in range for f16/bf16 P and fp32 sums, and the rescale
    // of O (held in accumulation registers) is rare after the first tiles.
    // The row's reference is shared by its four lanes (one per key group),
    // and the row maximum over them is needed only when some lane's own
    // maximum exceeds the reference by more than the slack.
    if (__any(mt > rg[g].m + kSlack)) {
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const bool grow = mt > rg[g].m + kSlack;
      const float mn = grow ? mt : rg[g].m;
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2_fast(rg[g].m - mu);
      rg[g].lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < NDB; ++nb) rg[g].o[nb] *= alpha;
      rg[g].m = mn;
    }
    make_p<KVT>(x, sl2, rg[g].m == -INFINITY ? 0.0f : -rg[g].m, ph[g], pl[g]);
  }
  pv_products<D, KVT, NR>(ph, pl, [&](int nb) { return vop(nb, full); }, rg);
}

// The common tile of the row-block kernel with the LDS ring: every key
// inside every row's keys and no score above its row's reference by more
// than the slack (the caller checked both), so there is nothing to mask and
// no reference moves; the same arithmetic as tile_update.
template <int D, int KVT, int NR, class VOp>
__device__ __forceinline__ void tile_update_plain(const mq_float4 (&sacc)[NR][2], VOp&& vop, RowGroup<D> (&rg)[NR],
                                                  float sl2) {
  uint4 ph[NR], pl[NR];
#pragma unroll
  for (int g = 0; g < NR; ++g) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sacc[g][j >> 2][j & 3];
    make_p<KVT>(x, sl2, rg[g].m == -INFINITY ? 0.0f : -rg[g].m, ph[g], pl[g]);
  }
  pv_products<D, KVT, NR>(ph, pl, vop, rg);
}

// The row's l, from register 0 of the row's lane in k-group 0.
template <int D>
__device__ __forceinline__ float row_sum(const RowGroup<D>& g) {
  return __shfl(g.lsum[0], static_cast<int>(threadIdx.x & 15), 64);
}

// Write O / l (one split) or the state (m, l, O) to slot s.
template <int D>
__device__ __forceinline__ void finish_rows(const KernelArgs& a, RowGroup<D>& g, int nsplit, int s, int q4) {
  const float l = row_sum(g);
  if (!g.ok) return;
  if (nsplit == 1) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_elem(a.out, g.qrow * D + nb * 16 + q4 * 4 + i, a.out_dtype, l > 0.0f ? g.o[nb][i] * inv : 0.0f);
    }
  } else {
    const int64_t srow = g.qrow * a.max_splits + s;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
      *reinterpret_cast<mq_float4*>(a.ws_o + srow * D + nb * 16 + q4 * 4) = g.o[nb];
    if (q4 == 0) {
      a.ws_ml[srow * 2] = g.m;
      a.ws_ml[srow * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Row-block kernel with direct global -> LDS staging (head_dim 64 and 128).
//
// The K and V tiles go from HBM into LDS without passing through registers:
// global_load_lds_dwordx4 writes lane i's 16 bytes at a wave-uniform LDS
// address + 16 i, so a wave instruction fills 1 KiB (four 256-byte or eight
// 128-byte key rows). Tiles are kept in a ring of LDS stages, and every
// wave copies its own 8 keys of each tile (one page, as pages hold a
// multiple of 8 keys): one scalar page lookup and D / 32 load instructions.
//
// Layout of a stage (row blocks; the 16-row blocks keep K like V). K in
// four blocks, block w holding keys 8 w .. 8 w + 7
// (the keys wave w copies) by 16-byte segment: segment s of key k at
// position s ^ (w % 2) of 128 bytes (8 keys x 16 bytes), key k at 16 (k % 8)
// within it. The 16 lanes of a K operand read (segment 4 ks + q4 of keys
// 16 kb .. 16 kb + 15) then take two runs of 128 bytes, blocks 2 kb and
// 2 kb + 1, and the swapped positions put the two runs in opposite halves
// of the 64 four-byte banks. (K rows with permuted slots, as V below,
// measured 2-way bank conflicted on those reads.) V row-major (key rows of
// 2 D bytes), the 16-byte segment c of tile key k stored in slot
// c ^ swz(k); V^T is read with the 16-bit transposing LDS read
// (ds_read_b64_tr_b16): within each
// 16-lane group, lane i receives element i % 4 of the 8-byte rows addressed
// by lanes (i % 16) / 4 + 4 j, j = 0..3. Lane (col, q4) addresses dims
// 16 nb + 4 (col % 4) .. +3 of key 4 q4 + col / 4 (and that key + 16), so
// it receives dim 16 nb + col of keys 4 q4 + j (and 16 + 4 q4 + j): its V^T
// operand in the contraction order of the P operand.
//
// V rows outside the split's keys are not zeroed in LDS (the load cannot);
// tiles that straddle those keys clear them in the operand instead.
// ---------------------------------------------------------------------------

// Slot permutation. swz(k) >> 1 = k mod 8 differs across the 8 keys that 32
// lanes of a transposing V read address, two segments each, so those lanes
// read 32 different 8-byte units of the 64 four-byte banks: measured free of
// bank conflicts on gfx950. swz is also a bijection on k mod 8 within each
// aligned group of 8, so a wave's 8 rows of a copy land in distinct slots.
// At head_dim 64 (128-byte rows, two per 256 bytes of banks) the same two
// properties hold for the pair (row parity, slot): swz is a bijection on
// (k >> 1) mod 8 within each row parity, and its bits 1-2 equal (k >> 1)
// mod 4.
template <int D>
__device__ __forceinline__ int swz(int k) {
  if constexpr (D == 64)
    return (((k >> 1) & 3) << 1) | ((k >> 3) & 1);
  else
    return ((k & 7) << 1) | (((k >> 2) ^ (k >> 3)) & 1);
}

// One wave's 1 KiB global -> LDS copy: lane i's 16 bytes from `src` land at
// LDS byte address lds_base + 16 i (lds_base wave-uniform, passed in m0).
// The copy carries the non-temporal hint: its 1 KiB covers whole cache lines,
// each consumed by this one instruction (4-token check over the long batch,
// 64-row blocks: 582 -> 531 us; 128-token suffix unchanged, although there
// the other row blocks of a KV head re-read each tile).
// Written as inline assembly: through the compiler's builtin, its wait
// analysis (which cannot tell which LDS bytes a pending copy writes) puts a
// wait for every copy in flight before each LDS read, which would empty the
// ring on every tile. The waits are explicit instead (wait_loads), and the
// compiler's own waits stay correct: copies it does not know of only make
// its counts conservative, as loads complete in order.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(lds_base) : "memory");
}

// Wait until at most N of this wave's global loads (the copies above among
// them) are outstanding. Loads complete in order.
template <int N>
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  // (a C-style cast is the address-space conversion to a 32-bit LDS offset)
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

typedef short mq_short4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr(const uint16_t* p) {
  const mq_short4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) mq_short4*)p);
  return __builtin_bit_cast(uint2, r);
}

// Stages in the LDS ring. The 16-row blocks and head_dim 256 compute each
// tile within its own ring step: NS - 1 tiles in flight (2 and 3 stages
// measured the same; at head_dim 256 a stage holds 32 KiB and two stages keep
// two work-groups per compute unit). The pipelined row blocks (head_dim 64
// and 128) hold two tiles at once (tile m's V and tile m + 1's K): NS - 2
// tiles in flight, 4 stages (64 KiB per work-group at head_dim 128).
template <int D, bool PIPE>
constexpr int lds_stages() {
  return D >= 256 ? 2 : (PIPE ? 4 : 3);
}

template <int NS>
__device__ __forceinline__ int ring(int s, int d) {
  s += d;
  return s >= NS ? s - NS : s;
}

// FEW: blocks of 16 rows (a few drafted tokens): wave 0 computes them and
// waves 1-3 only copy their share of each tile, passing the same barrier once
// per tile.
template <int D, int KVT, int NS, int NR, bool FEW = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? (NR == 1 ? 4 : 3) : (D == 128 && NR == 1 ? 3 : 2)))) void
multi_dma_kernel(const KernelArgs a) {
  static_assert(D == 64 || D == 128 || D == 256, "row layout and slot permutation of the LDS ring");
  static_assert(!FEW || NR == 1, "16-row blocks are one row group");
  constexpr int QB = FEW ? 16 : 64 * NR;  // query rows per work-group (4 waves x NR groups of 16, or 16)
  constexpr int ROWB = D * 2;      // bytes per K/V row
  constexpr int TILE = KT * D;     // 16-bit elements per K (or V) tile
  constexpr int NSEG = D / 8;      // 16-byte segments per key row
  constexpr int KPC = 1024 / ROWB; // key rows per 1 KiB copy
  constexpr int NCP = 8 / KPC;     // copies per wave per tile and tensor
  constexpr int LOADS = 2 * NCP;   // copies per wave per tile (K and V)
  constexpr bool PIPE = !FEW && D <= 128;  // software-pipelined plain tiles
  // K in blocks (conflict-free operand reads) for the row blocks; the 16-row
  // blocks, bound by HBM, keep K in whole rows like V (whole-row copies:
  // 4-token check over the long batch 506.4 -> 512.0 us with blocks).
  constexpr bool KBLK = !FEW;
  constexpr int LEAD = PIPE ? NS - 2 : NS - 1;  // tiles in flight ahead of the one begun
  static_assert(NS == lds_stages<D, PIPE>() && LEAD >= 1, "ring");
  static_assert(NS >= 2 && 2 * NS * TILE * 2 <= 65536, "LDS ring");
  __shared__ __align__(1024) uint16_t sk[NS][TILE];
  __shared__ __align__(1024) uint16_t sv[NS][TILE];

  const int kvh = blockIdx.x;
  const int b = blockIdx.z;
  const int S = a.max_splits;
  const int rb = blockIdx.y / S;
  const int s = blockIdx.y - rb * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int q4 = lane >> 4;

  const int T = a.query_len;
  const int G = a.group;
  const int R = T * G;
  const int P = a.page_size;
  const int W = a.window;
  // Wave-uniform in a scalar register, so that every tile and range test
  // derived from it is a scalar branch.
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);

  const int r_first = rb * QB;
  if (r_first >= R) return;
  const int r_last = (r_first + QB < R ? r_first + QB : R) - 1;
  int hi_blk = L - T + r_last / G + 1;
  hi_blk = hi_blk < 0 ? 0 : hi_blk;
  int lo_blk = W > 0 ? L - T + r_first / G + 1 - W : 0;
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

  RowGroup<D> rg[NR];
#pragma unroll
  for (int g = 0; g < NR; ++g)
    init_rows(rg[g], a, r_first + (FEW ? 0 : (wave * NR + g) * 16) + col, r_last, b, kvh, L, t_lo, t_hi, q4);
  // Let the q loads land here, in a wait the compiler sees: its own wait
  // before their first use would otherwise sit inside the key loop and wait
  // for every copy in flight on each tile (vmcnt(0), other counters at
  // their maximum: the gfx9 encoding).
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // Keys inside every row of this wave: rows r0 .. r1 (tokens t0 .. t1)
  // attend [lo(t), hi(t)) with both bounds growing in t, so the common keys
  // are [lo(t1), hi(t0)); a wave without rows takes the split's keys.
  int w_lo = t_lo, w_hi = t_hi;
  {
    const int r0 = r_first + (FEW ? 0 : wave * NR * 16);
    const int r1 = r0 + (FEW ? 16 : NR * 16) - 1 < r_last ? r0 + (FEW ? 16 : NR * 16) - 1 : r_last;
    if (r0 <= r1) {
      const int t0 = r0 / G, t1 = r1 / G;
      w_hi = L - T + t0 + 1 < t_hi ? L - T + t0 + 1 : t_hi;
      if (W > 0) w_lo = L - T + t1 + 1 - W > t_lo ? L - T + t1 + 1 - W : t_lo;
    }
  }

  const int tile_first = t_lo / KT;
  const int ntiles = t_hi > t_lo ? (t_hi + KT - 1) / KT - tile_first : 0;

  // Copies: this wave's keys 8 w .. 8 w + 7 of a tile, one page (pages hold
  // a multiple of 8 keys). K in blocks: lane i of copy j takes segment
  // (8 j + i / 8) ^ (w % 2) of key i % 8, so each copy reads whole 128-byte
  // lines of 8 rows and fills K block w in the order of the layout above.
  // V (and K in rows): lane i of copy j takes key KPC j + i / NSEG and fills
  // slot i % NSEG of its row, whole rows per copy.
  const int64_t block_bytes = static_cast<int64_t>(P) * ROWB;
  const int64_t page_bytes = block_bytes * a.num_kv_heads;
  const char* kbase = static_cast<const char*>(a.k_pool) + block_bytes * kvh;
  const char* vbase = static_cast<const char*>(a.v_pool) + block_bytes * kvh;
  const int krow = lane / NSEG;
  const int slot = lane % NSEG;
  int koff[NCP], voff[NCP];
#pragma unroll
  for (int j = 0; j < NCP; ++j) {
    voff[j] = (KPC * j + krow) * ROWB + 16 * (slot ^ swz<D>(8 * wave + KPC * j + krow));
    koff[j] = KBLK ? (lane & 7) * ROWB + 16 * ((8 * j + (lane >> 3)) ^ (wave & 1)) : voff[j];
  }
  // The page table is not written while the kernel runs: reading it through
  // the constant address space lets the wave-uniform lookups below be scalar
  // loads (the copies' memory clobbers would otherwise force vector loads,
  // whose wait would also wait for every copy in flight).
  const __attribute__((address_space(4))) int32_t* table_row =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + static_cast<int64_t>(b) * a.max_pages);
  const int pi_last = phi > plo ? phi - 1 : plo;
  // Wave-uniform cursor: page and in-page position of key 8 w of the next
  // tile to load; its physical page id is read one tile ahead.
  int cpi = (tile_first * KT + 8 * wave) / P;
  int coff = tile_first * KT + 8 * wave - cpi * P;
  int cphys = 0;
  auto fetch_id = [&]() {
    int pi = cpi < plo ? plo : (cpi > pi_last ? pi_last : cpi);
    pi = pi < a.max_pages ? pi : a.max_pages - 1;
    cphys = table_row[pi];
  };
  // Copies of the next tile from the page id fetched last (fetch_id after
  // each issue, before the next).
  auto issue = [&](int stage) {
    const int64_t off = static_cast<int64_t>(cphys) * page_bytes + static_cast<int64_t>(coff) * ROWB;
    const uint32_t lk = lds_address(&sk[stage][8 * wave * D]);
    const uint32_t lv = lds_address(&sv[stage][8 * wave * D]);
#pragma unroll
    for (int j = 0; j < NCP; ++j) dma16(kbase + off + koff[j], lk + 1024 * j);
#pragma unroll
    for (int j = 0; j < NCP; ++j) dma16(vbase + off + voff[j], lv + 1024 * j);
    coff += KT;
    while (coff >= P) {
      coff -= P;
      ++cpi;
    }
  };

  // Operand addresses (16-bit elements within a stage). K in blocks: key
  // col of the half, segment 4 ks + q4, in block 2 kb + col / 8 (see the
  // layout); K in rows: row kb 16 + col, slot (4 ks + q4) ^ swz(col).
  const int kgrp = col >> 3;
  const int klane = KBLK ? kgrp * (NSEG * 64) + ((q4 ^ kgrp) * 64) + (col & 7) * 8 : col * D;
  const int kswz = swz<D>(col);
  const int vkey = 4 * q4 + (col >> 2);
  const int fv = swz<D>(vkey);
  const int vbc = (col & 3) >> 1;
  const int vh = (col & 1) * 4;
  const float sl2 = positive_scale(a.scale_log2);

  // Ring steps, shared by every wave: the begin of tile j waits for this
  // wave's copies of tile j (at most the LEAD - 1 later tiles' copies stay
  // outstanding), passes the barrier (every wave's copies of tile j have
  // landed, and every wave is done with the stage the next copy overwrites),
  // and sends out the copies of tile j + LEAD. The last tiles wait for every
  // copy, so none is left in flight.
  // The page id for the copy after that is read here, or (defer) by the
  // caller once its LDS reads are consumed: a scalar load shares the LDS
  // reads' wait counter and may complete out of order, so while one is
  // outstanding every wait for an LDS read waits for all of them.
  auto begin_copies = [&](int j, int sj, bool defer = false) {
    if (j + LEAD - 1 < ntiles)
      wait_loads<(LEAD - 1) * LOADS>();
    else
      wait_loads<0>();
    lds_barrier();
    if (j + LEAD < ntiles) {
      issue(ring<NS>(sj, LEAD));
      if (!defer) fetch_id();
    }
  };

  if constexpr (FEW) {
    if (wave != 0) {
      // Copies only, the same ring steps as the computing wave.
      if (ntiles > 0) {
        fetch_id();
#pragma unroll
        for (int k = 0; k < LEAD; ++k)
          if (k < ntiles) {
            issue(k);
            fetch_id();
          }
        int stage = 0;
        for (int m = 0; m < ntiles; ++m) {
          begin_copies(m, stage);
          stage = ring<NS>(stage, 1);
        }
      }
      return;
    }
  }
  if (ntiles > 0) {
    fetch_id();
#pragma unroll
    for (int k = 0; k < LEAD; ++k)
      if (k < ntiles) {
        issue(k);
        fetch_id();
      }
    int stage = 0;
    int m = 0;
    mq_float4 sacc[NR][2];
    uint4 vt[D / 16];
    auto scores = [&](int sj, mq_float4(&acc)[NR][2]) {
      const uint16_t* ks_ = sk[sj];
      tile_scores<D, KVT, NR>(
          [&](int kb, int kstep) {
            if constexpr (KBLK)
              return *reinterpret_cast<const uint4*>(&ks_[klane + kb * (2 * NSEG * 64) + kstep * 256]);
            else
              return *reinterpret_cast<const uint4*>(&ks_[klane + kb * 16 * D + (((4 * kstep + q4) ^ kswz) * 8)]);
          },
          rg, acc);
    };
    auto read_v = [&](int sj) {
      const uint16_t* vs_ = sv[sj];
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const uint16_t* p = &vs_[vkey * D + (((2 * nb + vbc) ^ fv) * 8) + vh];
        const uint2 lo = read_tr(p);
        const uint2 hi = read_tr(p + 16 * D);
        vt[nb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    };
    // A tile is plain when it lies inside the split's keys and inside the
    // keys of every row of this wave (wave-uniform bounds w_lo, w_hi) and no
    // score of it exceeds its row's reference by more than the slack: then
    // nothing is masked and no reference moves (tile_update_plain).
    auto is_plain = [&](int tb, const mq_float4(&sc)[NR][2]) {
      if (tb < w_lo || tb + KT > w_hi) return false;
      bool ok = true;
#pragma unroll
      for (int g = 0; g < NR; ++g) {
        float mt = sc[g][0][0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sc[g][j >> 2][j & 3]);
        ok = ok & (mt * sl2 <= rg[g].m + kSlack);
      }
      return static_cast<bool>(__all(ok));
    };
    // Waves whose rows all lie past the block's last row compute too (on
    // zero q; nothing of theirs is written): a branch around the work would
    // put every accumulator through a join, and the compiler then copies
    // them on each tile. Likewise the tiles that need masks or move a
    // reference leave the plain loop for the general update below, so that
    // the plain loop carries O only through its matrix products.
    // Wave priority by progress: 3 for the first quarter of this wave's
    // tiles, down to 0 for the last. The two work-groups sharing a compute
    // unit start together with about equal work; the issue arbiter favours
    // the older waves, so without this the second one falls behind and then
    // runs alone at one wave per SIMD (its end 12 us after its partner's on
    // the 128-token suffix). A wave that lags keeps the higher priority.
    // Measured (split pass, us): 32-token suffix 34.0 -> 32.5, head_dim 64
    // suffix 51.4 -> 49.2, 512-token suffix 255.4 -> 248.7, the 4-token check
    // 506.3 -> 496.6, 64 query heads over the long batch 492.6 -> 484.5; the
    // 128-token suffix 81.4 -> 82.3 (its step 92.8 -> 91.8). Priorities by
    // the remaining tiles of a full split measured the same or slower.
    int plev = 3;
    int pnext = ntiles >> 2;
    __builtin_amdgcn_s_setprio(3);
    auto lower_prio = [&]() {
      if (m >= pnext) {
        --plev;
        pnext = plev == 2 ? (ntiles >> 1) : (plev == 1 ? 3 * (ntiles >> 2) : 0x7FFFFFFF);
        if (plev == 2)
          __builtin_amdgcn_s_setprio(2);
        else if (plev == 1)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
    };
    while (m < ntiles) {
      begin_copies(m, stage);
      scores(stage, sacc);
      if constexpr (PIPE) {
        // Software pipeline over plain tiles followed by another tile: tile
        // m + 1 is begun and its S^T products go out together with tile m's
        // softmax and P.V products (tile m's V and tile m + 1's K are both
        // resident: LEAD = NS - 2). Unrolled by two with the score
        // registers alternating, so that no scores are copied per tile.
        mq_float4 sb[NR][2];
        auto step = [&](mq_float4(&cur)[NR][2], mq_float4(&nxt)[NR][2]) {
          const int sn = ring<NS>(stage, 1);
          begin_copies(m + 1, sn, true);
          read_v(stage);
          scores(sn, nxt);
          tile_update_plain<D, KVT, NR>(cur, [&](int nb) { return vt[nb]; }, rg, sl2);
          // Scheduling groups for this block: the next tile's K operand
          // reads first, then each S^T product with three vector
          // instructions and one V^T read, then the P.V products. What the
          // compiler makes of them (it puts this tile's softmax ahead of the
          // products) measured 3-4 % faster than its own order and than a
          // strict one-product-one-exponential interleave (128-token suffix
          // 84.6 / 81.5 / 83.0 us, 512-token suffix 251 / 251 / 258 us).
          __builtin_amdgcn_sched_group_barrier(0x100, 4 * NR, 0);
#pragma unroll
          for (int i = 0; i < 8 * NR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 9 * NR, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (m + 1 + LEAD < ntiles) fetch_id();
          stage = sn;
          ++m;
          lower_prio();
        };
        for (;;) {
          if (m + 1 >= ntiles || !is_plain((tile_first + m) * KT, sacc)) break;
          step(sacc, sb);
          if (m + 1 >= ntiles || !is_plain((tile_first + m) * KT, sb)) {
#pragma unroll
            for (int g = 0; g < NR; ++g) {
              sacc[g][0] = sb[g][0];
              sacc[g][1] = sb[g][1];
            }
            break;
          }
          step(sb, sacc);
        }
      } else {
        for (;;) {
          if (!is_plain((tile_first + m) * KT, sacc)) break;
          read_v(stage);
          tile_update_plain<D, KVT, NR>(sacc, [&](int nb) { return vt[nb]; }, rg, sl2);
          stage = ring<NS>(stage, 1);
          ++m;
          lower_prio();
          if (m >= ntiles) break;
          begin_copies(m, stage);
          scores(stage, sacc);
        }
      }
      if (m >= ntiles) break;
      // Tile m, begun and scored: V rows of keys outside [t_lo, t_hi) may
      // hold anything, so tiles that straddle those keys clear them in the
      // operand (keys 4 q4 + j and 16 + 4 q4 + j, two per dword); then the
      // general update with masks and reference moves.
      read_v(stage);
      const int tb = (tile_first + m) * KT;
      if (tb < t_lo || tb + KT > t_hi) {
        uint32_t vmask[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int k0 = tb + (d >> 1) * 16 + 4 * q4 + (d & 1) * 2;
          vmask[d] = ((k0 >= t_lo && k0 < t_hi) ? 0x0000FFFFu : 0u) |
                     ((k0 + 1 >= t_lo && k0 + 1 < t_hi) ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          vt[nb].x &= vmask[0];
          vt[nb].y &= vmask[1];
          vt[nb].z &= vmask[2];
          vt[nb].w &= vmask[3];
        }
      }
      tile_update<D, KVT, NR>(sacc, [&](int nb, bool) { return vt[nb]; }, tb, rg, sl2, q4);
      stage = ring<NS>(stage, 1);
      ++m;
    }
  }
#pragma unroll
  for (int g = 0; g < NR; ++g) finish_rows(a, rg[g], nsplit, s, q4);
}

template <int D, int KVT>
hipError_t launch_nq(const KernelArgs& a, int rows, dim3 grid, hipStream_t st) {
  if (rows == 16) {
    hipLaunchKernelGGL((multi_dma_kernel<D, KVT, lds_stages<D, false>(), 1, true>), grid, dim3(256), 0, st, a);
  } else if (rows == 64) {
    hipLaunchKernelGGL((multi_dma_kernel<D, KVT, lds_stages<D, D <= 128>(), 1>), grid, dim3(256), 0, st, a);
  } else if (rows == 128) {
    if constexpr (D <= 128)
      hipLaunchKernelGGL((multi_dma_kernel<D, KVT, lds_stages<D, true>(), 2>), grid, dim3(256), 0, st, a);
    else
      return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
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
