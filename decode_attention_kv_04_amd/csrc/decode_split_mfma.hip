// Split pass of paged decode attention for gfx950, q.K on the matrix cores.
//
// Same work decomposition, streaming and epilogue as the vector split kernel
// (one work-group of four wave64s per (split, KV head, sequence); each K/V row
// read once for the G query heads of its GQA group, as in mlx-runner pull 3,
// GQA-shared split attention commit; per-split online-softmax states merged
// later, as in TVM pull 20426, sharded-nest commit message). Here the scores
// of a 16-key tile for all G heads are one chain of D/32
// v_mfma_f32_16x16x32_{f16,bf16} (A = 16 keys x 32 dims of K, B = 32 dims x
// 16 heads of q, fp32 accumulation): q.K is a real small dense contraction
// once G heads share the keys, so it leaves the vector ALUs, and no lane sum
// is needed.
//
// Lane layout (wave64; lane = 16*r + c):
//  * MFMA row m (lane c of the A operand) holds key (m % 4) * 4 + m / 4 of
//    the tile, so the result register i of lane (r, c) is the score of key
//    4*i + r for head c.
//  * V is read in rows: lane (r, c) holds row 4*i + r (i = 0..3) of the tile,
//    elements [v*128 + 8c, +8) for v < D/128, so one wave-wide load covers
//    four whole rows.
//  * K is read the same way (whole rows, four per load) and rearranged into
//    the operand layout through a per-wave LDS tile: loaded straight in
//    operand layout, each instruction would take 64 bytes of each of 16 rows,
//    and that pattern streams slower (a probe over shuffled 4 KiB blocks with
//    non-temporal loads: 5.85 TB/s against 6.5-6.6 for whole rows; this
//    kernel on the long batch: 504.8 -> 494.2 us per launch).
//  * Hence each lane already holds the scores of exactly the keys whose V rows
//    it holds; the online-softmax state (m, l) of head g and row slot r lives
//    in lane (r, g), and P and the rescale factors reach the P.V lanes of the
//    row slot with a DPP row broadcast. O (G x D/16 floats per lane) stays in
//    VGPRs; row slots and waves are merged once at the end.
//
// Used when q and K/V share a 16-bit type, D is 128 and the page size is a
// multiple of 16 (a 16-key tile then never straddles pages).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "device_common.h"
#include "kernels.h"
#include "plan.h"

#ifndef DA_MFMA_PREFETCH_TILES
#define DA_MFMA_PREFETCH_TILES 1
#endif

namespace da {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPD = DA_MFMA_PREFETCH_TILES;  // tiles in flight per wave while one is computed
constexpr float kRescaleSlack = DA_RESCALE_SLACK;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int KVT>
__device__ __forceinline__ float4_t mfma_16x16x32(const uint4& a, const uint4& b, float4_t c) {
  if constexpr (KVT == DA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a), __builtin_bit_cast(bf168_t, b),
                                                    c, 0, 0, 0);
}

// Broadcast lane g (g < GT) of each 16-lane row: out[g] = x of lane (r, g).
template <int GT>
__device__ __forceinline__ void row_bcast_all(float x, float* out) {
  out[0] = row_bcast<0>(x);
  if constexpr (GT > 1) out[1] = row_bcast<1>(x);
  if constexpr (GT > 2) {
    out[2] = row_bcast<2>(x);
    out[3] = row_bcast<3>(x);
  }
  if constexpr (GT > 4) {
    out[4] = row_bcast<4>(x);
    out[5] = row_bcast<5>(x);
    out[6] = row_bcast<6>(x);
    out[7] = row_bcast<7>(x);
  }
}

// Schedules of the split pass (the MODE template parameter):
//  kGrid      work-group (KV head, s, sequence) computes split s of that
//             (sequence, KV head) stream: pages_per_split pages from the
//             first attended page on;
//  kFixed     fixed-order mode: chunks_per_group consecutive chunks per
//             work-group, one state per chunk (a chunk's state depends only
//             on its keys);
//  kBalanced  work-group w computes units [w q, (w + 1) q), q =
//             pages_per_split, of the batch's (sequence, KV head) streams in
//             order, each weighing bal_overhead units and then one per
//             attended page (an empty stream one page), one state per piece
//             of a stream; the work-group holding a stream's first page
//             records its piece count for the combine.
constexpr int kGrid = 0;
constexpr int kFixed = 1;
constexpr int kBalanced = 2;

template <int D, int KVT, int GT, int MODE>
__global__ __launch_bounds__(kThreads) void split_kernel_mfma(const KernelArgs a) {
  static_assert(KVT == DA_F16 || KVT == DA_BF16, "matrix-core path needs a 16-bit KV type");
  static_assert(D == 128, "head_dim (256 does not fit the register budget in this layout)");
  static_assert(GT <= 8, "group width");
  constexpr int ELT = 2;
  constexpr int E = 8;          // elements per 16-byte vector
  constexpr int NJ = D / 32;    // MFMA k-steps per tile
  constexpr int DPL = D / 16;   // V elements per lane per row
  constexpr int VPL = DPL / E;  // V vectors per lane per row
  constexpr int SEG = 16 * E;   // elements per V row segment
  constexpr int TR = 16;        // keys per tile
  constexpr int RB = D * ELT;   // bytes per row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4;  // row slot / MFMA k-group
  const int c = lane & 15;  // column: head c of the scores, MFMA row of K
  const int key_of_lane = (c & 3) * 4 + (c >> 2);
  const int P = a.page_size;
  const int G = a.group;

  // q of head c of the group of KV head kvh in sequence b, as the B operand:
  // dims [32j + 8r, +8) for k-step j.
  auto load_q = [&](int b, int kvh, uint4 (&qb)[NJ]) {
    const int64_t qrow0 = static_cast<int64_t>(b) * a.rows_per_seq + a.row_base + kvh * G;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      qb[j] = make_uint4(0, 0, 0, 0);
      if (c < G)
        qb[j] =
            *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + ((qrow0 + c) * D + 32 * j + 8 * r) * ELT);
    }
  };

  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int64_t block_bytes = static_cast<int64_t>(P) * RB;
  const int64_t page_bytes = block_bytes * a.num_kv_heads;
  const uint32_t v_lane_off = static_cast<uint32_t>(r * RB + c * E * ELT);

  // K of the tile being computed, per wave: 16 rows of 16-byte slots, slot s
  // of row k stored at s ^ k, so the 16 lanes of a row write and the 16
  // lanes of an operand read (one slot of each of 16 rows) touch 16 different
  // slots. (The counters still show bank conflicts on this tile, 40 % of the
  // LDS-active cycles; 17-slot rows instead of the XOR measured the same
  // time, so they are off the critical path.)
  constexpr int NSL = D / 8;
  static_assert(NSL == TR, "slot permutation by row needs as many slots as rows");
  __shared__ uint4 sh_k[kWaves][TR][NSL];
  __shared__ float sh_o[kWaves][GT][D];
  __shared__ float sh_m[kWaves][GT];
  __shared__ float sh_l[kWaves][GT];

  // Keys [t_lo, t_hi) of the stream (sequence b, KV head kvh), held in its
  // logical pages [plo, phi): the four waves' tile loop, the merge of their
  // states, then either the output rows (direct: the stream has no other
  // piece) or the state (m, l, O) of every head in workspace slot `slot`.
  auto process = [&](int b, int kvh, const uint4 (&qb)[NJ], int plo, int phi, int t_lo, int t_hi, bool direct,
                     int slot) {
    const int64_t qrow0 = static_cast<int64_t>(b) * a.rows_per_seq + a.row_base + kvh * G;
    const int64_t head_bytes = block_bytes * kvh;
    const int32_t* table_row = a.page_table + static_cast<int64_t>(b) * a.max_pages;

    float m = -INFINITY, l = 0.0f;  // head c, row slot r
    float o[GT][DPL];
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[g][i] = 0.0f;

    const int tile_first = t_lo / TR;
    const int tile_end = (t_hi + TR - 1) / TR;
    const int my_first = tile_first + wave;
    const int ntiles = my_first < tile_end ? (tile_end - my_first + kWaves - 1) / kWaves : 0;

    struct Tile {
      uint4 k[NJ];
      uint4 v[4][VPL];
    };

    // Load cursor (one page per tile: P is a multiple of 16).
    constexpr int STEP = kWaves * TR;
    const int step_p = STEP / P;
    const int step_r = STEP - step_p * P;
    const int pi_last = phi > plo ? phi - 1 : plo;
    int cur_pi = (my_first * TR) / P;
    int cur_off = my_first * TR - cur_pi * P;
    int cur_phys = 0;
    auto fetch_id = [&]() {
      const int pi = cur_pi < plo ? plo : (cur_pi > pi_last ? pi_last : cur_pi);
      cur_phys = table_row[pi];
    };
    auto issue = [&](Tile& t) {
      const int64_t off = static_cast<int64_t>(cur_phys) * page_bytes + head_bytes + static_cast<int64_t>(cur_off) * RB;
      const char* kp = kbase + off + v_lane_off;
      const char* vp = vbase + off + v_lane_off;
#pragma unroll
      for (int j = 0; j < NJ; ++j) t.k[j] = load16(kp + 4 * j * RB);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < VPL; ++v) t.v[i][v] = load16(vp + 4 * i * RB + v * SEG * ELT);
      cur_pi += step_p;
      cur_off += step_r;
      if (cur_off >= P) {
        cur_off -= P;
        cur_pi += 1;
      }
      fetch_id();
    };

    const float sl2 = a.scale_log2;
    // One tile. FULL: every row of the tile is attended (no masking at all);
    // otherwise rows outside [t_lo, t_hi) get score -inf and zero V rows.
    auto compute = [&](const Tile& t, int tile, auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      const int tb = tile * TR;
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      // The previous tile's operand reads of sh_k come before these writes,
      // and the writes (rows of four lanes' loads each) before the operand
      // reads, which gather one slot of 16 rows written by other lanes.
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < NJ; ++j) sh_k[wave][4 * j + r][c ^ (4 * j + r)] = t.k[j];
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc = mfma_16x16x32<KVT>(sh_k[wave][key_of_lane][(4 * j + r) ^ key_of_lane], qb[j], acc);
      bool valid[4];
      float x[4];  // scores in base-2 units
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (FULL) {
          valid[i] = true;
          x[i] = acc[i] * sl2;
        } else {
          const int tok = tb + 4 * i + r;
          valid[i] = tok >= t_lo && tok < t_hi;
          x[i] = valid[i] ? acc[i] * sl2 : -INFINITY;
        }
      }
      const float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      // The reference max moves only past the rescale slack.
      const float mn = mt > m + kRescaleSlack ? mt : m;
      // P.V for this tile given the running max (p = 2^(x - m)).
      auto accumulate = [&]() {
        const float mu = (m == -INFINITY) ? 0.0f : m;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = exp2_fast(x[i] - mu);
        l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pb[GT];
          row_bcast_all<GT>(p[i], pb);
          if constexpr (FULL) {
            // Each V element is widened inside its FMA (v_fma_mix for fp16).
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
              const uint32_t w[4] = {t.v[i][v].x, t.v[i][v].y, t.v[i][v].z, t.v[i][v].w};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                  o[g][v * E + 2 * k] = fmaf(pb[g], lo16_to_f32<KVT>(w[k]), o[g][v * E + 2 * k]);
                  o[g][v * E + 2 * k + 1] = fmaf(pb[g], hi16_to_f32<KVT>(w[k]), o[g][v * E + 2 * k + 1]);
                }
              }
            }
          } else {
            float vf[DPL];
#pragma unroll
            for (int v = 0; v < VPL; ++v) unpack<KVT>(t.v[i][v], vf + v * E);
#pragma unroll
            for (int e = 0; e < DPL; ++e) vf[e] = valid[i] ? vf[e] : 0.0f;
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
              for (int e = 0; e < DPL; ++e) o[g][e] = fmaf(pb[g], vf[e], o[g][e]);
          }
        }
      };
      // O and l are rescaled only when some running max of the wave grew; the
      // accumulation is written out in both arms so that the common arm keeps
      // O in place.
      if (__any(c < G && mn > m)) {
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float alpha = exp2_fast(m - mu);
        l *= alpha;
        m = mn;
        float ab[GT];
        row_bcast_all<GT>(alpha, ab);
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
          for (int i = 0; i < DPL; ++i) o[g][i] *= ab[g];
        accumulate();
      } else {
        accumulate();
      }
    };
    auto compute_tile = [&](const Tile& t, int tile) {
      const int tb = tile * TR;
      if (tb >= t_lo && tb + TR <= t_hi)
        compute(t, tile, std::true_type());
      else
        compute(t, tile, std::false_type());
    };

    // Ring of kPD + 1 tiles, steady state with unconditional loads, unrolled
    // drain (as in the vector kernel).
    if (ntiles > 0) {
      Tile buf[kPD + 1];
      fetch_id();
#pragma unroll
      for (int k = 0; k < kPD; ++k)
        if (k < ntiles) issue(buf[k]);
      int n = 0;
      while (n + 2 * kPD < ntiles) {
#pragma unroll
        for (int j = 0; j <= kPD; ++j) {
          issue(buf[(j + kPD) % (kPD + 1)]);
          compute_tile(buf[j], my_first + (n + j) * kWaves);
        }
        n += kPD + 1;
      }
#pragma unroll
      for (int j = 0; j < 2 * kPD; ++j) {
        if (n + j < ntiles) {
          if (n + j + kPD < ntiles) issue(buf[(j + kPD) % (kPD + 1)]);
          compute_tile(buf[j % (kPD + 1)], my_first + (n + j) * kWaves);
        }
      }
    }

    // Every lane of row slot r takes (m, l) of each head g from lane (r, g);
    // then the four row slots are merged with lane shuffles.
    float mb[GT], lb[GT];
    row_bcast_all<GT>(m, mb);
    row_bcast_all<GT>(l, lb);
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float m2 = __shfl_xor(mb[g], off, 64);
        const float l2 = __shfl_xor(lb[g], off, 64);
        float o2[DPL];
#pragma unroll
        for (int i = 0; i < DPL; ++i) o2[i] = __shfl_xor(o[g][i], off, 64);
        merge_into<DPL>(mb[g], lb[g], o[g], m2, l2, o2);
      }
    }

    // Merge the four waves through LDS and write the result.
    if (r == 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int v = 0; v < VPL; ++v)
#pragma unroll
          for (int e = 0; e < E; ++e) sh_o[wave][g][v * SEG + c * E + e] = o[g][v * E + e];
      if (c == 0) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          sh_m[wave][g] = mb[g];
          sh_l[wave][g] = lb[g];
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
      const int64_t row = qrow0 + g;
      if (direct) {
        store_elem(a.out, row * D + d, a.out_dtype, lsum > 0.0f ? osum / lsum : 0.0f);
      } else {
        const int64_t srow = row * a.max_splits + slot;
        a.ws_o[srow * D + d] = osum;
        if (d == 0) {
          a.ws_ml[srow * 2] = M;
          a.ws_ml[srow * 2 + 1] = lsum;
        }
      }
    }
  };

  if constexpr (MODE == kBalanced) {
    // Each (sequence, KV head) stream weighs ov + n units: ov for the cost of
    // starting a piece (a few dependent memory round trips), then one per
    // attended page (at least one page, so that an empty stream writes its
    // zero rows). sh_pref[0 .. B] holds the exclusive prefix sums of H_kv
    // streams per sequence and sh_len the lengths: thread t sums sequences
    // [t C, (t + 1) C), then a scan over the threads.
    __shared__ int32_t sh_pref[kBalancedMaxBatch + 1];
    __shared__ int32_t sh_len[kBalancedMaxBatch];
    __shared__ int32_t sh_wsum[kWaves];
    const int B = a.batch;
    const int H = a.num_kv_heads;
    const int ov = a.bal_overhead;
    auto pages_of = [&](int Lb) {
      const int t0b = (a.window > 0 && Lb > a.window) ? Lb - a.window : 0;
      const int n = Lb > 0 ? (Lb + P - 1) / P - t0b / P : 0;
      return n > 1 ? n : 1;
    };
    const int C = (B + kThreads - 1) / kThreads;
    int local = 0;
    for (int i = 0; i < C; ++i) {
      const int bb = tid * C + i;
      if (bb < B) {
        const int Lb = a.seq_lens[bb];
        sh_len[bb] = Lb;
        local += ov + pages_of(Lb);
      }
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) sh_wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w2 = 0; w2 < wave; ++w2) run += sh_wsum[w2];
    for (int i = 0; i < C; ++i) {
      const int bb = tid * C + i;
      if (bb < B) {
        sh_pref[bb] = run * H;
        run += ov + pages_of(sh_len[bb]);
      }
    }
    if (tid == kThreads - 1) sh_pref[B] = run * H;
    __syncthreads();

    // This work-group's units [u0, u1); the sequence holding u0 is the last
    // b with sh_pref[b] <= u0 (prefix sums strictly increase).
    const int q = a.pages_per_split;
    const int w = blockIdx.x;
    const int u0 = w * q;
    const int U = __builtin_amdgcn_readfirstlane(sh_pref[B]);
    const int u1 = u0 + q < U ? u0 + q : U;
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(sh_pref[mid]) <= u0)
        lo = mid;
      else
        hi = mid - 1;
    }
    int b = lo;
    for (int u = u0; u < u1;) {
      while (__builtin_amdgcn_readfirstlane(sh_pref[b + 1]) <= u) ++b;
      const int sb = __builtin_amdgcn_readfirstlane(sh_pref[b]);
      const int wt = (__builtin_amdgcn_readfirstlane(sh_pref[b + 1]) - sb) / H;  // ov + pages
      const int kvh = (u - sb) / wt;
      const int s0 = sb + kvh * wt;  // the stream's first unit
      const int ps = s0 + ov;        // its first page's unit
      const int s1 = s0 + wt;
      const int pa = u > ps ? u : ps;  // pages [pa - ps, pb - ps) of the stream are this piece
      const int pb = u1 < s1 ? u1 : s1;
      if (pa < pb) {
        const int first = ps / q;  // work-group holding the stream's first page
        const int pieces = (s1 - 1) / q - first + 1;
        if (w == first && tid == 0 && a.ws_cnt != nullptr) a.ws_cnt[b * H + kvh] = pieces;
        const int L = __builtin_amdgcn_readfirstlane(sh_len[b]);
        const int t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
        const int pf = L > 0 ? t0 / P : 0;
        const int plo = pf + (pa - ps);
        const int phi = pf + (pb - ps);
        const int t_lo = L > 0 ? (t0 > plo * P ? t0 : plo * P) : 0;
        const int t_hi = L > 0 ? (L < phi * P ? L : phi * P) : 0;
        uint4 qb[NJ];
        load_q(b, kvh, qb);
        process(b, kvh, qb, plo, phi, t_lo, t_hi, pieces == 1, w - first);
        __syncthreads();  // the next piece rewrites the LDS
      }
      u = s1;
    }
  } else {
    // KV head fastest: the H_kv work-groups of one page range are dispatched
    // together, so their K/V blocks (adjacent in a page) are read at the same
    // time.
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    const int L = a.seq_lens[b] - a.len_offset;
    const int t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
    const int pf = L > 0 ? t0 / P : 0;
    const int pe = L > 0 ? (L + P - 1) / P : 0;
    const int cp = a.pages_per_split;
    int nsplit = (pe - pf + cp - 1) / cp;
    nsplit = nsplit < 1 ? 1 : (nsplit > a.max_splits ? a.max_splits : nsplit);
    // Splits (chunks in the fixed-order mode) [k_begin, k_end) of this group.
    const int k_begin = MODE == kFixed ? s * a.chunks_per_group : s;
    if (k_begin >= nsplit) return;  // whole work-group, uniform
    const int k_end =
        MODE == kFixed ? (k_begin + a.chunks_per_group < nsplit ? k_begin + a.chunks_per_group : nsplit) : k_begin + 1;
    uint4 qb[NJ];
    load_q(b, kvh, qb);
    for (int k = k_begin; k < k_end; ++k) {
      // Attended tokens of this split (chunk): [t_lo, t_hi).
      const int plo = pf + k * cp;
      const int phi = (plo + cp < pe) ? plo + cp : pe;
      const int t_lo = L > 0 ? (t0 > plo * P ? t0 : plo * P) : 0;
      const int t_hi = L > 0 ? (L < phi * P ? L : phi * P) : 0;
      process(b, kvh, qb, plo, phi, t_lo, t_hi, MODE == kGrid && nsplit == 1, k);
      if constexpr (MODE == kFixed) __syncthreads();  // the next chunk rewrites the LDS
    }
  }
}

template <int D, int KVT, int GT>
void launch_mode(const KernelArgs& a, dim3 grid, hipStream_t st) {
  if (a.balanced)
    hipLaunchKernelGGL((split_kernel_mfma<D, KVT, GT, kBalanced>), dim3(a.split_groups), dim3(kThreads), 0, st, a);
  else if (a.chunks_per_group > 0)
    hipLaunchKernelGGL((split_kernel_mfma<D, KVT, GT, kFixed>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((split_kernel_mfma<D, KVT, GT, kGrid>), grid, dim3(kThreads), 0, st, a);
}

template <int D, int KVT>
hipError_t launch_gt(const KernelArgs& a, int gt, dim3 grid, hipStream_t st) {
  switch (gt) {
    case 1: launch_mode<D, KVT, 1>(a, grid, st); break;
    case 2: launch_mode<D, KVT, 2>(a, grid, st); break;
    case 4: launch_mode<D, KVT, 4>(a, grid, st); break;
    case 8: launch_mode<D, KVT, 8>(a, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_kv(const KernelArgs& a, int kv, int gt, dim3 grid, hipStream_t st) {
  switch (kv) {
    case DA_F16: return launch_gt<D, DA_F16>(a, gt, grid, st);
    case DA_BF16: return launch_gt<D, DA_BF16>(a, gt, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split_mfma(const KernelArgs& a, int head_dim, int kv_dtype, int group_tile, hipStream_t stream) {
  const dim3 grid(a.num_kv_heads, a.split_groups, a.batch);
  switch (head_dim) {
    case 128: return launch_kv<128>(a, kv_dtype, group_tile, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace da
