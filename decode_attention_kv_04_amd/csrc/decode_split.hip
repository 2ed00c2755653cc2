// Split pass of paged decode attention for gfx950.
//
// One work-group of four wave64s owns one (KV head j, split s, sequence b):
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
// product (v_dot2 on packed 16-bit pairs when q and K share a 16-bit type,
// fp32 FMAs otherwise) finished by a sum over the LPR lanes of the row with
// DPP (no LDS, no barrier), which leaves the full score in every lane of the
// row (llm-web pull 8, decode-attention commit: one key's dot product shared
// by adjacent lanes, reduced without barrier trees). Each lane then owns the
// rows of its row slot as a private online-softmax shard: its m, l and O
// slice live in VGPRs, and the slots are merged once, at the end, across the
// wave with lane shuffles and across the four waves through LDS. No barrier
// is executed inside the key loop.
//
// Streaming. Each wave walks its tiles (TR rows) with PD tiles of K and V
// loads in flight in registers while it computes the oldest one. The page of
// every load group is tracked with a cursor advanced by additions (no integer
// division in the loop), and its physical page id is fetched with a scalar
// load one tile before the vector loads that need it. Only pages holding
// attended keys are read.
//
// Masking uses selects, never multiplication by zero, because rows outside
// the attended range may hold NaN: a score outside [t_lo, t_hi) becomes -inf
// and its value row is replaced by zeros before it is accumulated.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_attn.h"
#include "device_common.h"
#include "kernels.h"

#ifndef DA_PREFETCH_TILES
#define DA_PREFETCH_TILES 2
#endif

namespace da {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kPD = DA_PREFETCH_TILES;  // tiles in flight per wave while one is computed

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

// QPACK: q and K/V share a 16-bit dtype; q is kept as packed pairs and q.k
// uses v_dot2 with fp32 accumulation. Otherwise q is fp32 and q.k uses FMAs.
// FIXED: fixed-order mode. The work-group computes chunks_per_group
// consecutive chunks of pages_per_split pages each, one after the other, and
// writes each chunk's state to its own slot; the combine pass merges them in
// chunk order. A chunk's state depends only on its keys (its tiles are dealt
// to the waves from the chunk's first tile, and the waves are merged in a
// fixed order), never on which work-group computed it.
template <int D, int KVT, int GT, bool QPACK, bool FIXED>
__global__ __launch_bounds__(kThreads) void split_kernel(const KernelArgs a) {
  using LY = Layout<D, KVT, GT>;
  constexpr int LPR = LY::LPR, DPL = LY::DPL, VPL = LY::VPL, RPI = LY::RPI, NS = LY::NS, TR = LY::TR,
                E = LY::E, SEG = LY::SEG, ELT = LY::ELT;
  static_assert(!QPACK || KVT != DA_F32, "packed q needs a 16-bit KV type");

  // KV head fastest: the H_kv work-groups of one page range are dispatched
  // together, so their K/V blocks (adjacent in a page) are read at the same
  // time.
  const int kvh = blockIdx.x;
  const int s = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane % LPR;  // lane within the row
  const int r = lane / LPR;  // row slot within a load instruction

  // Attended tokens of this split: [t_lo, t_hi). Token counts fit int32 (the
  // planner bounds max_pages_per_seq * page_size).
  const int P = a.page_size;
  const int L = a.seq_lens[b] - a.len_offset;
  const int t0 = (a.window > 0 && L > a.window) ? L - a.window : 0;
  const int pf = L > 0 ? t0 / P : 0;
  const int pe = L > 0 ? (L + P - 1) / P : 0;
  const int cp = a.pages_per_split;
  int nsplit = (pe - pf + cp - 1) / cp;
  nsplit = nsplit < 1 ? 1 : (nsplit > a.max_splits ? a.max_splits : nsplit);
  // Splits (chunks in the fixed-order mode) [k_begin, k_end) of this group.
  const int k_begin = FIXED ? s * a.chunks_per_group : s;
  if (k_begin >= nsplit) return;  // whole work-group, uniform
  const int k_end = FIXED ? (k_begin + a.chunks_per_group < nsplit ? k_begin + a.chunks_per_group : nsplit)
                          : k_begin + 1;

  const int G = a.group;
  const int h0 = kvh * G;
  const int64_t qrow0 = static_cast<int64_t>(b) * a.rows_per_seq + a.row_base + h0;

  // q for the G heads of the group, this lane's elements.
  using QReg = typename std::conditional<QPACK, uint32_t, float>::type;
  constexpr int QW = QPACK ? DPL / 2 : DPL;
  QReg qv[GT][QW];
  if constexpr (QPACK) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (g < G)
          u = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                              ((qrow0 + g) * D + v * SEG + c * E) * ELT);
        qv[g][v * 4] = u.x;
        qv[g][v * 4 + 1] = u.y;
        qv[g][v * 4 + 2] = u.z;
        qv[g][v * 4 + 3] = u.w;
      }
    }
  } else {
    auto load_q = [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
      constexpr int QE = QT == DA_F32 ? 4 : 2;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          if (g < G) {
            load_row_f32<QT, E>(static_cast<const char*>(a.q) + ((qrow0 + g) * D + v * SEG + c * E) * QE,
                                &qv[g][v * E]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) qv[g][v * E + e] = 0.0f;
          }
        }
      }
    };
    if (a.q_dtype == DA_F32)
      load_q(std::integral_constant<int, DA_F32>());
    else if (a.q_dtype == DA_F16)
      load_q(std::integral_constant<int, DA_F16>());
    else
      load_q(std::integral_constant<int, DA_BF16>());
  }

  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const int64_t block_bytes = static_cast<int64_t>(P) * D * ELT;  // one (page, head) block
  const int64_t page_bytes = block_bytes * a.num_kv_heads;
  const int64_t head_bytes = block_bytes * kvh;
  const int32_t* table_row = a.page_table + static_cast<int64_t>(b) * a.max_pages;
  const uint32_t lane_off = static_cast<uint32_t>((r * D + c * E) * ELT);
  const float sl2 = a.scale_log2;

  __shared__ float sh_o[kWaves][GT][D];
  __shared__ float sh_m[kWaves][GT];
  __shared__ float sh_l[kWaves][GT];

  for (int k = k_begin; k < k_end; ++k) {
    // Attended tokens of this split (chunk): [t_lo, t_hi).
    const int plo = pf + k * cp;
    const int phi = (plo + cp < pe) ? plo + cp : pe;
    const int t_lo = L > 0 ? (t0 > plo * P ? t0 : plo * P) : 0;
    const int t_hi = L > 0 ? (L < phi * P ? L : phi * P) : 0;

    float m[GT], l[GT], o[GT][DPL];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.0f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[g][i] = 0.0f;
    }

    const int tile_first = t_lo / TR;
    const int tile_end = (t_hi + TR - 1) / TR;
    const int my_first = tile_first + wave;
    const int ntiles = my_first < tile_end ? (tile_end - my_first + kWaves - 1) / kWaves : 0;

    struct Tile {
      uint4 k[NS][VPL];
      uint4 v[NS][VPL];
    };

    // Load cursor: the next tile to load, the page index and in-page row of
    // each of its NS load groups, and their physical page ids (fetched one
    // step ahead).
    constexpr int STEP = kWaves * TR;
    const int step_p = STEP / P;
    const int step_r = STEP - step_p * P;
    int cur_tile = my_first;
    int cur_pi[NS], cur_off[NS], cur_phys[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int gs = my_first * TR + ns * RPI;
      cur_pi[ns] = gs / P;
      cur_off[ns] = gs - cur_pi[ns] * P;
    }
    // Page ids are read for every group, live or not, from an index clamped to
    // this split's own pages [plo, phi): always a mapped page, and the reads
    // need no branch (a branch would make the compiler wait on each one).
    // Rows of groups outside [t_lo, t_hi) are masked in compute().
    const int pi_last = phi > plo ? phi - 1 : plo;
    auto fetch_ids = [&]() {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int pi = cur_pi[ns] < plo ? plo : (cur_pi[ns] > pi_last ? pi_last : cur_pi[ns]);
        cur_phys[ns] = table_row[pi];
      }
    };
    auto advance = [&]() {
      cur_tile += kWaves;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        cur_pi[ns] += step_p;
        cur_off[ns] += step_r;
        if (cur_off[ns] >= P) {
          cur_off[ns] -= P;
          cur_pi[ns] += 1;
        }
      }
    };
    // Issue the loads of the cursor tile, then move the cursor and fetch the
    // next tile's page ids. A group outside [t_lo, t_hi) (only in the first and
    // last tile of a split) reads rows of a page of this split that compute()
    // masks out; the row offset is always inside its page.
    auto issue = [&](Tile& t) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int64_t off = static_cast<int64_t>(cur_phys[ns]) * page_bytes + head_bytes +
                            static_cast<int64_t>(cur_off[ns]) * (D * ELT);
        const char* kp = kbase + off + lane_off;
        const char* vp = vbase + off + lane_off;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          t.k[ns][v] = load16(kp + v * SEG * ELT);
          t.v[ns][v] = load16(vp + v * SEG * ELT);
        }
      }
      advance();
      fetch_ids();
    };

    auto compute = [&](const Tile& t, int tile) {
      const int tb = tile * TR;
      const bool full = tb >= t_lo && tb + TR <= t_hi;
      bool valid[NS];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int tok = tb + ns * RPI + r;
        valid[ns] = full || (tok >= t_lo && tok < t_hi);
      }
      // q.k partial sums, then the row sums.
      float sc[NS][GT];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        if constexpr (QPACK) {
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
              const uint4 u = t.k[ns][v];
              acc = dot2<KVT>(qv[g][v * 4], u.x, acc);
              acc = dot2<KVT>(qv[g][v * 4 + 1], u.y, acc);
              acc = dot2<KVT>(qv[g][v * 4 + 2], u.z, acc);
              acc = dot2<KVT>(qv[g][v * 4 + 3], u.w, acc);
            }
            sc[ns][g] = acc;
          }
        } else {
          float kf[DPL];
#pragma unroll
          for (int v = 0; v < VPL; ++v) unpack<KVT>(t.k[ns][v], kf + v * E);
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc = fmaf(qv[g][i], kf[i], acc);
            sc[ns][g] = acc;
          }
        }
      }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float x = row_sum<LPR>(sc[ns][g]) * sl2;
          sc[ns][g] = valid[ns] ? x : -INFINITY;
        }
      }
      // Online softmax. O and l are rescaled only when some running max of the
      // wave grew (a wave-uniform branch; a factor of exactly 1 is skipped).
      float mn[GT];
      bool grew = false;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float mt = sc[0][g];
#pragma unroll
        for (int ns = 1; ns < NS; ++ns) mt = fmaxf(mt, sc[ns][g]);
        mn[g] = mt > m[g] + DA_RESCALE_SLACK ? mt : m[g];  // moves only past the rescale slack
        grew |= mn[g] > m[g];
      }
      if (__any(grew)) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float mu = (mn[g] == -INFINITY) ? 0.0f : mn[g];
          const float alpha = exp2_fast(m[g] - mu);
          l[g] *= alpha;
#pragma unroll
          for (int i = 0; i < DPL; ++i) o[g][i] *= alpha;
          m[g] = mn[g];
        }
      }
      float p[NS][GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float mu = (m[g] == -INFINITY) ? 0.0f : m[g];
        float ps = 0.0f;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          p[ns][g] = exp2_fast(sc[ns][g] - mu);
          ps += p[ns][g];
        }
        l[g] += ps;
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

    // Ring of kPD + 1 tile buffers: tile n lives in buf[n % (kPD + 1)]. The
    // steady-state loop only runs while every tile it issues exists, so its
    // loads are unconditional and the compiler's wait counts stay exact (each
    // compute waits only for its own tile, kPD tiles of loads stay in flight);
    // the last tiles drain in an unrolled tail.
    if (ntiles > 0) {
      Tile buf[kPD + 1];
      fetch_ids();
#pragma unroll
      for (int k = 0; k < kPD; ++k)
        if (k < ntiles) issue(buf[k]);
      int n = 0;
      while (n + 2 * kPD < ntiles) {
#pragma unroll
        for (int j = 0; j <= kPD; ++j) {
          issue(buf[(j + kPD) % (kPD + 1)]);
          compute(buf[j], my_first + (n + j) * kWaves);
        }
        n += kPD + 1;
      }
      // Here ntiles - n <= 2 * kPD and n % (kPD + 1) == 0.
#pragma unroll
      for (int j = 0; j < 2 * kPD; ++j) {
        if (n + j < ntiles) {
          if (n + j + kPD < ntiles) issue(buf[(j + kPD) % (kPD + 1)]);
          compute(buf[j % (kPD + 1)], my_first + (n + j) * kWaves);
        }
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
      const int64_t row = qrow0 + g;
      if (!FIXED && nsplit == 1) {
        store_elem(a.out, row * D + d, a.out_dtype, lsum > 0.0f ? osum / lsum : 0.0f);
      } else {
        const int64_t srow = row * a.max_splits + k;
        a.ws_o[srow * D + d] = osum;
        if (d == 0) {
          a.ws_ml[srow * 2] = M;
          a.ws_ml[srow * 2 + 1] = lsum;
        }
      }
    }
    if constexpr (FIXED) __syncthreads();  // the next chunk rewrites the LDS
  }  // chunks
}

template <int D, int KVT, int GT, bool QPACK>
void launch_mode(const KernelArgs& a, dim3 grid, hipStream_t st) {
  if (a.chunks_per_group > 0)
    hipLaunchKernelGGL((split_kernel<D, KVT, GT, QPACK, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((split_kernel<D, KVT, GT, QPACK, false>), grid, dim3(kThreads), 0, st, a);
}

template <int D, int KVT, bool QPACK>
hipError_t launch_gt(const KernelArgs& a, int gt, dim3 grid, hipStream_t st) {
  switch (gt) {
    case 1: launch_mode<D, KVT, 1, QPACK>(a, grid, st); break;
    case 2: launch_mode<D, KVT, 2, QPACK>(a, grid, st); break;
    case 4: launch_mode<D, KVT, 4, QPACK>(a, grid, st); break;
    case 8: launch_mode<D, KVT, 8, QPACK>(a, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_kv(const KernelArgs& a, int kv, int gt, dim3 grid, hipStream_t st) {
  const bool qpack = a.q_dtype == kv;
  switch (kv) {
    case DA_F32: return launch_gt<D, DA_F32, false>(a, gt, grid, st);
    case DA_F16:
      return qpack ? launch_gt<D, DA_F16, true>(a, gt, grid, st) : launch_gt<D, DA_F16, false>(a, gt, grid, st);
    case DA_BF16:
      return qpack ? launch_gt<D, DA_BF16, true>(a, gt, grid, st) : launch_gt<D, DA_BF16, false>(a, gt, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split(const KernelArgs& a, int head_dim, int kv_dtype, int group_tile, hipStream_t stream) {
  const dim3 grid(a.num_kv_heads, a.split_groups, a.batch);
  switch (head_dim) {
    case 64: return launch_kv<64>(a, kv_dtype, group_tile, grid, stream);
    case 128: return launch_kv<128>(a, kv_dtype, group_tile, grid, stream);
    case 256: return launch_kv<256>(a, kv_dtype, group_tile, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace da
