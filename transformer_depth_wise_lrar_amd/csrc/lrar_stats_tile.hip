// Phase 1 of the two-phase block schedule on whole workgroups (AttnRes technical-report
// summary, "Method": a block's static site queries are batched into one inter-block attention
// over the cached block representations; LR-AttnRes paper §3.4: the sliced key keeps this
// valid).
//
// For up to kStatsMaxSrc cached sources and a group of up to kStatsMaxQ site queries:
//   * one workgroup per CU (12 wavefronts; 16 for bf16 sources with bf16 accumulators, 8 with
//     float32 ones)
//     shares one LDS copy of the group's queries, laid out from the first key unit's column
//     (columns of that unit before the key hold zero), so each key element is dotted with
//     every query of the group from LDS;
//   * each wave takes one token row at a time, rows dealt out in bands over all waves;
//   * score pass: per source, the key units are taken kStatsKeySlots slots at a time; float64
//     partial sums of q_s . k for every query s and of k . k accumulate per lane, and the
//     (queries + 1) sums are reduced together by a transposed butterfly (each lane of a quad
//     ends with four of them); the scores z_si go to LDS. The next round's key units (the next
//     source's first round after a source's last) are loaded while the current round is
//     folded;
//   * statistics: per query, m = max_i z_si rounded to float32, e_si = exp(z_si - m),
//     l = sum_i e_si (float64 on the lanes), written once per row;
//   * value pass: the row is walked in chunks of 64 units, from the first chunk that holds key
//     units; each chunk of every source is loaded once, and the accumulators of all the
//     group's queries come from matrix-core products (weights x values, float32) whose outputs
//     are whole units of the accumulator rows, written straight out (acc = sum_i e_si o_i, not
//     normalised). The next chunk is loaded right after the current chunk's stores, so the
//     loads are in flight while the next products run.
// Every load is issued by every lane whatever the source count and the row's width: a source
// slot past n reads source 0 and a unit past the row (or before the key) reads the nearest unit
// inside it, and those values are discarded. With loads under conditions the compiler cannot
// count the loads in flight and waits for all of them, and for every earlier store, before it
// uses any one.
// Each cached source row is read from HBM once per query group (its key again, from L2 when
// the key chunks are still there: the value pass visits them first), and every accumulator
// element is written once.

#include "lrar_device.h"
#include "lrar_launch.h"
#include "lrar_tile.h"

namespace lrar {

namespace {

// Waves per workgroup (one workgroup per CU: the staged queries take most of the LDS), at
// d = 7168, r = 1792, 8 sources x 12 queries, 32768 rows, measured on the same buffers: bf16
// sources with bf16 accumulators fit 4 waves per SIMD (at most 128 registers) and run 16,
// 3-6 % faster than 12 and 5 % faster than 8; with float32 accumulators, whose writes are
// twice as wide, 8 waves run 2.4 % faster than 12 and 10 % faster than 4 (their plain stream
// is fastest with few waves too). float32 sources keep 12 (16 measured no faster).
constexpr int kStatsWavesMax = 16;
static_assert(kStatsMaxQ <= 16 && kStatsMaxSrc % 4 == 0,
              "a query group fills at most the 16 rows of a matrix product, sources come in fours");
// LDS a workgroup holds besides the staged queries (z_lds, w_lds)
constexpr size_t kStatsStaticLds =
    kStatsWavesMax * kStatsMaxQ * kStatsMaxSrc * (sizeof(double) + sizeof(float));

}  // namespace

// FULLQ: the group holds kStatsMaxQ queries, so no pass or store depends on the group's size
// (with a smaller group, those branches leave the compiler unsure how many stores are in flight
// and its waits for loads then also wait for stores).
template <typename IO, int VEC, typename ACC, bool FULLQ, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_stats_tile(StatsParams p, int q0, int nq_arg) {
  constexpr int kStatsWaves = WAVES;
  constexpr int kStatsBlock = WAVES * kWave;
  static_assert(WAVES <= kStatsWavesMax, "the query group's LDS budget counts kStatsWavesMax");
  extern __shared__ __attribute__((aligned(16))) float q_lds[];  // [nqg][rq]
  const int nqg = FULLQ ? kStatsMaxQ : nq_arg;
  // Scores of the wave's current row: z[s][i] for query s, source i; and their weights.
  __shared__ double z_lds[kStatsWaves][kStatsMaxQ][kStatsMaxSrc];
  __shared__ __attribute__((aligned(16))) float w_lds[kStatsWaves][kStatsMaxSrc][kStatsMaxQ];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = wave_in_block();
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kStatsWaves + wv;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kStatsWaves;
  const int n = p.n;
  const int nur = (p.d + VEC - 1) / VEC;
  const int nslot = (nur + kWave - 1) / kWave;  // unit slots per lane
  const int c0 = p.d - p.r;
  const double rinv_r = 1.0 / static_cast<double>(p.r);
  const int ub = c0 / VEC;
  const int rq = p.d - ub * VEC;  // staged query columns
  const int k_lo = ub / kWave;    // first slot that can hold key units
  // query s of the group staged at q_lds + s * rq, transposed (QStage)
  const int nv = nur - ub;
  for (int s = 0; s < nqg; ++s) {
    QStage qs{q_lds + s * rq, nv};
    qs.fill<VEC>(p.q + static_cast<int64_t>(q0 + s) * p.q_ld, ub, c0, threadIdx.x, kStatsBlock);
  }
  __syncthreads();

  // source slots past n stand in with source 0 (read, never used)
  const IO* sp[kStatsMaxSrc];
  int64_t sld[kStatsMaxSrc];
#pragma unroll
  for (int i = 0; i < kStatsMaxSrc; ++i) {
    sp[i] = static_cast<const IO*>(i < n ? p.src.ptr[i] : p.src.ptr[0]);
    sld[i] = i < n ? p.src.ld[i] : p.src.ld[0];
  }

  for (int64_t row = wave; row < p.T; row += nwaves) {
    // ---- score pass: z_si of every (query, source) pair into z_lds. Rounds of kStatsKeySlots
    // slots run source by source; the next round's key units are loaded before this round's
    // are folded.
    const auto key_row = [&](int i) {
      return static_cast<const IO*>(p.src.ptr[i]) + row * p.src.ld[i];
    };
    const auto load_keys = [&](const IO* rp, int kb, Unit<IO, VEC>(&dst)[kStatsKeySlots]) {
#pragma unroll
      for (int t = 0; t < kStatsKeySlots; ++t) {
        int u = lane + kWave * (kb + t);
        u = u < ub ? ub : (u < nur ? u : nur - 1);
        dst[t].load_cached(rp + u * VEC);
      }
    };
    Unit<IO, VEC> kn[kStatsKeySlots];
    load_keys(key_row(0), k_lo, kn);
    double red[kStatsMaxQ + 1];
#pragma unroll
    for (int s = 0; s <= kStatsMaxQ; ++s) red[s] = 0.0;
    for (int i = 0, kb = k_lo; i < n;) {
      // this round's key values leave the load registers before the next round's loads
      // reuse them, so no register copy has to wait for those loads
      float x[kStatsKeySlots][VEC];
#pragma unroll
      for (int t = 0; t < kStatsKeySlots; ++t) {
        kn[t].get(x[t]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(x[t][e]));
      }
      const bool last = kb + kStatsKeySlots >= nslot;  // this round ends source i
      const int i_next = last ? (i + 1 < n ? i + 1 : i) : i;
      const int kb_next = last ? k_lo : kb + kStatsKeySlots;
      load_keys(key_row(i_next), kb_next, kn);
#pragma unroll
      for (int t = 0; t < kStatsKeySlots; ++t) {
        const int u = lane + kWave * (kb + t);
        if (kb + t < nslot && u >= ub && u < nur) {
          double kv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            kv[e] = (u * VEC + e) >= c0 ? static_cast<double>(x[t][e]) : 0.0;
            red[kStatsMaxQ] = fma(kv[e], kv[e], red[kStatsMaxQ]);
          }
          // One query at a time: the scheduling barrier keeps the query values of later
          // queries from being read ahead into registers.
#pragma unroll
          for (int s = 0; s < kStatsMaxQ; ++s) {
            if (s < nqg) {
              const QStage qs{q_lds + s * rq, nv};
              float qv[VEC];
              qs.get<VEC>(u - ub, qv);
#pragma unroll
              for (int e = 0; e < VEC; ++e)
                red[s] = fma(static_cast<double>(qv[e]), kv[e], red[s]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if (last) {
        // the query sums and k . k (value kStatsMaxQ) of the 16 reduced together: lane l < 4
        // holds values 4 l' .. 4 l' + 3 with l' = 2 (l & 1) + ((l >> 1) & 1), so k . k (value
        // 12) sits in lane 3, slot 0
        static_assert(kStatsMaxQ == 12, "k . k is value 12 of the transposed sums");
        double v16[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) v16[s] = s <= kStatsMaxQ ? red[s] : 0.0;
        double u[4];
        wave_sums_transposed16(v16, lane, u);
        const double rinv = score_from_sums(0.0, lane_f64(u[0], 3), rinv_r, p.eps).rinv;
        const int s0 = 8 * (lane & 1) + 4 * ((lane >> 1) & 1);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (lane < 4 && s0 + k < nqg) z_lds[wv][s0 + k][i] = u[k] * rinv;
#pragma unroll
        for (int s = 0; s <= kStatsMaxQ; ++s) red[s] = 0.0;
        ++i;
      }
      kb = kb_next;
    }

    // ---- statistics per query (lanes = sources)
    float ew[kStatsMaxQ];
#pragma unroll
    for (int s = 0; s < kStatsMaxQ; ++s) {
      ew[s] = 0.f;
      if (s < nqg) {
        const double z = lane < n ? z_lds[wv][s][lane] : -INFINITY;
        const double m = wave_max_dpp(z);
        const float mf = static_cast<float>(m);
        const double e = lane < n ? exp(z - static_cast<double>(mf)) : 0.0;
        const double L = wave_sum_dpp(e);
        ew[s] = static_cast<float>(e);
        if (lane == 0) {
          int64_t off = static_cast<int64_t>(q0 + s) * p.ml_ld + row;
          asm volatile("" : "+v"(off));  // computed here, not hoisted out of the row loop
          p.m[off] = mf;
          p.l[off] = static_cast<float>(L);
        }
      }
    }

    // ---- value pass on the matrix cores. Per row the accumulators are a small dense product,
    // acc[s][c] = sum_i w_si o_i[c] (queries x sources times sources x columns), which
    // v_mfma_f32_16x16x4f32 takes as A = w (16 queries x 4 sources), B = o (4 sources x 16
    // columns) and D = acc (16 x 16), all float32. Lane l supplies A[l % 16][l / 16] and
    // B[l / 16][l % 16] and receives D[4 (l / 16) + j][l % 16], j = 0..3. A lane that loads
    // the unit of source 4 kb + l / 16 at unit 16 b + l % 16 of a chunk, and feeds its element e
    // to the e-th product of block b, so holds after the VEC products the VEC columns of that
    // unit for four queries: one whole unit of each, stored as such.
    // Sources past n weigh zero (and read source 0).
#pragma unroll
    for (int s = 0; s < kStatsMaxQ; ++s)
      if (s < nqg && lane < n) w_lds[wv][lane][s] = ew[s];
    __builtin_amdgcn_wave_barrier();
    constexpr int kKb = kStatsMaxSrc / 4;  // blocks of four sources
    constexpr int kBlocks = kWave / 16;    // blocks of 16 units in a chunk of 64
    const int ql = lane & 15;              // A row (query), B and D column
    const int kq = lane >> 4;              // A column and B row (source in the block), D row / 4
    const int qa = ql < nqg ? ql : nqg - 1;  // rows past the group repeat the last query
    float aw[kKb];
    const IO* vrow[kKb];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      const int src = 4 * kb + kq;
      aw[kb] = src < n ? w_lds[wv][src][qa] : 0.f;
      const IO* b0 = sp[4 * kb] + row * sld[4 * kb];
      const IO* b1 = sp[4 * kb + 1] + row * sld[4 * kb + 1];
      const IO* b2 = sp[4 * kb + 2] + row * sld[4 * kb + 2];
      const IO* b3 = sp[4 * kb + 3] + row * sld[4 * kb + 3];
      vrow[kb] = kq == 0 ? b0 : (kq == 1 ? b1 : (kq == 2 ? b2 : b3));
    }
    const bool two_blocks = n > 4;
    // bf16 sources with float32 accumulators: a lane takes two runs of 4 columns of a block of
    // 128 (4 l and 64 + 4 l) instead of one unit of 8, so that each 16-byte store of the
    // accumulators lands next to its neighbour lanes' (256 contiguous bytes per 16 lanes).
    constexpr bool kSplit = std::is_same<IO, bf16_bits>::value && std::is_same<ACC, float>::value;
    constexpr int kBlockCols = 16 * VEC;
    Unit<IO, VEC> buf[kBlocks][kKb];
    const auto load_chunk = [&](int c) {
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        if constexpr (kSplit) {
          int col0 = (kBlocks * c + b) * kBlockCols + 4 * ql;
          int col1 = col0 + kBlockCols / 2;
          col0 = col0 < p.d ? col0 : p.d - 4;
          col1 = col1 < p.d ? col1 : p.d - 4;
#pragma unroll
          for (int kb = 0; kb < kKb; ++kb) {
            const u32x2 lo =
                __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vrow[kb] + col0));
            const u32x2 hi =
                __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vrow[kb] + col1));
            buf[b][kb].raw = u32x4{lo.x, lo.y, hi.x, hi.y};
            // issued in order, so a wait for one unit is a wait for it and the loads before it
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          int u = kWave * c + 16 * b + ql;
          u = u < nur ? u : nur - 1;
#pragma unroll
          for (int kb = 0; kb < kKb; ++kb) {
            buf[b][kb].load(vrow[kb] + u * VEC);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    ACC* const acc_row = static_cast<ACC*>(p.acc) + row * p.acc_ld;
    // The chunks are walked from the first one that holds key units (k_lo) to the row's end,
    // then from 0: the key units, just read by the score pass through the cache, are read again
    // while still there. Each chunk's sums depend on that chunk alone, so the order changes no
    // result.
    load_chunk(k_lo);
    for (int k = 0; k < nslot; ++k) {
      const int c = k_lo + k < nslot ? k_lo + k : k_lo + k - nslot;
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        f32x4 dacc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) dacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb) {
          if (kb == 0 || two_blocks) {
            float x[VEC];
            buf[b][kb].get(x);
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              dacc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[kb], x[e], dacc[e], 0, 0, 0);
          }
        }
        // Lanes whose query row lies past the group store nothing. These stores come before the
        // next chunk's loads, so skipping some of them leaves the waits for those loads exact.
        // A lane past the row's end loaded the row's last columns and stores their sums there
        // again: the same bytes as the owning lane.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = 4 * kq + j;
          float v[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = dacc[e][j];
          if (s < nqg) {
            if constexpr (kSplit) {
              int col0 = (kBlocks * c + b) * kBlockCols + 4 * ql;
              int col1 = col0 + kBlockCols / 2;
              col0 = col0 < p.d ? col0 : p.d - 4;
              col1 = col1 < p.d ? col1 : p.d - 4;
              float* dq = reinterpret_cast<float*>(acc_row) +
                          static_cast<int64_t>(q0 + s) * p.acc_qstride;
              out_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(dq + col0));
              out_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(dq + col1));
            } else {
              int u = kWave * c + 16 * b + ql;
              u = u < nur ? u : nur - 1;
              const int64_t off = static_cast<int64_t>(q0 + s) * p.acc_qstride + u * VEC;
              store_acc<ACC, VEC>(acc_row + off, v);
            }
          }
        }
      }
      // the next chunk, after this chunk's stores (the last chunk reloads itself)
      load_chunk(k + 1 < nslot ? (c + 1 < nslot ? c + 1 : 0) : c);
    }
    // the next row's weights overwrite w_lds only after every lane has read this row's
    __builtin_amdgcn_wave_barrier();
  }
}

namespace {

int device_cus_stats() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      cus = 256;
  }
  return cus;
}

// Largest LDS allocation one workgroup may use on this device.
size_t lds_limit() {
  static size_t lim = 0;
  if (lim == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
      lim = static_cast<size_t>(v);
    else
      lim = 64 * 1024;
  }
  return lim;
}

template <typename IO, int VEC, typename ACC, int WAVES>
hipError_t launch_stats_tile_t(const StatsParams& p, int qg, hipStream_t s) {
  constexpr int kStatsWaves = WAVES;
  constexpr int kStatsBlock = WAVES * kWave;
  const int ub = (p.d - p.r) / VEC;
  const int rq = p.d - ub * VEC;
  for (int q0 = 0; q0 < p.nq; q0 += qg) {
    const int nqg = (p.nq - q0) < qg ? (p.nq - q0) : qg;
    auto kern = nqg == kStatsMaxQ ? k_stats_tile<IO, VEC, ACC, true, WAVES>
                                  : k_stats_tile<IO, VEC, ACC, false, WAVES>;
    const size_t lds = static_cast<size_t>(nqg) * rq * sizeof(float);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kStatsBlock, lds) !=
            hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    const int64_t need = (p.T + kStatsWaves - 1) / kStatsWaves;
    int64_t blocks = static_cast<int64_t>(per_cu) * device_cus_stats();
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kStatsBlock), lds, s, p,
                       q0, nqg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int stats_tile_query_group(int d, int r, int vec) {
  const int ub = (d - r) / vec;
  const size_t per_q = static_cast<size_t>(d - ub * vec) * sizeof(float);
  const size_t lim = lds_limit();
  size_t fit = lim > kStatsStaticLds ? (lim - kStatsStaticLds) / per_q : 0;
  if (fit > static_cast<size_t>(kStatsMaxQ)) fit = kStatsMaxQ;
  return static_cast<int>(fit);
}

hipError_t launch_stats_tile(const StatsParams& p, int io_bf16, int acc_bf16, int qg,
                             hipStream_t s) {
  if (io_bf16) return acc_bf16 ? launch_stats_tile_t<bf16_bits, 8, bf16_bits, 16>(p, qg, s)
                               : launch_stats_tile_t<bf16_bits, 8, float, 8>(p, qg, s);
  return acc_bf16 ? launch_stats_tile_t<float, 4, bf16_bits, 12>(p, qg, s)
                  : launch_stats_tile_t<float, 4, float, 12>(p, qg, s);
}

}  // namespace lrar
