// Phase 1 of the two-phase block schedule (AttnRes technical-report summary, "Method":
// a block's static queries are batched into one inter-block attention over the cached block
// representations; LR-AttnRes paper §3.4: the sliced key keeps this valid).
//
// k_stats serves the shapes the workgroup kernel of lrar_stats_tile.hip does not (the
// scalar-element path, more than kStatsMaxSrc sources). One wavefront per token row. For a
// group of up to QB queries the kernel
//   1. reduces, per source, the key's sum of squares once and its dot product with every
//      query of the group (float64), so each key element is loaded once per group;
//   2. forms per query m = max z (rounded to float32), e_i = exp(z_i - m), l = sum e_i;
//   3. streams every source row once and accumulates all QB unnormalised partial sums
//      acc_s = sum_i e_si o_i in float32, written as float32 or bf16.
// Reading each cached source once for the whole group, instead of once per site, is the
// point of Phase 1.

#include "lrar_device.h"
#include "lrar_launch.h"

namespace lrar {

template <typename IO, int VEC, int QB, typename ACC>
__global__ __launch_bounds__(kBlock) void k_stats(StatsParams p) {
  constexpr int B = 4;  // sources loaded together in the value stream
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const KeyGeom g = key_geom<VEC>(p.d, p.r);
  const int slot = lane / g.group;
  const int sub = lane % g.group;
  const int iters = (p.n + g.per_it - 1) / g.per_it;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; row < p.T;
       row += step) {
    for (int q0 = 0; q0 < p.nq; q0 += QB) {
      const int nqg = (p.nq - q0) < QB ? (p.nq - q0) : QB;
      const float* qg = p.q + static_cast<int64_t>(q0) * p.q_ld;
      // 1. scores of every (query, source) pair; lane i keeps z_si of source i
      double zq[QB];
#pragma unroll
      for (int s = 0; s < QB; ++s) zq[s] = 0.0;
      for (int it = 0; it < iters; ++it) {
        const int i = it * g.per_it + slot;
        const IO* base = nullptr;
        int64_t ld = 0;
        for (int c = 0; c < g.per_it; ++c) {
          const int ic = it * g.per_it + c;
          if (ic < p.n && c == slot) {
            base = static_cast<const IO*>(p.src.ptr[ic]);
            ld = p.src.ld[ic];
          }
        }
        double dot[QB];
#pragma unroll
        for (int s = 0; s < QB; ++s) dot[s] = 0.0;
        double ss = 0.0;
        if (i < p.n) {
          const IO* rowp = base + row * ld;
          for (int u = g.ub + sub; u < g.nur; u += g.group) {
            Unit<IO, VEC> un;
            un.load_cached(rowp + u * VEC);
            float x[VEC];
            un.get(x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const int col = u * VEC + e;
              if (col >= g.c0) {
                const double k = static_cast<double>(x[e]);
                ss = fma(k, k, ss);
                const float* qc = qg + (col - g.c0);
#pragma unroll
                for (int s = 0; s < QB; ++s)
                  if (s < nqg) dot[s] = fma(static_cast<double>(qc[s * p.q_ld]), k, dot[s]);
              }
            }
          }
        }
        ss = group_sum(ss, g.group);
        const double rho = sqrt(ss / p.r + p.eps);
        const int src_lane = (lane % g.per_it) * g.group;
        const bool mine = (lane / g.per_it) == it;
#pragma unroll
        for (int s = 0; s < QB; ++s) {
          if (s < nqg) {
            const double z = group_sum(dot[s], g.group) / rho;
            const double zt = __shfl(z, src_lane, kWave);
            if (mine) zq[s] = zt;
          }
        }
      }
      // 2. per-query statistics
      float E[QB];
#pragma unroll
      for (int s = 0; s < QB; ++s) {
        E[s] = 0.f;
        if (s < nqg) {
          const double m = wave_max((lane < p.n) ? zq[s] : -INFINITY);
          const float mf = static_cast<float>(m);
          const double e = (lane < p.n) ? exp(zq[s] - static_cast<double>(mf)) : 0.0;
          const double L = wave_sum(e);
          E[s] = static_cast<float>(e);
          if (lane == 0) {
            p.m[static_cast<int64_t>(q0 + s) * p.ml_ld + row] = mf;
            p.l[static_cast<int64_t>(q0 + s) * p.ml_ld + row] = static_cast<float>(L);
          }
        }
      }
      // 3. unnormalised partial sums, one pass over every source per column chunk
      for (int cb = 0; cb < g.nur; cb += kWave) {
        const int u = cb + lane;
        float acc[QB][VEC];
#pragma unroll
        for (int s = 0; s < QB; ++s)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[s][e] = 0.f;
        int i = 0;
        for (; i + B <= p.n; i += B) {
          Unit<IO, VEC> un[B];
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const IO* srow = static_cast<const IO*>(p.src.ptr[i + b]) + row * p.src.ld[i + b];
            if (u < g.nur) un[b].load(srow + u * VEC); else un[b].zero();
          }
#pragma unroll
          for (int b = 0; b < B; ++b) {
            float x[VEC];
            un[b].get(x);
#pragma unroll
            for (int s = 0; s < QB; ++s) {
              if (s < nqg) {
                const float a = lane_f32(E[s], i + b);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[s][e] = fmaf(a, x[e], acc[s][e]);
              }
            }
          }
        }
        for (; i < p.n; ++i) {
          const IO* srow = static_cast<const IO*>(p.src.ptr[i]) + row * p.src.ld[i];
          Unit<IO, VEC> un;
          if (u < g.nur) un.load(srow + u * VEC); else un.zero();
          float x[VEC];
          un.get(x);
#pragma unroll
          for (int s = 0; s < QB; ++s) {
            if (s < nqg) {
              const float a = lane_f32(E[s], i);
#pragma unroll
              for (int e = 0; e < VEC; ++e) acc[s][e] = fmaf(a, x[e], acc[s][e]);
            }
          }
        }
        if (u < g.nur) {
#pragma unroll
          for (int s = 0; s < QB; ++s) {
            if (s < nqg) {
              ACC* dst = static_cast<ACC*>(p.acc) + static_cast<int64_t>(q0 + s) * p.acc_qstride +
                         row * p.acc_ld + u * VEC;
              store_acc<ACC, VEC>(dst, acc[s]);
            }
          }
        }
      }
    }
  }
}

namespace {

int grid_for_rows(int64_t T) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = 65536;
  return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

template <typename IO, int VEC, typename ACC>
hipError_t launch_stats_t(const StatsParams& p, hipStream_t s) {
  const dim3 grid(grid_for_rows(p.T)), block(kBlock);
  if (p.nq <= 1)
    hipLaunchKernelGGL((k_stats<IO, VEC, 1, ACC>), grid, block, 0, s, p);
  else if (p.nq <= 2)
    hipLaunchKernelGGL((k_stats<IO, VEC, 2, ACC>), grid, block, 0, s, p);
  else if (p.nq <= 4)
    hipLaunchKernelGGL((k_stats<IO, VEC, 4, ACC>), grid, block, 0, s, p);
  else if (p.nq <= 8)
    hipLaunchKernelGGL((k_stats<IO, VEC, 8, ACC>), grid, block, 0, s, p);
  else if (p.nq <= 12)
    hipLaunchKernelGGL((k_stats<IO, VEC, 12, ACC>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((k_stats<IO, VEC, 16, ACC>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stats(const StatsParams& p, int io_bf16, int vec, int acc_bf16, hipStream_t s) {
  if (vec > 1 && p.n <= kStatsMaxSrc) {
    const int qg = stats_tile_query_group(p.d, p.r, vec);
    if (qg >= 1) return launch_stats_tile(p, io_bf16, acc_bf16, qg, s);
  }
  if (io_bf16) {
    if (acc_bf16) return vec > 1 ? launch_stats_t<bf16_bits, 8, bf16_bits>(p, s)
                                 : launch_stats_t<bf16_bits, 1, bf16_bits>(p, s);
    return vec > 1 ? launch_stats_t<bf16_bits, 8, float>(p, s)
                   : launch_stats_t<bf16_bits, 1, float>(p, s);
  }
  if (acc_bf16) return vec > 1 ? launch_stats_t<float, 4, bf16_bits>(p, s)
                               : launch_stats_t<float, 1, bf16_bits>(p, s);
  return vec > 1 ? launch_stats_t<float, 4, float>(p, s) : launch_stats_t<float, 1, float>(p, s);
}

}  // namespace lrar
