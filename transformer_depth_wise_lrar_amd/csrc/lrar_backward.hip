// Backward of the depth-mix read, scalar-element path and the dq reduction (LR-AttnRes paper
// App. B.3: Lemma 2 gives
// dL/do_i = alpha_i g + alpha_i <g, o_i - h> grad z_i; Corollary 2.1 gives the slice-RMS
// gradient grad z_i = P_r^T (q - z_i kbar_i / r) / rho_i; the query gradient follows from
// z_i = q . kbar_i). Each source slot is an independent input, as in the paper.
//
// k_backward, one wavefront per token row:
//   1. key pass (float64): z_i, rho_i, alpha_i of every source, as in the forward;
//   2. the row of g = dL/dh is loaded once into registers (float32);
//   3. s_i = <g, o_i> over all d (float64 sums of exact products); then
//      dz_i = alpha_i (s_i - sum_j alpha_j s_j), which equals alpha_i <g, o_i - h>;
//   4. dsrc_i = alpha_i g, plus dz_i (q - z_i k_i / (r rho_i)) / rho_i on the key columns,
//      optionally added to the existing gradient, written in the gradient type (float32, or
//      bf16 rounded to nearest even once after the optional addition);
//   5. dz_i k_i / rho_i is accumulated into per-lane dq partials kept in registers across
//      all rows of the wave.
// At the end the four waves of a workgroup combine their dq partials through LDS in a fixed
// order and write one float64 partial per workgroup; two small kernels then sum those
// partials in a fixed order. The token sum of dq is therefore bitwise reproducible.

#include "lrar_device.h"
#include "lrar_launch.h"

namespace lrar {

namespace {
constexpr int kBwdMaxBlocks = 2048;
constexpr int kReduceGroups = 32;
}  // namespace

// NU: units per lane that cover a row. TU: how many of the last unit slots may hold key
// columns (the host checks that no key unit falls below slot NU - TU).
template <typename IO, typename GIO, int VEC, int NU, int TU>
__global__ __launch_bounds__(kBlock) void k_backward(BwdParams p, double* __restrict__ block_dq) {
  constexpr int B = NU >= 4 ? 1 : (NU >= 2 ? 2 : 4);  // sources loaded together in the <g, o_i> pass
  constexpr int K0 = NU - TU;        // first unit slot that may hold key columns
  __shared__ float lds[kWavesPerBlock][kWave * VEC];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int nur = (p.d + VEC - 1) / VEC;
  const int c0 = p.d - p.r;
  const int ub = c0 / VEC;

  float dqa[TU][VEC];
#pragma unroll
  for (int t = 0; t < TU; ++t)
#pragma unroll
    for (int e = 0; e < VEC; ++e) dqa[t][e] = 0.f;

  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; row < p.T;
       row += step) {
    // 1. weights
    double z, rho;
    row_scores<IO, VEC>(p.src, p.n, row, p.d, p.r, p.eps, p.q, lane, z, rho);
    const double m = wave_max((lane < p.n) ? z : -INFINITY);
    const double ex = (lane < p.n) ? exp(z - m) : 0.0;
    const double a = ex / wave_sum(ex);

    // 2. upstream gradient row
    float gr[NU][VEC];
    const GIO* grow = static_cast<const GIO*>(p.dout) + row * p.dout_ld;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = lane + kWave * k;
      if (u < nur) {
        load_grad<GIO, VEC>(grow + u * VEC, gr[k]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) gr[k][e] = 0.f;
      }
    }

    // 3. s_i = <g, o_i>, then dz_i
    double s_mine = 0.0;
    for (int i = 0; i < p.n; i += B) {
      const int nb = (p.n - i) < B ? (p.n - i) : B;
      Unit<IO, VEC> un[B][NU];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (b < nb) {
          const IO* orow = static_cast<const IO*>(p.src.ptr[i + b]) + row * p.src.ld[i + b];
#pragma unroll
          for (int k = 0; k < NU; ++k) {
            const int u = lane + kWave * k;
            if (u < nur) un[b][k].load_cached(orow + u * VEC); else un[b][k].zero();
          }
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (b < nb) {
          double part = 0.0;
#pragma unroll
          for (int k = 0; k < NU; ++k) {
            float x[VEC];
            un[b][k].get(x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              // keep the float64 copy of g local to this product (no hoisting out of the
              // source loop, which would double g's register footprint)
              float gv = gr[k][e];
              asm volatile("" : "+v"(gv));
              part = fma(static_cast<double>(gv), static_cast<double>(x[e]), part);
            }
          }
          const double s = wave_sum(part);
          if (lane == i + b) s_mine = s;
        }
      }
    }
    const double sbar = wave_sum((lane < p.n) ? a * s_mine : 0.0);
    const double dz = a * (s_mine - sbar);
    const float af = static_cast<float>(a);
    const float c1f = static_cast<float>(dz / rho);                       // dz / rho
    const float c2f = static_cast<float>(dz * z / (p.r * rho * rho));     // dz z / (r rho^2)

    // 4./5. source gradients and dq partials
    for (int i = 0; i < p.n; ++i) {
      const float ai = lane_f32(af, i);
      const float c1 = lane_f32(c1f, i);
      const float c2 = lane_f32(c2f, i);
      const IO* orow = static_cast<const IO*>(p.src.ptr[i]) + row * p.src.ld[i];
      GIO* drow = static_cast<GIO*>(p.dsrc.ptr[i]) + row * p.dsrc.ld[i];
#pragma unroll
      for (int k = 0; k < K0; ++k) {
        const int u = lane + kWave * k;
        if (u < nur) {
          float v[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = ai * gr[k][e];
          if (p.accumulate) {
            float old[VEC];
            load_grad<GIO, VEC>(drow + u * VEC, old);
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] += old[e];
          }
          store_grad<GIO, VEC>(drow + u * VEC, v);
        }
      }
#pragma unroll
      for (int t = 0; t < TU; ++t) {
        const int k = K0 + t;
        const int u = lane + kWave * k;
        if (u < nur) {
          float v[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = ai * gr[k][e];
          if (u >= ub) {
            Unit<IO, VEC> un;
            un.load_cached(orow + u * VEC);
            float x[VEC];
            un.get(x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              const int col = u * VEC + e;
              if (col >= c0) {
                const float qv = p.q[col - c0];
                v[e] += c1 * qv - c2 * x[e];
                dqa[t][e] = fmaf(c1, x[e], dqa[t][e]);
              }
            }
          }
          if (p.accumulate) {
            float old[VEC];
            load_grad<GIO, VEC>(drow + u * VEC, old);
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] += old[e];
          }
          store_grad<GIO, VEC>(drow + u * VEC, v);
        }
      }
    }
  }

  // Combine the four waves' dq partials in a fixed order and write this workgroup's partial.
  double* out = block_dq + static_cast<int64_t>(blockIdx.x) * p.r;
#pragma unroll
  for (int t = 0; t < TU; ++t) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) lds[wave][lane * VEC + e] = dqa[t][e];
    __syncthreads();
    if (wave == 0) {
      const int u = lane + kWave * (K0 + t);
      if (u >= ub && u < nur) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int col = u * VEC + e;
          if (col >= c0) {
            double s = 0.0;
#pragma unroll
            for (int w = 0; w < kWavesPerBlock; ++w) s += static_cast<double>(lds[w][lane * VEC + e]);
            out[col - c0] = s;
          }
        }
      }
    }
    __syncthreads();
  }
}

// Level 1: block (column tile, group) sums its group's workgroup partials for 64 columns.
__global__ __launch_bounds__(kBlock) void k_dq_reduce1(const double* __restrict__ block_dq,
                                                       int nblocks, int r,
                                                       double* __restrict__ level2) {
  __shared__ double lds[kWavesPerBlock][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = blockIdx.x * kWave + lane;
  const int group = blockIdx.y;
  const int per_group = (nblocks + kReduceGroups - 1) / kReduceGroups;
  const int b0 = group * per_group;
  const int b1 = (b0 + per_group) < nblocks ? (b0 + per_group) : nblocks;
  double s = 0.0;
  if (col < r)
    for (int b = b0 + wave; b < b1; b += kWavesPerBlock) s += block_dq[static_cast<int64_t>(b) * r + col];
  lds[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && col < r) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) t += lds[w][lane];
    level2[static_cast<int64_t>(group) * r + col] = t;
  }
}

// Level 2: dq[j] = sum over groups, in order.
__global__ __launch_bounds__(kBlock) void k_dq_reduce2(const double* __restrict__ level2, int r,
                                                       float* __restrict__ dq) {
  const int col = blockIdx.x * kBlock + threadIdx.x;
  if (col >= r) return;
  double s = 0.0;
  for (int g = 0; g < kReduceGroups; ++g) s += level2[static_cast<int64_t>(g) * r + col];
  dq[col] = static_cast<float>(s);
}

namespace {

template <int VEC>
int units_per_lane(int d) {
  const int nur = (d + VEC - 1) / VEC;
  return (nur + kWave - 1) / kWave;
}

// Smallest register window TU (among the built ones) that covers the key for this shape.
int needed_tail_slots(int nu, int d, int r, int vec) {
  const int ub = (d - r) / vec;
  const int first_slot = ub / kWave;  // lanes' unit slots below this never reach the key
  return nu - first_slot;
}

template <typename IO, typename GIO, int VEC, int NU>
hipError_t launch_nu(const BwdParams& p, double* block_dq, int grid, int need, hipStream_t s) {
  const dim3 g(grid), b(kBlock);
  if (need <= 1 && NU >= 1) {
    hipLaunchKernelGGL((k_backward<IO, GIO, VEC, NU, 1>), g, b, 0, s, p, block_dq);
  } else if (need <= 2 && NU >= 2) {
    hipLaunchKernelGGL((k_backward<IO, GIO, VEC, NU, (NU >= 2 ? 2 : NU)>), g, b, 0, s, p,
                       block_dq);
  } else if (need <= 4 && NU >= 4) {
    hipLaunchKernelGGL((k_backward<IO, GIO, VEC, NU, (NU >= 4 ? 4 : NU)>), g, b, 0, s, p,
                       block_dq);
  } else {
    hipLaunchKernelGGL((k_backward<IO, GIO, VEC, NU, NU>), g, b, 0, s, p, block_dq);
  }
  return hipGetLastError();
}

template <typename IO, typename GIO, int VEC>
hipError_t launch_bwd_t(const BwdParams& p, double* block_dq, int grid, hipStream_t s) {
  const int nu = units_per_lane<VEC>(p.d);
  const auto need = [&](int nu_b) { return needed_tail_slots(nu_b, p.d, p.r, VEC); };
  if (nu <= 1) return launch_nu<IO, GIO, VEC, 1>(p, block_dq, grid, need(1), s);
  if (nu <= 2) return launch_nu<IO, GIO, VEC, 2>(p, block_dq, grid, need(2), s);
  if (nu <= 4) return launch_nu<IO, GIO, VEC, 4>(p, block_dq, grid, need(4), s);
  if (nu <= 8) return launch_nu<IO, GIO, VEC, 8>(p, block_dq, grid, need(8), s);
  if (nu <= 16) return launch_nu<IO, GIO, VEC, 16>(p, block_dq, grid, need(16), s);
  if constexpr (VEC == 1) {
    if (nu <= 32) return launch_nu<IO, GIO, VEC, 32>(p, block_dq, grid, need(32), s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int backward_grid(int64_t T) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  return static_cast<int>(blocks < kBwdMaxBlocks ? (blocks > 0 ? blocks : 1) : kBwdMaxBlocks);
}

bool backward_supported(int d, int r, int vec) {
  const int nur = (d + vec - 1) / vec;
  const int nu = (nur + kWave - 1) / kWave;
  return vec > 1 ? nu <= backward_tile_max_chunks() : nu <= 32;
}

// Workspace: [grid][r] float64 workgroup partials, then [kReduceGroups][r] float64.
size_t backward_workspace(int64_t T, int r) {
  if (T <= 0) return 0;
  return (static_cast<size_t>(backward_grid(T)) + kReduceGroups) * static_cast<size_t>(r) * sizeof(double);
}

hipError_t launch_backward(const BwdParams& p, int io_bf16, int grad_bf16, int vec,
                           hipStream_t s) {
  // The workspace holds backward_grid(T) workgroup rows; a launch may fill fewer of them.
  const int max_grid = backward_grid(p.T);
  int grid = max_grid;
  double* block_dq = static_cast<double*>(p.workspace);
  double* level2 = block_dq + static_cast<int64_t>(max_grid) * p.r;
  hipError_t e;
  if (vec > 1) {
    // the vector path runs on row tiles (lrar_backward_tile.hip)
    e = launch_backward_tile(p, io_bf16, grad_bf16, block_dq, max_grid, &grid, s);
  } else if (io_bf16) {
    e = grad_bf16 ? launch_bwd_t<bf16_bits, bf16_bits, 1>(p, block_dq, grid, s)
                  : launch_bwd_t<bf16_bits, float, 1>(p, block_dq, grid, s);
  } else {
    e = grad_bf16 ? launch_bwd_t<float, bf16_bits, 1>(p, block_dq, grid, s)
                  : launch_bwd_t<float, float, 1>(p, block_dq, grid, s);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dq_reduce1, dim3((p.r + kWave - 1) / kWave, kReduceGroups), dim3(kBlock), 0, s,
                     block_dq, grid, p.r, level2);
  hipLaunchKernelGGL(k_dq_reduce2, dim3((p.r + kBlock - 1) / kBlock), dim3(kBlock), 0, s, level2, p.r,
                     p.dq);
  return hipGetLastError();
}

}  // namespace lrar
