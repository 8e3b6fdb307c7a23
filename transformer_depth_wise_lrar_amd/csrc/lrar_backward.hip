// Backward of the depth-mix read on one wavefront per token row, and the dq reduction
// (LR-AttnRes paper App. B.3: Lemma 2 gives dL/do_i = alpha_i g + alpha_i <g, o_i - h> grad z_i;
// Corollary 2.1 gives the slice-RMS gradient grad z_i = P_r^T (q - z_i kbar_i / r) / rho_i; the
// query gradient follows from z_i = q . kbar_i). Each source slot is an independent input, as
// in the paper. k_backward serves the rows the row-tile backward (lrar_backward_tile.hip) does
// not: the scalar-element path (unaligned widths or strides) at any width, and vector rows wider
// than a tile.
//
// k_backward, one wavefront per token row:
//   1. key pass (float64): z_i, rho_i, alpha_i of every source, as in the forward (or z_i and
//      rho_i from the forward's saved statistics);
//   2. s_i = <g, o_i> over all d (float64 sums of exact products), streaming g = dL/dh and the
//      source rows in column chunks (g is read again from the cache for every source); then
//      dz_i = alpha_i (s_i - sum_j alpha_j s_j), which equals alpha_i <g, o_i - h>;
//   3. dsrc_i = alpha_i g, plus dz_i (q - z_i k_i / (r rho_i)) / rho_i on the key columns,
//      optionally added to the existing gradient, written in the gradient type (float32, or
//      bf16 rounded to nearest even once after the optional addition);
//   4. dz_i k_i / rho_i is accumulated into per-lane dq partials kept in registers across all
//      rows of the wave. Only the key's columns have partials: the key window is the TU chunks
//      of 64 units from the chunk that holds the key's first unit (TU <= 64 on the element
//      path, <= 8 on the vector path), which bounds the key width this kernel serves.
// At the end the four waves of a workgroup combine their dq partials through LDS in a fixed
// order and write one float64 partial per workgroup; two small kernels then sum those
// partials in a fixed order. The token sum of dq is therefore bitwise reproducible.

#include "lrar_device.h"
#include "lrar_launch.h"

namespace lrar {

namespace {
constexpr int kBwdMaxBlocks = 2048;
constexpr int kReduceGroups = 32;
constexpr int kElemMaxWindow = 64;  // key-window chunks on the element path
constexpr int kVecMaxWindow = 8;    // and on the vector path (VEC floats per slot)

// First unit of the key window: the start of the 64-unit chunk holding the key's first unit.
__host__ __device__ __forceinline__ int key_window_start(int d, int r, int vec) {
  return (((d - r) / vec) / kWave) * kWave;
}
}  // namespace

template <typename IO, typename GIO, int VEC, int TU>
__global__ __launch_bounds__(kBlock) void k_backward(BwdParams p, double* __restrict__ block_dq) {
  __shared__ float lds[kWavesPerBlock][kWave * VEC];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int nur = (p.d + VEC - 1) / VEC;
  const int c0 = p.d - p.r;
  const int ub = c0 / VEC;
  const int ws = key_window_start(p.d, p.r, VEC);

  float dqa[TU][VEC];
#pragma unroll
  for (int t = 0; t < TU; ++t)
#pragma unroll
    for (int e = 0; e < VEC; ++e) dqa[t][e] = 0.f;

  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; row < p.T;
       row += step) {
    // 1. weights (the scores and key RMS from the forward's saved statistics when given)
    double z = 0.0, rho = 1.0;
    if (p.saved != nullptr) {
      if (lane < p.n) {
        z = p.saved[row * p.saved_ld + lane];
        rho = 1.0 / p.saved[row * p.saved_ld + p.n + lane];
      }
    } else {
      row_scores<IO, VEC>(p.src, p.n, row, p.d, p.r, p.eps, p.q, lane, z, rho);
    }
    const double m = wave_max((lane < p.n) ? z : -INFINITY);
    const double ex = (lane < p.n) ? exp(z - m) : 0.0;
    const double a = ex / wave_sum(ex);
    const GIO* grow = static_cast<const GIO*>(p.dout) + row * p.dout_ld;

    // 2. s_i = <g, o_i>, then dz_i
    double s_mine = 0.0;
    for (int i = 0; i < p.n; ++i) {
      const IO* orow = static_cast<const IO*>(p.src.ptr[i]) + row * p.src.ld[i];
      double part = 0.0;
#pragma unroll 4
      for (int u = lane; u < nur; u += kWave) {
        float gv[VEC], x[VEC];
        load_grad<GIO, VEC>(grow + u * VEC, gv);
        Unit<IO, VEC> un;
        un.load_cached(orow + u * VEC);
        un.get(x);
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          part = fma(static_cast<double>(gv[e]), static_cast<double>(x[e]), part);
      }
      const double s = wave_sum(part);
      if (lane == i) s_mine = s;
    }
    const double sbar = wave_sum((lane < p.n) ? a * s_mine : 0.0);
    const double dz = a * (s_mine - sbar);
    const float af = static_cast<float>(a);
    // d z / d k_j = (q_j - w k_j) / rho with w = z / (r rho). The difference cancels when r is
    // small (at r = 1 it is q (1 - kbar^2), about q eps / k^2), so w is held as two floats
    // w = wh + wl: q_j - wh k_j is taken by one fused multiply-add, whose single rounding
    // falls on the small result, and (dz / rho) wl k_j is taken off the gradient after it.
    const float c1f = static_cast<float>(dz / rho);  // dz / rho
    const double wd = z / (p.r * rho);
    const float whf = static_cast<float>(wd);
    const float c1wlf = static_cast<float>(static_cast<double>(c1f) * (wd - static_cast<double>(whf)));

    // 3./4. source gradients and dq partials
    for (int i = 0; i < p.n; ++i) {
      const float ai = lane_f32(af, i);
      const float c1 = lane_f32(c1f, i);
      const float wh = lane_f32(whf, i);
      const float c1wl = lane_f32(c1wlf, i);
      const IO* orow = static_cast<const IO*>(p.src.ptr[i]) + row * p.src.ld[i];
      GIO* drow = static_cast<GIO*>(p.dsrc.ptr[i]) + row * p.dsrc.ld[i];
      // columns before the key window: alpha_i g only
#pragma unroll 2
      for (int u = lane; u < ws; u += kWave) {
        float v[VEC];
        load_grad<GIO, VEC>(grow + u * VEC, v);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] *= ai;
        if (p.accumulate) {
          float old[VEC];
          load_grad<GIO, VEC>(drow + u * VEC, old);
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] += old[e];
        }
        store_grad<GIO, VEC>(drow + u * VEC, v);
      }
      // the key window, one register slot per chunk
#pragma unroll
      for (int t = 0; t < TU; ++t) {
        const int u = ws + kWave * t + lane;
        if (u < nur) {
          float v[VEC];
          load_grad<GIO, VEC>(grow + u * VEC, v);
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] *= ai;
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
                v[e] = fmaf(c1, fmaf(-wh, x[e], qv), v[e]);
                v[e] = fmaf(-c1wl, x[e], v[e]);
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
      const int u = ws + kWave * t + lane;
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

// Key-window chunks this shape needs (see k_backward).
int key_window_chunks(int d, int r, int vec) {
  const int nur = (d + vec - 1) / vec;
  return (nur - key_window_start(d, r, vec) + kWave - 1) / kWave;
}

template <typename IO, typename GIO, int VEC, int TU>
void launch_tu(const BwdParams& p, double* block_dq, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_backward<IO, GIO, VEC, TU>), dim3(grid), dim3(kBlock), 0, s, p, block_dq);
}

template <typename IO, typename GIO, int VEC>
hipError_t launch_bwd_t(const BwdParams& p, double* block_dq, int grid, hipStream_t s) {
  const int need = key_window_chunks(p.d, p.r, VEC);
  if (need <= 1) launch_tu<IO, GIO, VEC, 1>(p, block_dq, grid, s);
  else if (need <= 2) launch_tu<IO, GIO, VEC, 2>(p, block_dq, grid, s);
  else if (need <= 4) launch_tu<IO, GIO, VEC, 4>(p, block_dq, grid, s);
  else if (need <= 8) launch_tu<IO, GIO, VEC, 8>(p, block_dq, grid, s);
  else if constexpr (VEC == 1) {
    if (need <= 16) launch_tu<IO, GIO, VEC, 16>(p, block_dq, grid, s);
    else if (need <= 32) launch_tu<IO, GIO, VEC, 32>(p, block_dq, grid, s);
    else if (need <= 64) launch_tu<IO, GIO, VEC, 64>(p, block_dq, grid, s);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int backward_grid(int64_t T) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  return static_cast<int>(blocks < kBwdMaxBlocks ? (blocks > 0 ? blocks : 1) : kBwdMaxBlocks);
}

bool backward_uses_tile(int d, int vec) {
  const int nur = (d + vec - 1) / vec;
  return vec > 1 && (nur + kWave - 1) / kWave <= backward_tile_max_chunks();
}

bool backward_supported(int d, int r, int vec) {
  if (backward_uses_tile(d, vec)) return true;
  return key_window_chunks(d, r, vec) <= (vec > 1 ? kVecMaxWindow : kElemMaxWindow);
}

// Workspace: [grid][r] float64 workgroup partials, then [kReduceGroups][r] float64.
size_t backward_workspace(int64_t T, int r) {
  if (T <= 0) return 0;
  return backward_workspace_rows(backward_grid(T), r);
}

size_t backward_workspace_rows(int grid, int r) {
  return (static_cast<size_t>(grid) + kReduceGroups) * static_cast<size_t>(r) * sizeof(double);
}

hipError_t launch_backward(const BwdParams& p, int io_bf16, int grad_bf16, int vec,
                           hipStream_t s, int ws_grid) {
  // The workspace holds max_grid workgroup rows (backward_grid(T) unless the caller sized it
  // for fewer); a launch may fill fewer of them.
  const int max_grid = ws_grid > 0 ? ws_grid : backward_grid(p.T);
  int grid = max_grid;
  double* block_dq = static_cast<double*>(p.workspace);
  double* level2 = block_dq + static_cast<int64_t>(max_grid) * p.r;
  hipError_t e;
  if (backward_uses_tile(p.d, vec)) {
    // vector rows that fit a tile run on row tiles (lrar_backward_tile.hip)
    e = launch_backward_tile(p, io_bf16, grad_bf16, block_dq, max_grid, &grid, s);
  } else if (io_bf16) {
    if (vec > 1)
      e = grad_bf16 ? launch_bwd_t<bf16_bits, bf16_bits, 8>(p, block_dq, grid, s)
                    : launch_bwd_t<bf16_bits, float, 8>(p, block_dq, grid, s);
    else
      e = grad_bf16 ? launch_bwd_t<bf16_bits, bf16_bits, 1>(p, block_dq, grid, s)
                    : launch_bwd_t<bf16_bits, float, 1>(p, block_dq, grid, s);
  } else {
    if (vec > 1)
      e = grad_bf16 ? launch_bwd_t<float, bf16_bits, 4>(p, block_dq, grid, s)
                    : launch_bwd_t<float, float, 4>(p, block_dq, grid, s);
    else
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
