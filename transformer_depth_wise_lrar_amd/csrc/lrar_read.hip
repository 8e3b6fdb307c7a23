// The column-chunked read and merge (LR-AttnRes paper §3.1/§3.3 and §3.4; AttnRes
// technical-report summary, "Method", for the two-phase schedule).
//
// k_read_two_pass, one wavefront per token row: the key slices of all n sources are loaded
// and reduced (float64), the softmax is taken once, then the full rows are streamed in column
// chunks with float32 accumulation. It handles any width, so it serves the rows that do not
// fit a register tile (lrar_tile.hip), including the scalar-element path for wide unaligned
// rows.
//
// With PRIOR the kernel merges Phase-1 statistics (m, l, acc) of earlier sources into the
// softmax as one more term; that is lrar_merge for such rows.

#include "lrar_device.h"
#include "lrar_launch.h"

namespace lrar {

namespace {

// Weights of one row. On return lane i < n holds w_i = e_i / L in float32, and w_prior is
// the coefficient of the prior accumulator (0 without PRIOR).
template <bool PRIOR>
__device__ __forceinline__ void row_weights(const ReadParams& p, int64_t row, int lane,
                                            double z, float& w, float& w_prior, float& m_f_out,
                                            float& l_out) {
  double m = (lane < p.n) ? z : -INFINITY;
  m = wave_max(m);
  double m_prior = 0.0, l_prior = 0.0;
  if constexpr (PRIOR) {
    m_prior = static_cast<double>(p.m_in[row]);
    l_prior = static_cast<double>(p.l_in[row]);
    m = fmax(m, m_prior);
  }
  // With PRIOR the running maximum is rounded to float32 first, so that an (m', l') pair
  // written back is self-consistent.
  const double mr = PRIOR ? static_cast<double>(static_cast<float>(m)) : m;
  const double e = (lane < p.n) ? exp(z - mr) : 0.0;
  double L = wave_sum(e);
  double c_prior = 0.0;
  if constexpr (PRIOR) {
    c_prior = exp(m_prior - mr);  // e^{m - m'}
    L = fma(l_prior, c_prior, L);
  }
  const double inv = 1.0 / L;
  w = static_cast<float>(e * inv);
  w_prior = static_cast<float>(c_prior * inv);
  m_f_out = static_cast<float>(mr);
  l_out = static_cast<float>(L);
}

}  // namespace

template <typename IO, int VEC, int NUC, bool PRIOR, typename ACC>
__global__ __launch_bounds__(kBlock) void k_read_two_pass(ReadParams p) {
  constexpr int B = (16 / NUC) > 1 ? (16 / NUC) : 1;  // sources loaded together
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int nur = (p.d + VEC - 1) / VEC;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; row < p.T;
       row += step) {
    double z, rho;
    row_scores<IO, VEC>(p.src, p.n, row, p.d, p.r, p.eps, p.q, lane, z, rho);
    float w, w_prior, m_f, l_f;
    row_weights<PRIOR>(p, row, lane, z, w, w_prior, m_f, l_f);
    if (p.alpha != nullptr && lane < p.n) p.alpha[row * p.alpha_ld + lane] = w;
    if constexpr (PRIOR) {
      if (lane == 0) {
        if (p.m_out) p.m_out[row] = m_f;
        if (p.l_out) p.l_out[row] = l_f;
      }
    }
    IO* out_row = static_cast<IO*>(p.out) + row * p.out_ld;
    for (int cb = 0; cb < nur; cb += kWave * NUC) {
      float acc[NUC][VEC];
      if constexpr (PRIOR) {
        const ACC* prow = static_cast<const ACC*>(p.acc) + row * p.acc_ld;
#pragma unroll
        for (int k = 0; k < NUC; ++k) {
          const int u = cb + lane + kWave * k;
          float x[VEC];
          if (u < nur) {
            load_acc<ACC, VEC>(prow + u * VEC, x);
          } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = 0.f;
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[k][e] = w_prior * x[e];
        }
      } else {
#pragma unroll
        for (int k = 0; k < NUC; ++k)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[k][e] = 0.f;
      }
      int i = 0;
      for (; i + B <= p.n; i += B) {
        Unit<IO, VEC> un[B][NUC];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const IO* srow = static_cast<const IO*>(p.src.ptr[i + b]) + row * p.src.ld[i + b];
#pragma unroll
          for (int k = 0; k < NUC; ++k) {
            const int u = cb + lane + kWave * k;
            if (u < nur) un[b][k].load(srow + u * VEC); else un[b][k].zero();
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float wb = lane_f32(w, i + b);
#pragma unroll
          for (int k = 0; k < NUC; ++k) {
            float x[VEC];
            un[b][k].get(x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[k][e] = fmaf(wb, x[e], acc[k][e]);
          }
        }
      }
      for (; i < p.n; ++i) {
        const IO* srow = static_cast<const IO*>(p.src.ptr[i]) + row * p.src.ld[i];
        const float wi = lane_f32(w, i);
#pragma unroll
        for (int k = 0; k < NUC; ++k) {
          const int u = cb + lane + kWave * k;
          Unit<IO, VEC> un;
          if (u < nur) un.load(srow + u * VEC); else un.zero();
          float x[VEC];
          un.get(x);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[k][e] = fmaf(wi, x[e], acc[k][e]);
        }
      }
#pragma unroll
      for (int k = 0; k < NUC; ++k) {
        const int u = cb + lane + kWave * k;
        if (u < nur) store_unit<IO, VEC>(out_row + u * VEC, acc[k]);
      }
    }
  }
}

// ---- launchers ---------------------------------------------------------------------------------

namespace {

int grid_for_rows(int64_t T) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = 65536;
  return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

template <typename IO, int VEC, bool PRIOR, typename ACC>
hipError_t launch_two_pass_t(const ReadParams& p, hipStream_t s) {
  const int grid = grid_for_rows(p.T);
  const int nur = (p.d + VEC - 1) / VEC;
  if (nur <= kWave * 1)
    hipLaunchKernelGGL((k_read_two_pass<IO, VEC, 1, PRIOR, ACC>), dim3(grid), dim3(kBlock), 0, s, p);
  else if (nur <= kWave * 2 || VEC == 1)
    hipLaunchKernelGGL((k_read_two_pass<IO, VEC, 2, PRIOR, ACC>), dim3(grid), dim3(kBlock), 0, s, p);
  else
    hipLaunchKernelGGL((k_read_two_pass<IO, VEC, 4, PRIOR, ACC>), dim3(grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_read(const ReadParams& p, ReadKind kind, int io_bf16, int vec, int acc_bf16,
                       hipStream_t s) {
  if (kind == ReadKind::kTwoPass || kind == ReadKind::kOnline) {
    if (io_bf16) return vec > 1 ? launch_two_pass_t<bf16_bits, 8, false, float>(p, s)
                                : launch_two_pass_t<bf16_bits, 1, false, float>(p, s);
    return vec > 1 ? launch_two_pass_t<float, 4, false, float>(p, s)
                   : launch_two_pass_t<float, 1, false, float>(p, s);
  }
  // merge: two-pass with a prior accumulator of type float or bf16
  if (io_bf16) {
    if (acc_bf16) return vec > 1 ? launch_two_pass_t<bf16_bits, 8, true, bf16_bits>(p, s)
                                 : launch_two_pass_t<bf16_bits, 1, true, bf16_bits>(p, s);
    return vec > 1 ? launch_two_pass_t<bf16_bits, 8, true, float>(p, s)
                   : launch_two_pass_t<bf16_bits, 1, true, float>(p, s);
  }
  if (acc_bf16) return vec > 1 ? launch_two_pass_t<float, 4, true, bf16_bits>(p, s)
                               : launch_two_pass_t<float, 1, true, bf16_bits>(p, s);
  return vec > 1 ? launch_two_pass_t<float, 4, true, float>(p, s)
                 : launch_two_pass_t<float, 1, true, float>(p, s);
}

}  // namespace lrar
