// The column-chunked read and merge (LR-AttnRes paper §3.1/§3.3 and §3.4; AttnRes
// technical-report summary, "Method", for the two-phase schedule).
//
// k_read_two_pass, one wavefront per token row: the keys of all n sources are loaded and
// reduced (float64), the softmax is taken once, then the full rows are streamed in column
// chunks with float32 accumulation. It handles any width, so it serves the rows that do not
// fit a register tile (lrar_tile.hip), including the scalar-element path for wide unaligned
// rows. KM picks the key: the row's last r columns (the read), the same columns over the
// whole row's RMS (the full-width-RMS control, LR-AttnRes paper §4.4 Eq. 13), or the source's
// own key row (the separate-key read, App. C.1-C.2).
//
// With PRIOR the kernel merges Phase-1 statistics (m, l, acc) of earlier sources into the
// softmax as one more term; that is lrar_merge for such rows.
//
// k_add_rows forms b' = b + o (rounded to the element type) for the fused Phase-2 update on
// rows too wide for a tile; the merge then reads b' as its one extra source.

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

template <typename IO, int VEC, int NUC, bool PRIOR, typename ACC, int KM>
__global__ __launch_bounds__(kBlock) void k_read_two_pass(ReadParams p, SrcList keys) {
  constexpr int B = (16 / NUC) > 1 ? (16 / NUC) : 1;  // sources loaded together
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int nur = (p.d + VEC - 1) / VEC;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave; row < p.T;
       row += step) {
    double z, rho;
    row_scores<IO, VEC, KM>(p.src, p.n, row, p.d, p.r, p.eps, p.q, lane, z, rho, &keys);
    float w, w_prior, m_f, l_f;
    row_weights<PRIOR>(p, row, lane, z, w, w_prior, m_f, l_f);
    if (p.alpha != nullptr && lane < p.n) p.alpha[row * p.alpha_ld + lane] = w;
    if (p.saved != nullptr && lane < p.n) {
      double* srow = p.saved + row * p.saved_ld;
      srow[lane] = z;
      srow[p.n + lane] = 1.0 / rho;
    }
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

// b_out = b + o element by element (b may be null: b_out = o), rounded to the element type;
// b_out may be b or o itself (each element is read before it is written, by the same lane).
template <typename IO, int VEC>
__global__ __launch_bounds__(kBlock) void k_add_rows(const IO* b, int64_t b_ld, const IO* o,
                                                     int64_t o_ld, IO* bout, int64_t bout_ld,
                                                     int64_t T, int d) {
  const int nur = (d + VEC - 1) / VEC;
  const int64_t total = T * nur;
  const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; idx < total;
       idx += step) {
    const int64_t row = idx / nur;
    const int u = static_cast<int>(idx - row * nur);
    Unit<IO, VEC> uo;
    uo.load(o + row * o_ld + u * VEC);
    float x[VEC];
    uo.get(x);
    if (b != nullptr) {
      Unit<IO, VEC> ub;
      ub.load(b + row * b_ld + u * VEC);
      float y[VEC];
      ub.get(y);
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] += y[e];
    }
    store_unit<IO, VEC>(bout + row * bout_ld + u * VEC, x);
  }
}

// ---- launchers ---------------------------------------------------------------------------------

namespace {

int grid_for_rows(int64_t T) {
  const int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = 65536;
  return static_cast<int>(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

template <typename IO, int VEC, bool PRIOR, typename ACC, int KM>
hipError_t launch_two_pass_t(const ReadParams& p, const SrcList& keys, hipStream_t s) {
  const int grid = grid_for_rows(p.T);
  const int nur = (p.d + VEC - 1) / VEC;
  if (nur <= kWave * 1)
    hipLaunchKernelGGL((k_read_two_pass<IO, VEC, 1, PRIOR, ACC, KM>), dim3(grid), dim3(kBlock), 0,
                       s, p, keys);
  else if (nur <= kWave * 2 || VEC == 1)
    hipLaunchKernelGGL((k_read_two_pass<IO, VEC, 2, PRIOR, ACC, KM>), dim3(grid), dim3(kBlock), 0,
                       s, p, keys);
  else
    hipLaunchKernelGGL((k_read_two_pass<IO, VEC, 4, PRIOR, ACC, KM>), dim3(grid), dim3(kBlock), 0,
                       s, p, keys);
  return hipGetLastError();
}

template <typename IO, int VEC, int KM>
hipError_t launch_read_km(const ReadParams& p, bool prior, int acc_bf16, const SrcList& keys,
                          hipStream_t s) {
  if (!prior) return launch_two_pass_t<IO, VEC, false, float, KM>(p, keys, s);
  return acc_bf16 ? launch_two_pass_t<IO, VEC, true, bf16_bits, KM>(p, keys, s)
                  : launch_two_pass_t<IO, VEC, true, float, KM>(p, keys, s);
}

template <typename IO, int VEC>
hipError_t launch_read_io(const ReadParams& p, bool prior, int acc_bf16, int key_mode,
                          const SrcList* keys, hipStream_t s) {
  if (key_mode == kKeySeparate) return launch_read_km<IO, VEC, kKeySeparate>(p, false, 0, *keys, s);
  SrcList none;
  none.ptr[0] = nullptr;
  none.ld[0] = 0;
  if (key_mode == kKeyFullRms) return launch_read_km<IO, VEC, kKeyFullRms>(p, false, 0, none, s);
  return launch_read_km<IO, VEC, kKeySlice>(p, prior, acc_bf16, none, s);
}

}  // namespace

hipError_t launch_read(const ReadParams& p, ReadKind kind, int io_bf16, int vec, int acc_bf16,
                       hipStream_t s, int key_mode, const SrcList* keys) {
  // two-pass for the read (online needs a register tile), with a prior accumulator for merges
  const bool prior = kind == ReadKind::kMerge;
  if (io_bf16) return vec > 1 ? launch_read_io<bf16_bits, 8>(p, prior, acc_bf16, key_mode, keys, s)
                              : launch_read_io<bf16_bits, 1>(p, prior, acc_bf16, key_mode, keys, s);
  return vec > 1 ? launch_read_io<float, 4>(p, prior, acc_bf16, key_mode, keys, s)
                 : launch_read_io<float, 1>(p, prior, acc_bf16, key_mode, keys, s);
}

hipError_t launch_add_rows(const void* b, int64_t b_ld, const void* o, int64_t o_ld, void* bout,
                           int64_t bout_ld, int64_t T, int d, int io_bf16, int vec,
                           hipStream_t s) {
  const int64_t units = T * ((d + vec - 1) / vec);
  int64_t blocks = (units + kBlock - 1) / kBlock;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  const dim3 g(static_cast<unsigned>(blocks)), bk(kBlock);
  if (io_bf16) {
    using T16 = bf16_bits;
    if (vec > 1)
      hipLaunchKernelGGL((k_add_rows<T16, 8>), g, bk, 0, s, static_cast<const T16*>(b), b_ld,
                         static_cast<const T16*>(o), o_ld, static_cast<T16*>(bout), bout_ld, T, d);
    else
      hipLaunchKernelGGL((k_add_rows<T16, 1>), g, bk, 0, s, static_cast<const T16*>(b), b_ld,
                         static_cast<const T16*>(o), o_ld, static_cast<T16*>(bout), bout_ld, T, d);
  } else {
    if (vec > 1)
      hipLaunchKernelGGL((k_add_rows<float, 4>), g, bk, 0, s, static_cast<const float*>(b), b_ld,
                         static_cast<const float*>(o), o_ld, static_cast<float*>(bout), bout_ld, T,
                         d);
    else
      hipLaunchKernelGGL((k_add_rows<float, 1>), g, bk, 0, s, static_cast<const float*>(b), b_ld,
                         static_cast<const float*>(o), o_ld, static_cast<float*>(bout), bout_ld, T,
                         d);
  }
  return hipGetLastError();
}

}  // namespace lrar
