// Backward of the depth-mix read on row tiles (LR-AttnRes paper App. B.3: Lemma 2 gives
// dL/do_i = alpha_i g + alpha_i <g, o_i - h> grad z_i; Corollary 2.1 gives the slice-RMS
// gradient grad z_i = P_r^T (q - z_i kbar_i / r) / rho_i; the query gradient follows from
// z_i = q . kbar_i). Each source slot is an independent input, as in the paper.
//
// A row group (one wave, or the four waves of a workgroup for wide rows, each holding every
// fourth chunk of 64 units as in lrar_tile.hip) takes one token row at a time, rows dealt out
// in bands:
//   pass A  the upstream gradient g of the row is loaded once into registers; the sources
//           stream through a prefetch ring and, from each row, the float64 sums q . k, k . k
//           and s_i = <g, o_i> are reduced (DPP, then across the row's waves through LDS in a
//           fixed order); lane i keeps z_i, 1 / rho_i, s_i. With the forward's saved statistics
//           (SAVED) z_i and 1 / rho_i are read from them and only s_i is reduced;
//   then    alpha = softmax(z), sbar = sum_j alpha_j s_j, dz_i = alpha_i (s_i - sbar), which
//           equals alpha_i <g, o_i - h>;
//   pass B  dsrc_i = alpha_i g, plus dz_i (q - z_i k_i / (r rho_i)) / rho_i on the key columns
//           (the key units were kept in LDS in pass A when n r elements fit 32 KiB per row
//           group; otherwise they are read again), written in the gradient type (float32,
//           or bf16 rounded once; optionally added to the existing gradient first); dz_i k_i /
//           rho_i accumulates into per-lane dq partials kept in registers across the group's
//           rows.
// The dq partials of a workgroup are combined in a fixed order and written as one float64 row
// of the workspace; the reduction kernels of lrar_backward.hip then sum the workgroups' rows in
// a fixed order, so dq is bitwise reproducible.

#include <type_traits>

#include "lrar_device.h"
#include "lrar_launch.h"
#include "lrar_tile.h"

namespace lrar {

template <typename IO, typename GIO, int VEC, int NU, int TU, int WPR, bool SAVED>
__global__ __launch_bounds__(kBlock) void k_backward_tile(BwdParams p, double* __restrict__ block_dq) {
  static_assert(kWavesPerBlock % WPR == 0, "a workgroup holds whole row groups");
  constexpr int PF = 2;
  constexpr int K0 = NU - TU;  // first unit slot that may hold key columns
  constexpr bool kRunStores = std::is_same<GIO, float>::value && VEC == 8;
  extern __shared__ __attribute__((aligned(16))) float q_lds[];
  __shared__ double xch[2][kWavesPerBlock][3];
  const int lane = threadIdx.x & (kWave - 1);
  const int wib = wave_in_block();
  const int64_t group = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wib) / WPR;
  const int64_t ngroups = static_cast<int64_t>(gridDim.x) * kWavesPerBlock / WPR;
  const int n = p.n;
  TileGeom g;
  g.lane = lane;
  g.w = wib % WPR;
  g.wpr = WPR;
  g.nur = (p.d + VEC - 1) / VEC;
  g.c0 = p.d - p.r;
  g.ub = g.c0 / VEC;
  g.r = p.r;
  const double rinv_r = 1.0 / static_cast<double>(p.r);
  const int rq = p.d - g.ub * VEC;  // staged query columns
  QStage qst;
  qst.base = q_lds;
  qst.nv = g.nur - g.ub;
  qst.fill<VEC>(p.q, g.ub, g.c0, threadIdx.x, kBlock);
  // Key stash (when the host sized it): the key units of every source of the row group's
  // current row, written in pass A and read back in pass B by the lane that wrote them.
  const int nkey = g.nur - g.ub;
  Unit<IO, VEC>* stash = nullptr;
  if (p.key_stash)
    stash = reinterpret_cast<Unit<IO, VEC>*>(q_lds + ((rq + 3) & ~3)) +
            static_cast<int64_t>(wib / WPR) * n * nkey;
  __syncthreads();

  float dqa[TU][VEC];
#pragma unroll
  for (int t = 0; t < TU; ++t)
#pragma unroll
    for (int e = 0; e < VEC; ++e) dqa[t][e] = 0.f;

  int parity = 0;
  const auto src_base = [&](int i) { return static_cast<const IO*>(p.src.ptr[i]); };
  // One-wave rows of up to two chunks (d <= 1024 bf16) meet at a workgroup barrier once per
  // row, as the reads keep their waves in lockstep: +7 % (fp32 gradients, 10 sources) and +1 %
  // (49 sources) at d = 1024, bf16 gradients level; at d = 2048 it measured 1.9 % slower with
  // fp32 gradients. It is taken only in the steps where every row group of the workgroup has a
  // row, a condition the same for all of its waves.
  constexpr bool kLockRows = WPR == 1 && NU <= 2;
  const int64_t last_group =
      (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + kWavesPerBlock - 1) / WPR;
  for (int64_t row = group; row < p.T; row += ngroups) {
    if (kLockRows && (row - group) + last_group < p.T) __syncthreads();
    g.r0 = row;
    g.nrow = 1;
    // upstream gradient of the row
    float gr[NU][VEC];
    const GIO* grow = static_cast<const GIO*>(p.dout) + row * p.dout_ld;
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = g.unit(k);
      if (u < g.nur) {
        load_grad<GIO, VEC>(grow + u * VEC, gr[k]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) gr[k][e] = 0.f;
      }
    }

    // ---- pass A: z_i, 1 / rho_i, s_i (lane i)
    double zi = 0.0, rinvi = 1.0, si = 0.0;
    if constexpr (SAVED) {
      if (lane < n) {
        const double* srow = p.saved + row * p.saved_ld;
        zi = srow[lane];
        rinvi = srow[n + lane];
      }
    }
    Stage<IO, VEC, NU, 1, 0> ring[PF + 1];
    const auto fold_a = [&](const Stage<IO, VEC, NU, 1, 0>& st, int i) {
      double red[3] = {0.0, 0.0, 0.0};
      if constexpr (!SAVED) key_partial_units<TU>(st.t.u[0], qst, g, red[0], red[1]);
      double s = 0.0;
#pragma unroll
      for (int k = 0; k < NU; ++k) {
        float x[VEC];
        st.t.u[0][k].get(x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          // the float64 copy of g stays local to the product (hoisting it out of the source
          // loop would double g's register footprint)
          float gv = gr[k][e];
          asm volatile("" : "+v"(gv));
          s = fma(static_cast<double>(gv), static_cast<double>(x[e]), s);
        }
      }
      red[2] = s;
      if constexpr (SAVED) {
        // only g . o: the transposed butterfly of two values (the second zero) leaves it in
        // lane 0 (transposed_index<1>(0) = 0)
        const double v2[2] = {s, 0.0};
        const double x = wave_sums_transposed<1>(v2, lane);
        if constexpr (WPR == 1) {
          red[2] = lane_f64(x, 0);
        } else {
          if (lane == 0) xch[parity][wib][2] = x;
          __syncthreads();
          const int base = wib - g.w;
          double t = xch[parity][base][2];
#pragma unroll
          for (int v = 1; v < WPR; ++v) t += xch[parity][base + v][2];
          red[2] = t;
          parity ^= 1;
        }
        if (lane == i) si = red[2];
      } else {
        // The three sums (q . k, k . k, g . o) by the transposed butterfly, as a fourth zero
        // value: lane l < 4 then holds sum v4[transposed_index<2>(l)].
        const double v4[4] = {red[0], red[1], red[2], 0.0};
        const double x = wave_sums_transposed<2>(v4, lane);
        if constexpr (WPR == 1) {
          // transposed_index<2>: lane 0 holds q . k, lane 2 k . k, lane 1 g . o
          red[0] = lane_f64(x, 0);
          red[1] = lane_f64(x, 2);
          red[2] = lane_f64(x, 1);
        } else {
          const int idx = transposed_index<2>(lane);
          if (lane < 4 && idx < 3) xch[parity][wib][idx] = x;
          __syncthreads();
          const int base = wib - g.w;
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            double t = xch[parity][base][j];
#pragma unroll
            for (int v = 1; v < WPR; ++v) t += xch[parity][base + v][j];
            red[j] = t;
          }
          parity ^= 1;
        }
        const Score sc = score_from_sums(red[0], red[1], rinv_r, p.eps);
        if (lane == i) {
          zi = sc.z;
          rinvi = sc.rinv;
          si = red[2];
        }
      }
      if (stash != nullptr) {
#pragma unroll
        for (int k = K0; k < NU; ++k) {
          const int u = g.unit(k);
          if (u >= g.ub && u < g.nur) stash[i * nkey + (u - g.ub)] = st.t.u[0][k];
        }
      }
    };
#pragma unroll
    for (int b = 0; b < PF; ++b)
      if (b < n) load_stage<false>(ring[b], src_base(b), p.src.ld[b], g);
    for (int i0 = 0; i0 < n; i0 += PF + 1) {
#pragma unroll
      for (int b = 0; b <= PF; ++b) {
        const int i = i0 + b;
        if (i < n) {
          if (i + PF < n)
            load_stage<false>(ring[(b + PF) % (PF + 1)], src_base(i + PF), p.src.ld[i + PF], g);
          fold_a(ring[b], i);
        }
      }
    }

    // ---- weights and score gradients (lanes = sources)
    const double m = wave_max_dpp(lane < n ? zi : -INFINITY);
    const double ex = lane < n ? exp(zi - m) : 0.0;
    const double a = ex / wave_sum_dpp(ex);
    const double sbar = wave_sum_dpp(lane < n ? a * si : 0.0);
    const double dz = a * (si - sbar);
    const float af = static_cast<float>(a);
    // d z / d k_j = (q_j - w k_j) / rho with w = z / (r rho). The difference cancels when r is
    // small (at r = 1 it is q (1 - kbar^2), about q eps / k^2), so w is held as two floats
    // w = wh + wl: q_j - wh k_j is taken by one fused multiply-add, whose single rounding
    // falls on the small result, and (dz / rho) wl k_j is taken off the gradient after it.
    const float c1f = static_cast<float>(dz * rinvi);  // dz / rho
    const double wd = zi * rinvi * rinv_r;
    const float whf = static_cast<float>(wd);
    const float c1wlf = static_cast<float>(static_cast<double>(c1f) * (wd - static_cast<double>(whf)));

    // ---- pass B: source gradients (the key units from the LDS stash, or streamed through the
    // ring again when the stash would be too large)
    const auto store_b = [&](const Unit<IO, VEC> (&ku)[NU], int i) {
      const float ai = lane_f32(af, i);
      const float c1 = lane_f32(c1f, i);
      const float wh = lane_f32(whf, i);
      const float c1wl = lane_f32(c1wlf, i);
      GIO* drow = static_cast<GIO*>(p.dsrc.ptr[i]) + row * p.dsrc.ld[i];
#pragma unroll
      for (int k = 0; k < NU; ++k) {
        const int u = g.unit(k);
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] = ai * gr[k][e];  // gr is 0 past the row
        if (k >= K0 && u >= g.ub && u < g.nur) {
          float x[VEC];
          ku[k].get(x);
          if (u * VEC < g.c0) {
            // the one unit that straddles the window's first column: the staged query is 0
            // before it, so zeroing those source values leaves their columns alpha_i g alone
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              if (u * VEC + e < g.c0) x[e] = 0.f;
          }
          float qv[VEC];
          qst.get<VEC>(u - g.ub, qv);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            v[e] = fmaf(c1, fmaf(-wh, x[e], qv[e]), v[e]);
            v[e] = fmaf(-c1wl, x[e], v[e]);
            dqa[k >= K0 ? k - K0 : 0][e] = fmaf(c1, x[e], dqa[k >= K0 ? k - K0 : 0][e]);
          }
        }
        if constexpr (kRunStores) {
          // float32 gradients of 16-byte bf16 units: regroup the wave's 512 values so that
          // every store covers 1 KiB (the chunk exists for all lanes or none)
          const int cu = u - lane;  // the chunk's first unit
          if (cu < g.nur) {
            float lo[4], hi[4];
            run_halves(v, lane, lo, hi);
            float* cp = reinterpret_cast<float*>(drow) + static_cast<int64_t>(cu) * VEC;
            const int l2 = lane >> 1;
            if (cu + l2 < g.nur) {
              if (p.accumulate) {
                float old[4];
                load_f32<4>(cp + 4 * lane, old);
#pragma unroll
                for (int e = 0; e < 4; ++e) lo[e] += old[e];
              }
              store_unit<float, 4>(cp + 4 * lane, lo);
            }
            if (cu + 32 + l2 < g.nur) {
              if (p.accumulate) {
                float old[4];
                load_f32<4>(cp + 256 + 4 * lane, old);
#pragma unroll
                for (int e = 0; e < 4; ++e) hi[e] += old[e];
              }
              store_unit<float, 4>(cp + 256 + 4 * lane, hi);
            }
          }
        } else if (u < g.nur) {
          if (p.accumulate) {
            float old[VEC];
            load_grad<GIO, VEC>(drow + u * VEC, old);
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] += old[e];
          }
          store_grad<GIO, VEC>(drow + u * VEC, v);
        }
      }
    };
    if (stash != nullptr) {
      for (int i = 0; i < n; ++i) {
        Unit<IO, VEC> ku[NU];
#pragma unroll
        for (int k = 0; k < NU; ++k) {
          const int u = g.unit(k);
          if (k >= K0 && u >= g.ub && u < g.nur) ku[k] = stash[i * nkey + (u - g.ub)];
          else ku[k].zero();
        }
        store_b(ku, i);
      }
    } else {
#pragma unroll
      for (int b = 0; b < PF; ++b)
        if (b < n) load_stage<true>(ring[b], src_base(b), p.src.ld[b], g);
      for (int i0 = 0; i0 < n; i0 += PF + 1) {
#pragma unroll
        for (int b = 0; b <= PF; ++b) {
          const int i = i0 + b;
          if (i < n) {
            if (i + PF < n)
              load_stage<true>(ring[(b + PF) % (PF + 1)], src_base(i + PF), p.src.ld[i + PF], g);
            store_b(ring[b].t.u[0], i);
          }
        }
      }
    }
  }

  // ---- this workgroup's dq partial: one float64 row of the workspace
  double* out = block_dq + static_cast<int64_t>(blockIdx.x) * p.r;
  if constexpr (WPR == kWavesPerBlock) {
    // the four waves hold disjoint key columns
#pragma unroll
    for (int t = 0; t < TU; ++t) {
      const int u = g.unit(K0 + t);
      if (u >= g.ub && u < g.nur) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int col = u * VEC + e;
          if (col >= g.c0) out[col - g.c0] = static_cast<double>(dqa[t][e]);
        }
      }
    }
  } else {
    // every wave holds the same columns: sum them in wave order, one slot at a time
    __shared__ float dq_lds[kWavesPerBlock][kWave * VEC];
#pragma unroll
    for (int t = 0; t < TU; ++t) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) dq_lds[wib][lane * VEC + e] = dqa[t][e];
      __syncthreads();
      const int u = g.unit(K0 + t);
      if (wib == 0 && u >= g.ub && u < g.nur) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int col = u * VEC + e;
          if (col >= g.c0) {
            double sum = 0.0;
#pragma unroll
            for (int w = 0; w < kWavesPerBlock; ++w)
              sum += static_cast<double>(dq_lds[w][lane * VEC + e]);
            out[col - g.c0] = sum;
          }
        }
      }
      __syncthreads();
    }
  }
}

namespace {

int device_cus_bwd() {
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

// Largest key stash a workgroup takes (beyond it pass B reads the key units again from memory):
// small enough that several workgroups still share a CU's LDS.
constexpr size_t kStashMaxBytes = 32 * 1024;

// Bytes of the key stash of one workgroup: the key units of every source for each of its
// row groups.
template <typename IO, int VEC>
size_t stash_bytes(const BwdParams& p, int wpr) {
  const int nur = (p.d + VEC - 1) / VEC;
  const int nkey = nur - (p.d - p.r) / VEC;
  return static_cast<size_t>(kWavesPerBlock / wpr) * p.n * nkey * sizeof(Unit<IO, VEC>);
}

template <typename IO, typename GIO, int VEC, int NU, int TU, int WPR>
hipError_t launch_bwd_tile_t(const BwdParams& p, double* block_dq, int max_blocks, int* grid_out,
                             hipStream_t s) {
  auto kern = p.saved != nullptr ? k_backward_tile<IO, GIO, VEC, NU, TU, WPR, true>
                                 : k_backward_tile<IO, GIO, VEC, NU, TU, WPR, false>;
  BwdParams pk = p;
  pk.key_stash = stash_bytes<IO, VEC>(p, WPR) <= kStashMaxBytes ? 1 : 0;
  const int ub = (p.d - p.r) / VEC;
  const int rq = p.d - ub * VEC;
  const size_t lds = static_cast<size_t>((rq + 3) & ~3) * sizeof(float) +
                     (pk.key_stash ? stash_bytes<IO, VEC>(p, WPR) : 0);
  static thread_local size_t cached_lds = ~size_t(0);
  static thread_local int cached_per_cu = 0;
  static thread_local bool cached_saved = false;
  if (cached_lds != lds || cached_saved != (p.saved != nullptr)) {
    cached_saved = p.saved != nullptr;
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, kBlock, lds) != hipSuccess ||
        per < 1)
      per = 1;
    cached_per_cu = per;
    cached_lds = lds;
  }
  constexpr int kGroupsPerBlock = kWavesPerBlock / WPR;
  // float32 gradients write twice the bytes they read: with at most 2 workgroups (8 waves) per
  // CU, fewer write streams are open at once, which measured 2 % faster than the 3 that fit
  // (d = 4096, r = 1024, 10 sources); bf16 gradients measured 8 % slower so capped, and 1
  // workgroup per CU was 24-37 % slower for both.
  const int per_cu = std::is_same<GIO, float>::value && cached_per_cu > 2 ? 2 : cached_per_cu;
  int64_t blocks = static_cast<int64_t>(per_cu) * device_cus_bwd();
  const int64_t need = (p.T + kGroupsPerBlock - 1) / kGroupsPerBlock;
  if (blocks > need) blocks = need;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  *grid_out = static_cast<int>(blocks);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), lds, s, pk, block_dq);
  return hipGetLastError();
}

template <typename IO, typename GIO, int VEC, int NU, int WPR>
hipError_t launch_bwd_tile_tu(const BwdParams& p, double* block_dq, int max_blocks, int* grid,
                              hipStream_t s) {
  const int first_key_chunk = ((p.d - p.r) / VEC) / kWave;
  if constexpr (NU > 1) {
    if (first_key_chunk / WPR >= NU - 1)
      return launch_bwd_tile_t<IO, GIO, VEC, NU, 1, WPR>(p, block_dq, max_blocks, grid, s);
  }
  return launch_bwd_tile_t<IO, GIO, VEC, NU, NU, WPR>(p, block_dq, max_blocks, grid, s);
}

template <typename IO, typename GIO, int VEC>
hipError_t launch_bwd_tile_io(const BwdParams& p, double* block_dq, int max_blocks, int* grid,
                              hipStream_t s) {
  const int nur = (p.d + VEC - 1) / VEC;
  const int chunks = (nur + kWave - 1) / kWave;
  if (chunks <= 1) return launch_bwd_tile_tu<IO, GIO, VEC, 1, 1>(p, block_dq, max_blocks, grid, s);
  if (chunks <= 2) return launch_bwd_tile_tu<IO, GIO, VEC, 2, 1>(p, block_dq, max_blocks, grid, s);
  if (chunks <= 4) return launch_bwd_tile_tu<IO, GIO, VEC, 4, 1>(p, block_dq, max_blocks, grid, s);
  if (chunks <= 8) return launch_bwd_tile_tu<IO, GIO, VEC, 2, 4>(p, block_dq, max_blocks, grid, s);
  if (chunks <= 16) return launch_bwd_tile_tu<IO, GIO, VEC, 4, 4>(p, block_dq, max_blocks, grid, s);
  if (chunks <= 32) return launch_bwd_tile_tu<IO, GIO, VEC, 8, 4>(p, block_dq, max_blocks, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

int backward_tile_max_chunks() { return 32; }

hipError_t launch_backward_tile(const BwdParams& p, int io_bf16, int grad_bf16, double* block_dq,
                                int max_blocks, int* grid, hipStream_t s) {
  if (io_bf16)
    return grad_bf16 ? launch_bwd_tile_io<bf16_bits, bf16_bits, 8>(p, block_dq, max_blocks, grid, s)
                     : launch_bwd_tile_io<bf16_bits, float, 8>(p, block_dq, max_blocks, grid, s);
  return grad_bf16 ? launch_bwd_tile_io<float, bf16_bits, 4>(p, block_dq, max_blocks, grid, s)
                   : launch_bwd_tile_io<float, float, 4>(p, block_dq, max_blocks, grid, s);
}

}  // namespace lrar
