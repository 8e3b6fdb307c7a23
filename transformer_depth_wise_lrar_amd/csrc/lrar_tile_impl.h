// The depth-mix read on register-resident row tiles (LR-AttnRes paper §3.1/§3.3; the Phase-2
// merge of §3.4 and of the AttnRes technical-report summary, "Method").
//
// Layout. Each 64-lane wavefront owns tiles of R token rows. Lane l holds units l, l + 64, ...
// (NU of them, 16 bytes each on the vector path) of every row of the tile, so the tile's rows
// and their float32 accumulators live in registers for the whole read. The wave visits the
// sources in order and keeps PF sources in flight ahead of the one it folds in. Tiles are
// dealt to the waves in bands, so at any moment the resident waves read one contiguous window
// of rows of the same few sources: long sequential HBM streams instead of one short stream per
// (row, source).
//
// Modes.
//   kTileOnline   one pass: every source byte is read once. Each source's score is computed
//                 from the tile already in flight, and an online softmax folds the rows in.
//                 The accumulator is rescaled only when a score passes the running reference
//                 by more than kLazyRescale, so the weights stay <= e^8 and each rescale
//                 shrinks every earlier rounding error together with the terms it scales.
//   kTileTwoPass  pass 1 reads only the key slices and scores them; the softmax is taken once
//                 per row in float64; pass 2 streams the full rows with the fixed float32
//                 weights. The key bytes are read twice (normally from L2 the second time).
//   kTileMerge    kTileOnline started from Phase-1 statistics (m, l, acc): lrar_merge.
//   kTileFullRms  kTileOnline with the full-width-RMS control score (LR-AttnRes paper §4.4,
//                 Eq. 13): the key columns are divided by the RMS of the whole row, which is
//                 summed from the row units already in registers.
//   kTileKeys     kTileOnline with a separate r-wide key per source (the read side of the
//                 paper's Projected LR-AttnRes, App. C.1-C.2): the spread key pieces are
//                 loaded from the key rows, the values from the source rows.
//   kTileMergeAcc kTileMerge whose one extra source is the updated partial sum b' = b + o
//                 (§3.3 "Partial-block routing"): the tiles of b and of the new output o are
//                 added in registers, rounded to the element type, written out as b', and
//                 scored and folded in from the registers (the key from the row units).
//
// Key arithmetic (float64: bf16/fp32 x fp32 products are exact in float64).
//   KS = 0   the key is taken from the row units in registers: only the last TU unit slots of
//            a lane can hold key columns, and the site query is staged once per workgroup in
//            LDS. Used for wide keys, where the key fills whole slots.
//   KS > 0   "spread" key for r <= 64 KS: each lane also loads KS consecutive key elements
//            (an ordinary cached load issued just before the row's streaming load, so the row
//            load finds those lines in L2) and the products use every lane instead of the few
//            that hold the key's units. The query's matching KS values stay in registers.
//
// This header holds the kernel template and its launchers; each mode is instantiated in a
// translation unit of its own (lrar_tile_online.hip, lrar_tile_twopass.hip, lrar_tile_merge.hip).
#pragma once

#include "lrar_device.h"
#include "lrar_launch.h"
#include "lrar_tile.h"

namespace lrar {

// Sources in flight ahead of the one being folded for reads of many sources (the three-deep
// ring; the launchers below say when it is used).
constexpr int kDeepPrefetch = 3;
// Reads through the shallower rings keep their one-wave rows in lockstep from this many sources.
constexpr int kLockMinSources = 8;

template <typename IO, int VEC, int NU, int TU, int KS, bool ROWRED, int R, int PF, int WPR,
          int MODE, typename ACC, bool KA>
__global__ __launch_bounds__(kBlock) void k_read_tile(ReadParams p, KeyTable<MODE> keys) {
  static_assert(kWavesPerBlock % WPR == 0, "a workgroup holds whole row groups");
  extern __shared__ __attribute__((aligned(16))) float q_lds[];
  // Partial key sums of the waves that share a row (two slots, alternating by source).
  __shared__ double xch[2][kWavesPerBlock][2 * R];
  const int lane = threadIdx.x & (kWave - 1);
  const int wib = threadIdx.x / kWave;  // wave in block
  const int64_t group =
      p.tile_begin + (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wib) / WPR;
  const int n = p.n;
  TileGeom g;
  g.lane = lane;
  g.w = wib % WPR;
  g.wpr = WPR;
  g.nur = (p.d + VEC - 1) / VEC;
  g.c0 = p.d - p.r;
  g.ub = g.c0 / VEC;
  g.r = p.r;
  // The query: spread over the lanes (KS > 0), or staged in LDS from the first key unit's
  // column (KS = 0; the columns of that unit that precede the key hold zero).
  QStageD qst;
  qst.base = reinterpret_cast<double*>(q_lds);
  qst.nv = g.nur - g.ub;
  SpreadQ<KS> qs[ks_slots(KS)];
#pragma unroll
  for (int e = 0; e < ks_slots(KS); ++e) qs[e] = 0;
  if constexpr (KS > 0) {
    if (n > 0) {
#pragma unroll
      for (int e = 0; e < KS; ++e) {
        const int idx = lane * KS + e;
        if (idx < p.r) qs[e] = static_cast<SpreadQ<KS>>(p.q[idx]);
      }
    }
  } else {
    if (n > 0) qst.fill<VEC>(p.q, g.ub, g.c0, threadIdx.x, kBlock);
    __syncthreads();
  }
  // Spread key pieces sit in lanes [0, gp) (gp: a power of two).
  int gp = 1;
  if constexpr (KS > 0) {
    const int used = (p.r + KS - 1) / KS;
    while (gp < used) gp <<= 1;
  }

  // Tiles are dealt out in bands: in its k-th step row group w takes tile
  // tile_begin + w + k * ngroups, so the resident waves together read one contiguous window of
  // rows of every source at a time. (All waves of a group see the same tiles, so they meet the
  // same barriers.) ntiles is the end of this launch's tiles.
  const int64_t ngroups = static_cast<int64_t>(gridDim.x) * kWavesPerBlock / WPR;
  const int64_t ntiles = p.tile_end;
  int parity = 0;
  const auto src_base = [&](int i) { return static_cast<const IO*>(p.src.ptr[i]); };
  // The ring issues one stage load per item, also for the items past the last source: those
  // load over an empty span (no memory read), so every item leaves the same loads in flight
  // and a wait for a stage is a wait for that stage only.
  const auto clamp_src = [&](int i) { return i < n ? i : n - 1; };
  const IO* const kNoKeys = nullptr;  // the key base of a read whose keys are in its rows
  constexpr bool kSep = MODE == kTileKeys;
  const auto key_base = [&](int i) -> const IO* {
    if constexpr (kSep) return static_cast<const IO*>(keys.ptr[i]);
    else return nullptr;
  };
  const auto key_ld = [&](int i) -> int64_t {
    if constexpr (kSep) return keys.ld[i];
    else return 0;
  };
  // 1 / width of the mean of squares in the key's RMS: the key, or the whole row for the
  // control.
  const double rinv_nrm = 1.0 / static_cast<double>(MODE == kTileFullRms ? p.d : p.r);
  constexpr bool kMerge = MODE == kTileMerge || MODE == kTileMergeAcc;
  const auto set_tile = [&](TileGeom& t, int64_t tile) {
    t = g;
    t.r0 = tile * R;
    t.nrow = (p.T - t.r0) < R ? static_cast<int>(p.T - t.r0) : R;
  };

  float acc[R][NU][VEC];
  double zk[R];  // lane i: score (two-pass: weight) of source i in row j
  double rk[R];  // lane i: 1 / rho of source i in row j (kept only for the saved statistics)
  const bool keep_scores = p.alpha != nullptr || p.saved != nullptr;
  // Online-softmax state of row j, held in lane j: reference mref, running sum lsum of
  // e^{z - mref}, running maximum mtop. One vector exp then serves all R rows.
  double mref = -INFINITY, lsum = 0.0, mtop = -INFINITY;

  // bf16 Phase-1 accumulators of a single-source merge (with or without the fused update) are
  // loaded a tile ahead, raw (16 registers a row at four units per lane), and decoded when
  // their tile starts.
  constexpr bool kAccPre = (MODE == kTileMerge || MODE == kTileMergeAcc) &&
                           std::is_same<ACC, bf16_bits>::value && VEC == 8;
  Unit<bf16_bits, 8> apre[kAccPre ? R : 1][kAccPre ? NU : 1];
  const auto load_acc_ahead = [&](const TileGeom& t) {
    if constexpr (kAccPre) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const bf16_bits* prow =
            static_cast<const bf16_bits*>(p.acc) + (t.r0 + j) * p.acc_ld;
#pragma unroll
        for (int k = 0; k < NU; ++k) {
          const int u = t.unit(k);
          if (j < t.nrow && u < t.nur) apre[j][k].load(prow + u * VEC);
          else apre[j][k].zero();
        }
      }
    }
  };

  // Starts a tile: clears the accumulators, or loads the Phase-1 statistics for a merge
  // (ahead: the accumulators were loaded by load_acc_ahead).
  const auto begin_tile = [&](const TileGeom& t, bool ahead = false) {
    mref = -INFINITY;
    lsum = 0.0;
    mtop = -INFINITY;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      zk[j] = 0.0;
      rk[j] = 0.0;
#pragma unroll
      for (int k = 0; k < NU; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][k][e] = 0.f;
    }
    if constexpr (kMerge) {
      if (lane < t.nrow) {
        mref = static_cast<double>(p.m_in[t.r0 + lane]);
        mtop = mref;
        lsum = static_cast<double>(p.l_in[t.r0 + lane]);
      }
      bool decoded = false;
      if constexpr (kAccPre) {
        if (ahead) {
#pragma unroll
          for (int j = 0; j < R; ++j)
#pragma unroll
            for (int k = 0; k < NU; ++k) apre[j][k].get(acc[j][k]);
          decoded = true;
        }
      }
      if (!decoded) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          if (j < t.nrow) {
            const ACC* prow = static_cast<const ACC*>(p.acc) + (t.r0 + j) * p.acc_ld;
#pragma unroll
            for (int k = 0; k < NU; ++k) {
              const int u = t.unit(k);
              if (u < t.nur) load_acc<ACC, VEC>(prow + u * VEC, acc[j][k]);
            }
          }
        }
      }
    }
  };

  // Writes the saved statistics of a tile's rows: z_i and 1 / rho_i of source i in lane i.
  const auto save_scores = [&](const TileGeom& t) {
    if (p.saved != nullptr && t.w == 0 && lane < n) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if (j < t.nrow) {
          double* srow = p.saved + (t.r0 + j) * p.saved_ld;
          srow[lane] = zk[j];
          srow[n + lane] = rk[j];
        }
      }
    }
  };

  // Normalises and writes a tile's h (and the weights / merged statistics).
  const auto finish_tile = [&](const TileGeom& t) {
    if constexpr (MODE != kTileTwoPass) save_scores(t);
    const float inv = static_cast<float>(1.0 / lsum);  // lane j: row j (online and merge)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j < t.nrow) {
        const int64_t row = t.r0 + j;
        float scale = 1.f;
        if constexpr (MODE != kTileTwoPass) scale = lane_f32(inv, j);
        IO* orow = static_cast<IO*>(p.out) + row * p.out_ld;
#pragma unroll
        for (int k = 0; k < NU; ++k) {
          const int u = t.unit(k);
          if (u < t.nur) {
            float y[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) y[e] = acc[j][k][e] * scale;
            store_unit<IO, VEC>(orow + u * VEC, y);
          }
        }
        if (p.alpha != nullptr && t.w == 0) {
          double a = zk[j];
          if constexpr (MODE != kTileTwoPass)
            a = exp(zk[j] - lane_f64(mref, j)) / lane_f64(lsum, j);
          if (lane < n) p.alpha[row * p.alpha_ld + lane] = static_cast<float>(a);
        }
      }
    }
    if constexpr (kMerge) {
      if (lane < t.nrow && t.w == 0) {
        const float mf = static_cast<float>(mtop);
        if (p.m_out) p.m_out[t.r0 + lane] = mf;
        if (p.l_out)
          p.l_out[t.r0 + lane] = static_cast<float>(lsum * exp(mref - static_cast<double>(mf)));
      }
    }
  };

  // Scores of one stage's rows; lane j returns row j's.
  const auto stage_scores = [&](const Stage<IO, VEC, NU, R, KS>& st,
                                const TileGeom& t) -> Score {
    double red[2 * R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if constexpr (KS > 0)
        key_partial_spread<IO, KS>(st.kp[j], qs, red[2 * j], red[2 * j + 1]);
      else if constexpr (MODE == kTileFullRms)
        row_partial_full<KA>(st.t.u[j], qst, t, red[2 * j], red[2 * j + 1]);
      else
        key_partial_units<TU, KA>(st.t.u[j], qst, t, red[2 * j], red[2 * j + 1]);
    }
    if constexpr (KS > 0 && ROWRED && R <= 2) {
      // the spread key sits in lanes 0..31 of every wave of the row
      return row_scores_rowlocal<R>(red, lane, rinv_nrm, p.eps);
    } else if constexpr (KS > 0) {
      lanes_sums_dpp(red, gp);  // every wave of the row holds the whole spread key
    } else if constexpr (WPR == 1 && R <= 2) {
      return row_scores_wave<R>(red, lane, rinv_nrm, p.eps);
    } else if constexpr (R <= 2) {
      // the row's waves each reduce their own sums, then add all waves' in a fixed order (so
      // every wave of the row gets bitwise the same score)
      const double x = wave_sums_transposed<R>(red, lane);
      if (lane < 2 * R) xch[parity][wib][transposed_index<R>(lane)] = x;
      __syncthreads();
      const int base = wib - t.w;
#pragma unroll
      for (int j = 0; j < 2 * R; ++j) {
        double v = xch[parity][base][j];
#pragma unroll
        for (int o = 1; o < WPR; ++o) v += xch[parity][base + o][j];
        red[j] = v;
      }
      parity ^= 1;
    } else {
      wave_sums_dpp(red);
      if constexpr (WPR > 1) {
        // add the partial sums of the row's other waves, in a fixed order (so every wave of
        // the row gets bitwise the same score)
        double mine = red[0];
#pragma unroll
        for (int j = 1; j < 2 * R; ++j)
          if (lane == j) mine = red[j];
        if (lane < 2 * R) xch[parity][wib][lane] = mine;
        __syncthreads();
        const int base = wib - t.w;
#pragma unroll
        for (int j = 0; j < 2 * R; ++j) {
          double v = xch[parity][base][j];
#pragma unroll
          for (int o = 1; o < WPR; ++o) v += xch[parity][base + o][j];
          red[j] = v;
        }
        parity ^= 1;
      }
    }
    return row_scores_to_lanes<R>(red, lane, rinv_nrm, p.eps);
  };

  // Keeps the scores (and reciprocal RMS) of source i for the weights and saved statistics.
  const auto keep_source = [&](const Score& sc, int i) {
    if (keep_scores) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const double zj = lane_f64(sc.z, j);
        if (lane == i) zk[j] = zj;
      }
    }
    if (p.saved != nullptr) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const double rj = lane_f64(sc.rinv, j);
        if (lane == i) rk[j] = rj;
      }
    }
  };

  // Scores source i's stage and folds its rows into the online-softmax accumulators.
  const auto fold_source = [&](const Stage<IO, VEC, NU, R, KS>& st, const TileGeom& t, int i) {
    const Score sc = stage_scores(st, t);  // lane j: row j
    const double z = sc.z;
    keep_source(sc, i);
    if constexpr (kMerge) mtop = fmax(mtop, z);  // only the merge reports the maximum
    // Rescale a row only when its score passes the reference by more than kLazyRescale
    // (always on its first source, whose reference is -inf).
    const bool grow = !(z <= mref + kLazyRescale);
    if (__builtin_amdgcn_ballot_w64(grow && lane < R) != 0) {
      const double sc = grow ? exp_weight(mref - z) : 1.0;
      mref = grow ? z : mref;
      lsum *= sc;
      const float scf = static_cast<float>(sc);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float sj = lane_f32(scf, j);
#pragma unroll
        for (int k = 0; k < NU; ++k)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[j][k][e] *= sj;
      }
    }
    const double ez = exp_weight(z - mref);
    lsum += ez;
    const float ef = static_cast<float>(ez);
#pragma unroll
    for (int j = 0; j < R; ++j) fma_row(acc[j], lane_f32(ef, j), st.t.u[j]);
  };

  // Ring of PF + 1 stages: the item PF ahead is loading while the current one is folded in.
  // Loops over the ring are unrolled by PF + 1 so that every stage index is a constant and no
  // stage is copied (a copy would wait for its loads). Exact loads (see load_stage_exact) for
  // keys read from the row units and for the one- and two-deep rings; spread keys through the
  // three-deep ring, and the drained one-ahead reads of short pieces (spread_drained, the only
  // one-deep ring over 4 slots with such pieces), keep the branchy loads.
  constexpr bool kDrained = MODE == kTileOnline && KS > 0 && KS < 16 && NU == 4 && PF == 1;
  constexpr bool kExact = !kDrained && (KS == 0 || PF < 3);
  Stage<IO, VEC, NU, R, KS> ring[PF + 1];

  if constexpr (MODE == kTileTwoPass) {
    for (int64_t tile = group; tile < ntiles; tile += ngroups) {
      TileGeom t;
      set_tile(t, tile);
      begin_tile(t);
      // pass 1: scores from the key slices
#pragma unroll
      for (int b = 0; b < PF; ++b) {
        const int ia = clamp_src(b);
        load_stage_as<true, false, kExact>(ring[b], src_base(ia), p.src.ld[ia], t, kNoKeys, 0,
                                           b < n);
        if constexpr (kExact) __builtin_amdgcn_sched_barrier(0);  // stages issued in ring order
      }
      for (int i0 = 0; i0 < n; i0 += PF + 1) {
#pragma unroll
        for (int b = 0; b <= PF; ++b) {
          const int i = i0 + b;
          const int ia = clamp_src(i + PF);
          load_stage_as<true, false, kExact>(ring[(b + PF) % (PF + 1)], src_base(ia),
                                             p.src.ld[ia], t, kNoKeys, 0, i + PF < n);
          if (i < n) {
            const Score sc = stage_scores(ring[b], t);
#pragma unroll
            for (int j = 0; j < R; ++j) {
              const double zj = lane_f64(sc.z, j);
              if (lane == i) zk[j] = zj;
            }
            if (p.saved != nullptr) {
#pragma unroll
              for (int j = 0; j < R; ++j) {
                const double rj = lane_f64(sc.rinv, j);
                if (lane == i) rk[j] = rj;
              }
            }
          }
        }
      }
      save_scores(t);
      // softmax once per row (lanes = sources)
      float w[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const double m = wave_max_dpp(lane < n ? zk[j] : -INFINITY);
        const double e = lane < n ? exp(zk[j] - m) : 0.0;
        const double L = wave_sum_dpp(e);
        zk[j] = e / L;
        w[j] = static_cast<float>(zk[j]);
      }
      // pass 2: the values (the row units only)
      Stage<IO, VEC, NU, R, 0> vring[PF + 1];
#pragma unroll
      for (int b = 0; b < PF; ++b) {
        const int ia = clamp_src(b);
        load_stage_as<false, false, true>(vring[b], src_base(ia), p.src.ld[ia], t, kNoKeys, 0,
                                          b < n);
        __builtin_amdgcn_sched_barrier(0);  // stages issued in ring order
      }
      for (int i0 = 0; i0 < n; i0 += PF + 1) {
#pragma unroll
        for (int b = 0; b <= PF; ++b) {
          const int i = i0 + b;
          const int ia = clamp_src(i + PF);
          load_stage_as<false, false, true>(vring[(b + PF) % (PF + 1)], src_base(ia),
                                            p.src.ld[ia], t, kNoKeys, 0, i + PF < n);
          if (i < n) {
#pragma unroll
            for (int j = 0; j < R; ++j) fma_row(acc[j], lane_f32(w[j], i), vring[b].t.u[j]);
          }
        }
      }
      finish_tile(t);
    }
  } else if constexpr (MODE == kTileMergeAcc) {
    // one extra source, the updated partial sum b' = b + o, formed in registers
    static_assert(KS == 0, "the key of b' is taken from the row units");
    const IO* bprev = static_cast<const IO*>(p.b_prev);
    IO* bout = static_cast<IO*>(p.b_out);
    if (group < ntiles) {
      TileGeom t;
      set_tile(t, group);
      load_acc_ahead(t);
    }
    // One-wave rows meet at a workgroup barrier once per tile, as the reads do (d = 1024 and
    // 2048: +1.6 to +3 % in four of six dtype and key cases, level in the others; the plain
    // merges measured level). It is taken only in the steps where every row group of the
    // workgroup has a tile, a condition the same for all of its waves.
    const int64_t last_group =
        p.tile_begin +
        (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + kWavesPerBlock - 1) / WPR;
    for (int64_t tile = group; tile < ntiles; tile += ngroups) {
      TileGeom t;
      set_tile(t, tile);
      if (WPR == 1 && (tile - group) + last_group < ntiles) __syncthreads();
      begin_tile(t, true);
      if (tile + ngroups < ntiles) {
        TileGeom tn;
        set_tile(tn, tile + ngroups);
        load_acc_ahead(tn);
      }
      Stage<IO, VEC, NU, R, KS>& st = ring[0];
      load_stage_branchy<false>(st, src_base(0), p.src.ld[0], t);
      if (bprev != nullptr) {
        Tile<IO, VEC, NU, R> bt;
#pragma unroll
        for (int j = 0; j < R; ++j) {
#pragma unroll
          for (int k = 0; k < NU; ++k) {
            const int u = t.unit(k);
            if (j < t.nrow && u < t.nur) bt.u[j][k].load(bprev + (t.r0 + j) * p.b_prev_ld + u * VEC);
            else bt.u[j][k].zero();
          }
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
#pragma unroll
          for (int k = 0; k < NU; ++k) {
            float x[VEC], y[VEC];
            st.t.u[j][k].get(x);
            bt.u[j][k].get(y);
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] += y[e];
            st.t.u[j][k].set(x);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int k = 0; k < NU; ++k) {
          const int u = t.unit(k);
          if (j < t.nrow && u < t.nur) st.t.u[j][k].store(bout + (t.r0 + j) * p.b_out_ld + u * VEC);
        }
      }
      fold_source(st, t, 0);
      finish_tile(t);
    }
  } else if (n == 0) {
    // a merge with no further sources: normalise the statistics
    for (int64_t tile = group; tile < ntiles; tile += ngroups) {
      TileGeom t;
      set_tile(t, tile);
      begin_tile(t);
      finish_tile(t);
    }
  } else if (n == 1) {
    // One source per tile (a merge with the partial sum, the embedding-only read): the tiles
    // alternate between two stages, so the next tile's rows load while this tile is scored
    // and folded in.
    static_assert(PF >= 1, "two stages");
    int64_t tile = group;
    TileGeom t0, t1;
    if (tile < ntiles) {
      set_tile(t0, tile);
      load_stage_branchy<false, kSep>(ring[0], src_base(0), p.src.ld[0], t0, key_base(0),
                                      key_ld(0));
      load_acc_ahead(t0);
    }
    for (; tile < ntiles; tile += 2 * ngroups) {
      const bool more = tile + ngroups < ntiles;
      if (more) {
        set_tile(t1, tile + ngroups);
        load_stage_branchy<false, kSep>(ring[1], src_base(0), p.src.ld[0], t1, key_base(0),
                                        key_ld(0));
      }
      begin_tile(t0, true);
      if (more) load_acc_ahead(t1);
      fold_source(ring[0], t0, 0);
      finish_tile(t0);
      if (more) {
        const bool next = tile + 2 * ngroups < ntiles;
        if (next) {
          set_tile(t0, tile + 2 * ngroups);
          load_stage_branchy<false, kSep>(ring[0], src_base(0), p.src.ld[0], t0, key_base(0),
                                          key_ld(0));
        }
        begin_tile(t1, true);
        if (next) load_acc_ahead(t0);
        fold_source(ring[1], t1, 0);
        finish_tile(t1);
      }
    }
  } else {
    // Rows held by one wave meet at a workgroup barrier, so the workgroup's waves stream the
    // same sources together, which HBM serves best: once per ring cycle through the three-deep
    // ring (d = 1024, sites of 20..49 sources: +2.7 to +3.6 %; the separate-key read of 49
    // sources: +3 %; per source or per tile gained less), once per tile through the shallower
    // rings of reads of 8 or more sources (d = 2048: +0.6 to +2.5 %; d = 1024, 9 and 13
    // sources: +2 %; 5 sources lost 1 %, and a barrier per source or per ring cycle lost up to
    // 1.5 % there). A barrier is taken only in the steps where every row group of the workgroup
    // has a tile, a condition that is the same for all of its waves (as n is), so they all meet
    // the same barriers.
    constexpr bool kDeep = PF == kDeepPrefetch;
    const bool lock_reads = WPR == 1 && (kDeep || n >= kLockMinSources);
    const int64_t last_group =
        p.tile_begin +
        (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + kWavesPerBlock - 1) / WPR;
    for (int64_t tile = group; tile < ntiles; tile += ngroups) {
      TileGeom t;
      set_tile(t, tile);
      begin_tile(t);
      const bool lockstep = lock_reads && (tile - group) + last_group < ntiles;
      if (!kDeep && lockstep) __syncthreads();
      // Rows that span the workgroup's four waves with a spread key exchange no key sums, so
      // nothing else keeps their waves together: they meet once per tile (+1 % at d = 7168,
      // +3 % at d = 4096, r = 64; once per source gained less). All four waves hold the same
      // tiles.
      if constexpr (WPR == kWavesPerBlock && KS > 0) __syncthreads();
#pragma unroll
      for (int b = 0; b < PF; ++b) {
        const int ia = clamp_src(b);
        load_stage_as<false, kSep, kExact>(ring[b], src_base(ia), p.src.ld[ia], t, key_base(ia),
                                           key_ld(ia), b < n);
        // stages issued in ring order, so a wait for the oldest is a wait for it alone
        if constexpr (kExact) __builtin_amdgcn_sched_barrier(0);
      }
      for (int i0 = 0; i0 < n; i0 += PF + 1) {
#pragma unroll
        for (int b = 0; b <= PF; ++b) {
          const int i = i0 + b;
          const int ia = clamp_src(i + PF);
          load_stage_as<false, kSep, kExact>(ring[(b + PF) % (PF + 1)], src_base(ia),
                                             p.src.ld[ia], t, key_base(ia), key_ld(ia),
                                             i + PF < n);
          if (i < n) {
            if (kDeep && b == 0 && lockstep) __syncthreads();
            fold_source(ring[b], t, i);
          }
        }
      }
      finish_tile(t);
    }
  }
}

// ---- launchers -----------------------------------------------------------------------------------

namespace {

int device_cus() {
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

// Rows per tile and prefetch depth for NU units per lane: the tile's accumulators and its
// PF + 1 stages must leave room for several waves per SIMD, and the loads in flight
// (waves x PF tiles) must cover the HBM latency.
constexpr int tile_rows(int nu) { return nu <= 1 ? 4 : (nu <= 2 ? 2 : 1); }
constexpr int tile_prefetch(int nu) { return nu <= 4 ? 2 : 1; }
// Keys read from the row units that reach every unit slot of a 4-slot row (r = d at d = 2048;
// r >= 1792 at d = 7168) keep one source in flight instead of two: their float64 scoring keeps
// the vector unit busy, and the smaller ring measured 2-3 % faster there (r = d = 2048,
// r = 1792 at d = 7168) but 4 % slower for a key in the last slot alone (r = 512, d = 2048).
constexpr bool key_fills_slots(int ks, int tu, int nu) { return ks == 0 && nu == 4 && tu == nu; }

// Reads of many sources (DEEP) keep one more source in flight: three sources ahead measured 8 %
// (d = 1024, 49 sources) and 5 % (d = 2048, 9 sources) faster than two for spread keys, in
// both variants, at the price of a third wave per SIMD. One-pass reads of short pieces on
// 4-slot rows now take the drained one-ahead ring instead (spread_drained, below), which beat
// three ahead. Reads of few sources, and slice keys taken from the row units (whose float64
// scoring already keeps the vector unit busy), keep the shallower ring. The full-width-RMS
// control, which scores every column of the row in float64, keeps one source ahead: 7 % (13
// sources) and 3 % (25) faster than three ahead, level at 49 (d = 1024).
constexpr int kDeepMinSources = 8;
// Reads with the key in the row's last columns, spread over the lanes, and two units per lane
// (d <= 1024 bf16) take the three-deep ring only from 20 sources: below that the two-deep ring
// with exact waits measured 4-7 % faster (9 and 13 sources), above it 2-5 % slower (25 to 49).
// The separate-key read keeps the lower threshold (its r = 64 keys measured 6 % slower at 13
// sources with the two-deep ring).
constexpr int kDeepMinSourcesNarrow = 20;
constexpr int deep_min_sources(int nu, int mode) {
  return nu <= 2 && mode != kTileKeys ? kDeepMinSourcesNarrow : kDeepMinSources;
}

// How much a read keeps in flight matters beyond covering the load latency: a plain stream of
// the same traffic (10 sources, d = 2048) ran 0.81 of peak with one source in flight per wave
// and short launches, 0.75 with three. HBM serves fewer, better-ordered requests faster.
//
// Reads of 16-element spread key pieces (r = 257..512) keep one source in flight, loaded exactly:
// their per-source float64 scoring covers the load latency (r = 512, d = 2048, 10 sources: 6 %
// faster than three ahead, 4 % faster than two; 9 % faster than the same ring with branchy
// loads). Pieces of 4 and 8 elements measured 4-5 % slower that way.
constexpr bool spread_single(int ks, int mode) { return ks >= 16 && mode == kTileOnline; }
// One-pass reads of many sources whose short pieces (up to 8 elements) sit on rows of 4 unit
// slots (d = 1536..2048 per wave, and the 4-wave rows up to d = 8192) fetch one source ahead
// with branchy loads, whose wait for the oldest stage is a
// wait for every load in flight: each source is drained before it is folded, the pattern of the
// plain stream above. Against the three-deep ring: 1-2 % faster at d = 2048 (r = 16, 64; 9 and 10
// sources) and 3 % at d = 7168 (r = 64, 9 sources). Rows of 1-2 slots (d <= 1024) measured
// 2-6 % slower that way and keep their rings.
constexpr bool spread_drained(int ks, int nu, int mode, bool deep) {
  return mode == kTileOnline && deep && ks > 0 && ks < 16 && nu == 4;
}

// Tiles per row group in one launch of a one-pass read. Over a long launch the waves drift
// apart, the window of rows they read together widens, and HBM serves it more slowly. Spread-key
// reads: at 64 tiles per group they measured 4-7 % slower than cut into launches of 16 tiles per
// group (d = 1024 to 7168, 9 sources), and 8 tiles per group measured 1-2 % faster again (d =
// 2048, r = 16 and 64; d = 7168, r = 64); the drained reads above take 4 (as did the plain
// stream) where several waves share a row, and 8 for one-wave rows, which the lockstep and the
// 8-wave cap keep together (+2 % at d = 2048, r = 16 and 64; 4 there before the lockstep; the
// four-wave rows measured 2 % slower at 8). Keys read from the row units of one wave (rows of
// up to 4 chunks): 8 tiles per group measured 4 % faster than one launch (r = d = 2048) and 3 %
// faster than 4; where several waves share a row (d = 7168) such cuts measured 3-7 % slower, as
// did the two-pass read and the merges (2-10 % at 12 tiles per group), so those run as one
// launch.
constexpr int64_t max_tiles_per_group(bool drained, int wpr) {
  return drained && wpr > 1 ? 4 : 8;
}
constexpr bool cut_into_launches(int mode, int ks, int wpr) {
  return (ks > 0 && (mode == kTileOnline || mode == kTileKeys)) ||
         (ks == 0 && mode == kTileOnline && wpr == 1);
}

template <typename IO, int VEC, int NU, int TU, int KS, bool ROWRED, int WPR, int MODE,
          typename ACC, bool DEEP = false, bool KA = false>
hipError_t launch_tile_t(const ReadParams& p, const KeyTable<MODE>& kt, hipStream_t s) {
  constexpr int R = tile_rows(NU);
  constexpr bool kDrained = spread_drained(KS, NU, MODE, DEEP);
  constexpr int PF = MODE == kTileFullRms || spread_single(KS, MODE) ||
                             key_fills_slots(KS, TU, NU) || kDrained
                         ? 1
                         : (DEEP ? kDeepPrefetch : tile_prefetch(NU));
  auto kern = k_read_tile<IO, VEC, NU, TU, KS, ROWRED, R, PF, WPR, MODE, ACC, KA>;
  const int ub = (p.d - p.r) / VEC;
  const int nur = (p.d + VEC - 1) / VEC;
  const size_t lds = KS > 0 ? 0 : static_cast<size_t>(nur - ub) * VEC * sizeof(double);
  // Workgroups per CU for this instantiation and LDS size (cached: the query is not free).
  static thread_local size_t cached_lds = ~size_t(0);
  static thread_local int cached_per_cu = 0;
  if (cached_lds != lds) {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, kBlock, lds) != hipSuccess ||
        per < 1)
      per = 1;
    cached_per_cu = per;
    cached_lds = lds;
  }
  // The drained one-ahead reads of one-wave rows run two workgroups (8 waves) per CU, as their
  // same-traffic stream runs fastest: +1 % at d = 2048 (r = 16, 64; 9 and 10 sources) against
  // the 3 that fit; the four-wave rows of that ring measured 2.6 % slower so capped.
  const int per_cu = kDrained && WPR == 1 && cached_per_cu > 2 ? 2 : cached_per_cu;
  // As many row groups as fit at once, trimmed so that no group gets more tiles than needed:
  // each launch runs in one round and the groups' tile counts differ by at most one. The reads
  // of cut_into_launches are cut into launches of at most max_tiles_per_group tiles per group,
  // every launch but the last giving each resident group the same count; any other read is one
  // launch.
  const int64_t resident = static_cast<int64_t>(per_cu) * device_cus() * kWavesPerBlock / WPR;
  const int64_t tiles = (p.T + R - 1) / R;
  const int64_t per_group_all = (tiles + resident - 1) / resident;
  const int64_t launches =
      cut_into_launches(MODE, KS, WPR)
          ? (per_group_all + max_tiles_per_group(kDrained, WPR) - 1) /
                max_tiles_per_group(kDrained, WPR)
          : 1;
  const int64_t per_launch = ((per_group_all + launches - 1) / launches) * resident;
  constexpr int kGroupsPerBlock = kWavesPerBlock / WPR;
  ReadParams pc = p;
  for (int64_t t0 = 0; t0 < tiles; t0 += per_launch) {
    const int64_t nt = tiles - t0 < per_launch ? tiles - t0 : per_launch;
    const int64_t per_group = (nt + resident - 1) / resident;
    const int64_t groups = (nt + per_group - 1) / per_group;
    const int64_t blocks = (groups + kGroupsPerBlock - 1) / kGroupsPerBlock;
    pc.tile_begin = t0;
    pc.tile_end = t0 + nt;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), lds, s, pc, kt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// A spread-key launch, with the deeper ring when it pays (see kDeepPrefetch).
template <typename IO, int VEC, int NU, int KS, bool ROWRED, int WPR, int MODE, typename ACC>
hipError_t launch_tile_spread(const ReadParams& p, const KeyTable<MODE>& kt, hipStream_t s) {
  if constexpr ((MODE == kTileOnline || MODE == kTileKeys || MODE == kTileTwoPass) && NU >= 2 &&
                NU <= 4 && !spread_single(KS, MODE)) {
    if (p.n >= deep_min_sources(NU, MODE))
      return launch_tile_t<IO, VEC, NU, 1, KS, ROWRED, WPR, MODE, ACC, true>(p, kt, s);
  }
  return launch_tile_t<IO, VEC, NU, 1, KS, ROWRED, WPR, MODE, ACC>(p, kt, s);
}

// A read with the key in the row units (KS = 0). A key that starts on a unit boundary (always,
// at one element per unit) fills every unit it touches, and takes the instantiation whose key
// sums carry no per-column mask (KA); only a key whose first unit straddles its first column
// keeps the masked sums. The masked and unmasked sums are the same numbers in the same order.
template <typename IO, int VEC, int NU, int TU, int WPR, int MODE, typename ACC,
          bool DEEP = false>
hipError_t launch_tile_units(const ReadParams& p, const KeyTable<MODE>& kt, hipStream_t s) {
  if constexpr (VEC == 1) {
    return launch_tile_t<IO, VEC, NU, TU, 0, false, WPR, MODE, ACC, DEEP, true>(p, kt, s);
  } else {
    if ((p.d - p.r) % VEC == 0)
      return launch_tile_t<IO, VEC, NU, TU, 0, false, WPR, MODE, ACC, DEEP, true>(p, kt, s);
    return launch_tile_t<IO, VEC, NU, TU, 0, false, WPR, MODE, ACC, DEEP, false>(p, kt, s);
  }
}

// The spread key piece a read of the value row's last r columns takes (see launch_tile_key):
// key_piece_code(KS, row-local), or 0 when the key is read from the row units. Preferably
// KS = r / 32 rounded up to a power of two, so the key fits lanes 0..31 (row-local sums), else 1
// or 2 elements over up to 64 lanes; a piece size must divide r and keep the loads aligned.
// Pieces of 16 elements (r up to 512) measured 2 % faster than the row units at r = 512,
// d = 2048.
inline int spread_piece(const ReadParams& p, int vec) {
  if (vec == 1) return 0;
  const int c0 = p.d - p.r;
  const auto fits = [&](int ks) { return p.r % ks == 0 && c0 % (ks < vec ? ks : vec) == 0; };
  if (p.r <= 32 && fits(1)) return key_piece_code(1, true);
  if (p.r <= 64 && fits(2)) return key_piece_code(2, true);
  if (p.r <= 128 && fits(4)) return key_piece_code(4, true);
  if (p.r <= 256 && fits(8)) return key_piece_code(8, true);
  if (p.r <= 512 && fits(16)) return key_piece_code(16, true);
  if (p.r <= kWave) return key_piece_code(1, false);
  if (p.r <= 2 * kWave && fits(2)) return key_piece_code(2, false);
  return 0;
}

// Key path. Spread pieces (spread_piece) when the key is short; otherwise the row units, with
// TU = 1 when every key chunk lands in a wave's last slot. The full-width-RMS control always
// sums the row units (TU = NU); the separate-key read takes the piece the host chose
// (p.key_piece, see tile_keys_piece).
template <typename IO, int VEC, int NU, int WPR, int MODE, typename ACC>
hipError_t launch_tile_key(const ReadParams& p, const KeyTable<MODE>& kt, hipStream_t s) {
  if constexpr (MODE == kTileFullRms) {
    return launch_tile_units<IO, VEC, NU, NU, WPR, MODE, ACC>(p, kt, s);
  } else if constexpr (MODE == kTileMergeAcc) {
    const int first_key_chunk = ((p.d - p.r) / VEC) / kWave;
    if constexpr (NU > 1) {
      if (first_key_chunk / WPR >= NU - 1)
        return launch_tile_units<IO, VEC, NU, 1, WPR, MODE, ACC>(p, kt, s);
    }
    return launch_tile_units<IO, VEC, NU, NU, WPR, MODE, ACC>(p, kt, s);
  } else if constexpr (MODE == kTileKeys) {
    switch (p.key_piece) {
      case key_piece_code(1, true):
        return launch_tile_spread<IO, VEC, NU, 1, true, WPR, MODE, ACC>(p, kt, s);
      case key_piece_code(1, false):
        return launch_tile_spread<IO, VEC, NU, 1, false, WPR, MODE, ACC>(p, kt, s);
      default: break;
    }
    if constexpr (VEC > 1) {
      switch (p.key_piece) {
        case key_piece_code(2, true):
          return launch_tile_spread<IO, VEC, NU, 2, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(4, true):
          return launch_tile_spread<IO, VEC, NU, 4, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(8, true):
          return launch_tile_spread<IO, VEC, NU, 8, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(2, false):
          return launch_tile_spread<IO, VEC, NU, 2, false, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(4, false):
          return launch_tile_spread<IO, VEC, NU, 4, false, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(8, false):
          return launch_tile_spread<IO, VEC, NU, 8, false, WPR, MODE, ACC>(p, kt, s);
        default: break;
      }
    }
    return hipErrorInvalidValue;
  } else {
    const int c0 = p.d - p.r;
    if constexpr (VEC > 1) {
      switch (spread_piece(p, VEC)) {
        case key_piece_code(1, true):
          return launch_tile_spread<IO, VEC, NU, 1, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(2, true):
          return launch_tile_spread<IO, VEC, NU, 2, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(4, true):
          return launch_tile_spread<IO, VEC, NU, 4, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(8, true):
          return launch_tile_spread<IO, VEC, NU, 8, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(16, true):
          return launch_tile_spread<IO, VEC, NU, 16, true, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(1, false):
          return launch_tile_spread<IO, VEC, NU, 1, false, WPR, MODE, ACC>(p, kt, s);
        case key_piece_code(2, false):
          return launch_tile_spread<IO, VEC, NU, 2, false, WPR, MODE, ACC>(p, kt, s);
        default: break;
      }
    }
    const int first_key_chunk = (c0 / VEC) / kWave;
    if constexpr (NU > 1) {
      if (first_key_chunk / WPR >= NU - 1)
        return launch_tile_units<IO, VEC, NU, 1, WPR, MODE, ACC>(p, kt, s);
    }
    return launch_tile_units<IO, VEC, NU, NU, WPR, MODE, ACC>(p, kt, s);
  }
}

// Rows of up to 4 chunks of 64 units are held by one wave; wider rows by the 4 waves of a
// workgroup, each taking every fourth chunk. The one-pass reads of 9 to 16 chunks whose key,
// read from the row units, spans at most a quarter of the row take two waves of 8 slots per row
// instead: one exchange of key sums between two waves per source instead of four. That
// measured 6 % faster at r = 1792, d = 7168, but 4 % slower at r = d = 7168 (the key fills
// every slot, and the 256 registers of the two-wave tile leave one wave per SIMD for that
// float64 work) and 3 % slower for spread keys (r = 64), whose sums need no exchange.
template <typename IO, int VEC, int MODE, typename ACC>
hipError_t launch_tile_nu(const ReadParams& p, const KeyTable<MODE>& kt, hipStream_t s) {
  const int nur = (p.d + VEC - 1) / VEC;
  const int chunks = (nur + kWave - 1) / kWave;
  if (chunks <= 1) return launch_tile_key<IO, VEC, 1, 1, MODE, ACC>(p, kt, s);
  if (chunks <= 2) return launch_tile_key<IO, VEC, 2, 1, MODE, ACC>(p, kt, s);
  if (chunks <= 4) return launch_tile_key<IO, VEC, 4, 1, MODE, ACC>(p, kt, s);
  if (chunks <= 8) return launch_tile_key<IO, VEC, 2, 4, MODE, ACC>(p, kt, s);
  if constexpr (VEC > 1 && (MODE == kTileOnline || MODE == kTileTwoPass)) {
    if (chunks <= 16 && spread_piece(p, VEC) == 0 && 4 * p.r <= p.d)
      return launch_tile_key<IO, VEC, 8, 2, MODE, ACC>(p, kt, s);
  }
  if (chunks <= 16) return launch_tile_key<IO, VEC, 4, 4, MODE, ACC>(p, kt, s);
  if (chunks <= 32) return launch_tile_key<IO, VEC, 8, 4, MODE, ACC>(p, kt, s);
  return hipErrorInvalidValue;
}

template <typename IO, int VEC, int MODE, typename ACC>
hipError_t launch_tile_nu(const ReadParams& p, hipStream_t s) {
  return launch_tile_nu<IO, VEC, MODE, ACC>(p, KeyTable<MODE>{}, s);
}

}  // namespace

}  // namespace lrar
