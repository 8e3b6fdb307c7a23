// Register-tile building blocks shared by the tile kernels of liblrattnres (internal; not
// installed): the row-unit tiles, the spread key pieces, the per-source stages of the prefetch
// ring, and the float64 key partial sums. See lrar_tile.hip for the layout they serve.
#pragma once

#include <type_traits>

#include "lrar_device.h"

namespace lrar {

enum TileMode : int {
  kTileOnline = 0,   // the read, one pass
  kTileTwoPass = 1,  // the read, key slices first
  kTileMerge = 2,    // Phase 2: the online pass started from Phase-1 statistics
  kTileFullRms = 3,  // the full-width-RMS control read, one pass
  kTileKeys = 4,     // the separate-key read, one pass
  kTileMergeAcc = 5  // Phase 2 with the partial-sum update b' = b + o fused in
};

// Per-source key table: only the separate-key read has one (an empty argument otherwise).
struct NoKeyTable {};
template <int MODE>
using KeyTable = typename std::conditional<MODE == kTileKeys, SrcList, NoKeyTable>::type;

constexpr double kLazyRescale = 8.0;

template <typename IO, int VEC, int NU, int R>
struct Tile {
  Unit<IO, VEC> u[R][NU];
};

// KS consecutive key elements of one row, raw.
template <typename IO, int KS>
struct KeyPiece;

template <typename IO>
struct KeyPiece<IO, 0> {
  __device__ __forceinline__ void load(const IO*) {}
  __device__ __forceinline__ void load_span(const Span&, uint32_t) {}
  __device__ __forceinline__ void zero() {}
};

template <>
struct KeyPiece<bf16_bits, 1> {
  uint32_t raw;
  __device__ __forceinline__ void load(const bf16_bits* p) { raw = *p; }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    raw = s.b16<false>(off);
  }
  __device__ __forceinline__ void zero() { raw = 0u; }
  __device__ __forceinline__ void get(float (&x)[1]) const { x[0] = __uint_as_float(raw << 16); }
};

template <>
struct KeyPiece<bf16_bits, 2> {
  uint32_t raw;
  __device__ __forceinline__ void load(const bf16_bits* p) {
    raw = *reinterpret_cast<const uint32_t*>(p);
  }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    raw = s.b32<false>(off);
  }
  __device__ __forceinline__ void zero() { raw = 0u; }
  __device__ __forceinline__ void get(float (&x)[2]) const {
    x[0] = __uint_as_float(raw << 16);
    x[1] = __uint_as_float(raw & 0xffff0000u);
  }
};

template <>
struct KeyPiece<bf16_bits, 4> {
  uint32_t raw[2];
  __device__ __forceinline__ void load(const bf16_bits* p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    raw[0] = v.x;
    raw[1] = v.y;
  }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    const u32x2 v = s.b64<false>(off);
    raw[0] = v.x;
    raw[1] = v.y;
  }
  __device__ __forceinline__ void zero() { raw[0] = raw[1] = 0u; }
  __device__ __forceinline__ void get(float (&x)[4]) const {
    x[0] = __uint_as_float(raw[0] << 16);
    x[1] = __uint_as_float(raw[0] & 0xffff0000u);
    x[2] = __uint_as_float(raw[1] << 16);
    x[3] = __uint_as_float(raw[1] & 0xffff0000u);
  }
};

template <>
struct KeyPiece<float, 1> {
  float raw;
  __device__ __forceinline__ void load(const float* p) { raw = *p; }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    raw = __uint_as_float(s.b32<false>(off));
  }
  __device__ __forceinline__ void zero() { raw = 0.f; }
  __device__ __forceinline__ void get(float (&x)[1]) const { x[0] = raw; }
};

template <>
struct KeyPiece<float, 2> {
  float raw[2];
  __device__ __forceinline__ void load(const float* p) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = *reinterpret_cast<const f32x2*>(p);
    raw[0] = v.x;
    raw[1] = v.y;
  }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    const u32x2 v = s.b64<false>(off);
    raw[0] = __uint_as_float(v.x);
    raw[1] = __uint_as_float(v.y);
  }
  __device__ __forceinline__ void zero() { raw[0] = raw[1] = 0.f; }
  __device__ __forceinline__ void get(float (&x)[2]) const {
    x[0] = raw[0];
    x[1] = raw[1];
  }
};

template <>
struct KeyPiece<float, 4> {
  float raw[4];
  __device__ __forceinline__ void load(const float* p) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
    raw[0] = v.x;
    raw[1] = v.y;
    raw[2] = v.z;
    raw[3] = v.w;
  }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    const u32x4 v = s.b128<false>(off);
    raw[0] = __uint_as_float(v.x);
    raw[1] = __uint_as_float(v.y);
    raw[2] = __uint_as_float(v.z);
    raw[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ void zero() { raw[0] = raw[1] = raw[2] = raw[3] = 0.f; }
  __device__ __forceinline__ void get(float (&x)[4]) const {
    x[0] = raw[0];
    x[1] = raw[1];
    x[2] = raw[2];
    x[3] = raw[3];
  }
};

// 8 or 16 consecutive key elements: one or more 16-byte units.
template <typename IO, int KS>
struct KeyPieceUnits {
  static constexpr int kPer = 16 / sizeof(IO);  // elements per 16-byte unit
  static constexpr int kUnits = KS / kPer;
  Unit<IO, 16 / sizeof(IO)> u[kUnits];
  __device__ __forceinline__ void load(const IO* p) {
#pragma unroll
    for (int k = 0; k < kUnits; ++k) u[k].load_cached(p + k * kPer);
  }
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
#pragma unroll
    for (int k = 0; k < kUnits; ++k) u[k].template load_span<false>(s, off + 16u * k);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < kUnits; ++k) u[k].zero();
  }
  __device__ __forceinline__ void get(float (&x)[KS]) const {
#pragma unroll
    for (int k = 0; k < kUnits; ++k) {
      float y[kPer];
      u[k].get(y);
#pragma unroll
      for (int e = 0; e < kPer; ++e) x[k * kPer + e] = y[e];
    }
  }
};

template <>
struct KeyPiece<bf16_bits, 8> : KeyPieceUnits<bf16_bits, 8> {};
template <>
struct KeyPiece<bf16_bits, 16> : KeyPieceUnits<bf16_bits, 16> {};
template <>
struct KeyPiece<float, 8> : KeyPieceUnits<float, 8> {};
template <>
struct KeyPiece<float, 16> : KeyPieceUnits<float, 16> {};

// One source's tile in flight: the rows and, with KS > 0, the spread key pieces of each row.
template <typename IO, int VEC, int NU, int R, int KS>
struct Stage {
  Tile<IO, VEC, NU, R> t;
  KeyPiece<IO, KS> kp[R];
};

struct TileGeom {
  int64_t r0;  // first row of the tile
  int nrow;    // rows of the tile that exist (<= R)
  int lane, nur, ub, c0, r;
  int w, wpr;  // this wave's place among the wpr waves that share a row
  // Unit held in slot k: the row is cut into chunks of 64 units and chunk c belongs to wave
  // c % wpr, so the waves of a row share the chunks (and the key) evenly.
  __device__ __forceinline__ int unit(int k) const { return (k * wpr + w) * kWave + lane; }
};

// Loads one source's tile. KEYS_ONLY: only the key (the spread pieces, or the key units when
// KS = 0). SEP: the spread key pieces come from the source's own key rows (kbase, row stride
// kld) instead of the value row's last r columns. Slots outside the tile (a row past the
// tile's last, a unit past the row's end or, KEYS_ONLY, before the key, a key piece past the
// key) read as zero.
//
// Two ways to skip those slots. load_stage_branchy skips them under branches, and a stage that
// is not needed (live false) is not loaded at all; the compiler then cannot count the loads in
// flight and waits for all of them before it uses the oldest stage. load_stage_exact issues
// every load in every lane through a Span: skipped slots take the offset kNoLoad and a stage
// that is not needed loads over an empty span, reading no memory either way, so every item of
// the ring leaves the same loads in flight and a wait for a stage is a wait for it alone.
// Measured on MI355X, exact waits pay where each stage carries much vector work (the key read
// from the row units, KS = 0: wide keys and the full-RMS control, up to a fifth faster) and on
// short-key reads of few sources (the two-deep ring: 5-11 % at 2 to 7 sources), and cost a few
// percent on short-key reads of many sources through the three-deep ring, where the other
// waves already hide the latency. The read kernel picks per instance (load_stage_as), the
// backward by KS (load_stage).
template <bool KEYS_ONLY, bool SEP = false, typename IO, int VEC, int NU, int R, int KS>
__device__ __forceinline__ void load_stage_branchy(Stage<IO, VEC, NU, R, KS>& st,
                                                   const IO* __restrict__ base, int64_t ld,
                                                   const TileGeom& g, const IO* kbase = nullptr,
                                                   int64_t kld = 0, bool live = true) {
  if (!live) return;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const IO* rowp = base + (g.r0 + j) * ld;  // wave-uniform: lane offsets stay 32-bit
    if constexpr (KS > 0) {
      const IO* keyp = SEP ? kbase + (g.r0 + j) * kld : rowp + g.c0;
      if (j < g.nrow && g.lane * KS < g.r) st.kp[j].load(keyp + g.lane * KS);
      else st.kp[j].zero();
    }
    if constexpr (!(KEYS_ONLY && KS > 0)) {
#pragma unroll
      for (int k = 0; k < NU; ++k) {
        const int u = g.unit(k);
        const bool want = j < g.nrow && u < g.nur && (!KEYS_ONLY || u >= g.ub);
        if (want) st.t.u[j][k].load(rowp + u * VEC);
        else st.t.u[j][k].zero();
      }
    }
  }
}

template <bool KEYS_ONLY, bool SEP = false, typename IO, int VEC, int NU, int R, int KS>
__device__ __forceinline__ void load_stage_exact(Stage<IO, VEC, NU, R, KS>& st,
                                                 const IO* __restrict__ base, int64_t ld,
                                                 const TileGeom& g, const IO* kbase = nullptr,
                                                 int64_t kld = 0, bool live = true) {
  constexpr uint32_t es = sizeof(IO);
  const uint32_t row_bytes = static_cast<uint32_t>(ld) * es;
  const uint32_t span = live ? static_cast<uint32_t>((g.nrow - 1) * ld + g.nur * VEC) * es : 0u;
  const Span rows(base + g.r0 * ld, span);
  if constexpr (KS > 0) {
    const bool lane_ok = g.lane * KS < g.r;
    if constexpr (SEP) {
      const uint32_t kspan = live ? static_cast<uint32_t>((g.nrow - 1) * kld + g.r) * es : 0u;
      const Span keys(kbase + g.r0 * kld, kspan);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const uint32_t off = static_cast<uint32_t>(j * kld + g.lane * KS) * es;
        st.kp[j].load_span(keys, j < g.nrow && lane_ok ? off : kNoLoad);
      }
    } else {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const uint32_t off = j * row_bytes + static_cast<uint32_t>(g.c0 + g.lane * KS) * es;
        st.kp[j].load_span(rows, j < g.nrow && lane_ok ? off : kNoLoad);
      }
    }
  }
  if constexpr (!(KEYS_ONLY && KS > 0)) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int k = 0; k < NU; ++k) {
        const int u = g.unit(k);
        const bool want = j < g.nrow && u < g.nur && (!KEYS_ONLY || u >= g.ub);
        const uint32_t off = j * row_bytes + static_cast<uint32_t>(u) * (VEC * es);
        st.t.u[j][k].load_span(rows, want ? off : kNoLoad);
      }
    }
  }
}

template <bool KEYS_ONLY, bool SEP, bool EXACT, typename IO, int VEC, int NU, int R, int KS>
__device__ __forceinline__ void load_stage_as(Stage<IO, VEC, NU, R, KS>& st,
                                              const IO* __restrict__ base, int64_t ld,
                                              const TileGeom& g, const IO* kbase = nullptr,
                                              int64_t kld = 0, bool live = true) {
  if constexpr (EXACT) load_stage_exact<KEYS_ONLY, SEP>(st, base, ld, g, kbase, kld, live);
  else load_stage_branchy<KEYS_ONLY, SEP>(st, base, ld, g, kbase, kld, live);
}

// Exact for keys read from the row units, branchy for spread keys.
template <bool KEYS_ONLY, bool SEP = false, typename IO, int VEC, int NU, int R, int KS>
__device__ __forceinline__ void load_stage(Stage<IO, VEC, NU, R, KS>& st,
                                           const IO* __restrict__ base, int64_t ld,
                                           const TileGeom& g, const IO* kbase = nullptr,
                                           int64_t kld = 0, bool live = true) {
  load_stage_as<KEYS_ONLY, SEP, KS == 0>(st, base, ld, g, kbase, kld, live);
}

// This lane's share of q . k and k . k for one row from its key units (KS = 0). Only the
// last TU unit slots can hold key columns (the host picks TU so that the key starts in slot
// NU - TU or later).
template <int TU, bool KA = false, typename IO, int VEC, int NU, typename QS>
__device__ __forceinline__ void key_partial_units(const Unit<IO, VEC> (&row)[NU],
                                                  const QS& qs, const TileGeom& g,
                                                  double& dot, double& ss) {
  dot = 0.0;
  ss = 0.0;
#pragma unroll
  for (int k = NU - TU; k < NU; ++k) {
    const int u = g.unit(k);
    if (u >= g.ub && u < g.nur) {
      float x[VEC];
      row[k].get(x);
      typename QS::value_type qv[VEC];
      qs.template get<VEC>(u - g.ub, qv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        // KA: the key starts on a unit boundary, so every column of a key unit is a key column
        const double kv =
            KA || u * VEC + e >= g.c0 ? static_cast<double>(x[e]) : 0.0;
        dot = fma(static_cast<double>(qv[e]), kv, dot);
        ss = fma(kv, kv, ss);
      }
    }
  }
}

// This lane's share of q . k over the key columns and of o . o over the whole row, for the
// full-width-RMS control: every unit slot of the row counts toward the square sum.
template <bool KA = false, typename IO, int VEC, int NU, typename QS>
__device__ __forceinline__ void row_partial_full(const Unit<IO, VEC> (&row)[NU],
                                                 const QS& qs, const TileGeom& g,
                                                 double& dot, double& ss) {
  dot = 0.0;
  ss = 0.0;
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    const int u = g.unit(k);
    if (u < g.nur) {
      float x[VEC];
      row[k].get(x);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const double v = static_cast<double>(x[e]);
        ss = fma(v, v, ss);
      }
      if (u >= g.ub) {
        typename QS::value_type qv[VEC];
        qs.template get<VEC>(u - g.ub, qv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const double kv = KA || u * VEC + e >= g.c0 ? static_cast<double>(x[e]) : 0.0;
          dot = fma(static_cast<double>(qv[e]), kv, dot);
        }
      }
    }
  }
}

// This lane's share of q . k and k . k from its spread key piece (KS > 0); qs holds the
// matching query values (0 beyond the key).
template <typename IO, int KS, typename QT>
__device__ __forceinline__ void key_partial_spread(const KeyPiece<IO, KS>& kp,
                                                   const QT (&qs)[KS], double& dot,
                                                   double& ss) {
  float x[KS];
  kp.get(x);
  dot = 0.0;
  ss = 0.0;
#pragma unroll
  for (int e = 0; e < KS; ++e) {
    const double kv = static_cast<double>(x[e]);
    dot = fma(static_cast<double>(qs[e]), kv, dot);
    ss = fma(kv, kv, ss);
  }
}

// A source's score z and the reciprocal 1 / rho of its key's RMS.
struct Score {
  double z, rinv;
};

// z = dot / sqrt(ss / r + eps) as dot * rsq(ss / r + eps), with 1 / r passed in (rinv_r,
// computed once per kernel). The hardware reciprocal square root is good to about 2^-23
// relative; one Newton step y <- y (3 - a y^2) / 2 squares that error, to about 2^-45. A zero key
// with eps = 0 gives 0 * inf = NaN, as the division does.
__device__ __forceinline__ Score score_from_sums(double dot, double ss, double rinv_r,
                                                 double eps) {
  const double a = fma(ss, rinv_r, eps);
  double y = __builtin_amdgcn_rsq(a);
  y = y * fma(-0.5 * a, y * y, 1.5);
  return Score{dot * y, y};
}

// e^x for x <= kLazyRescale, accurate to about 2^-31 relative (the weights it feeds are
// rounded to float32): x = k ln 2 + f with |f| <= ln 2 / 2, e^f by its Taylor series to the
// 8th power (truncation < 2^-31), then scaled by 2^k. Arguments below -745 give 0; NaN stays
// NaN.
__device__ __forceinline__ double exp_weight(double x) {
  constexpr double kLog2e = 1.4426950408889634;
  constexpr double kLn2Hi = 6.93147180369123816490e-01;  // ln 2 split so k * kLn2Hi is exact
  constexpr double kLn2Lo = 1.90821492927058770002e-10;
  const double xc = x < -745.0 ? -745.0 : x;  // a comparison, so NaN passes through
  const double k = rint(xc * kLog2e);
  const double f = fma(-k, kLn2Lo, fma(-k, kLn2Hi, xc));
  double p = 1.0 / 40320.0;
  p = fma(p, f, 1.0 / 5040.0);
  p = fma(p, f, 1.0 / 720.0);
  p = fma(p, f, 1.0 / 120.0);
  p = fma(p, f, 1.0 / 24.0);
  p = fma(p, f, 1.0 / 6.0);
  p = fma(p, f, 0.5);
  p = fma(p, f, 1.0);
  p = fma(p, f, 1.0);
  return ldexp(p, static_cast<int>(k));
}

// Lane i ^ 16 within each half-wave (ds_swizzle in bit-mask mode: and 0x1f, xor 0x10).
__device__ __forceinline__ double swizzle_xor16_f64(double v) {
  constexpr int kXor16 = 0x1f | (0x10 << 10);
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_ds_swizzle(static_cast<int>(b), kXor16);
  const int hi = __builtin_amdgcn_ds_swizzle(static_cast<int>(b >> 32), kXor16);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Sums over each half of the wave (lanes 0..31, 32..63) of R = 1 or 2 rows' (q . k, k . k)
// pairs by a transposed butterfly. Partners that differ in lane bit 0, then bit 1, swap halves
// of their value set, so after two steps each lane carries one value summed over its quad;
// rotations of each DPP row by 4 and 8 lanes add the row's four quads, and a lane-xor-16
// swizzle adds the half's second row. Lane l then holds the half's sum of
// red[transposed_index<R>(l & 3)].
template <int R>
__device__ __forceinline__ double half_sums_transposed(const double (&red)[2 * R], int lane) {
  static_assert(R == 1 || R == 2, "two or four values");
  constexpr int kRor4 = 0x124, kRor8 = 0x128;
  const bool b0 = (lane & 1) != 0;
  double x;
  if constexpr (R == 2) {
    // values 0..3 = dot0, ss0, dot1, ss1; after the xor-1 step lanes with bit 0 clear carry
    // {dot0, ss0}, the others {dot1, ss1}; after the xor-2 step lane (b1 b0) carries value
    // 2 b0 + b1: lane 0 dot0, lane 1 dot1, lane 2 ss0, lane 3 ss1.
    const double keep0 = b0 ? red[2] : red[0], send0 = b0 ? red[0] : red[2];
    const double keep1 = b0 ? red[3] : red[1], send1 = b0 ? red[1] : red[3];
    const double w0 = keep0 + dpp_f64_all<kDppXor1>(send0);
    const double w1 = keep1 + dpp_f64_all<kDppXor1>(send1);
    const bool b1 = (lane & 2) != 0;
    x = (b1 ? w1 : w0) + dpp_f64_all<kDppXor2>(b1 ? w0 : w1);
  } else {
    // values 0, 1 = dot, ss; lane 0 ends with dot, lane 1 with ss
    x = (b0 ? red[1] : red[0]) + dpp_f64_all<kDppXor1>(b0 ? red[0] : red[1]);
    x += dpp_f64_all<kDppXor2>(x);
  }
  x += dpp_f64_all<kRor4>(x);
  x += dpp_f64_all<kRor8>(x);
  x += swizzle_xor16_f64(x);
  return x;
}

// The score of row j (< R) in lane j from transposed (dot, ss) sums: the ss of row j sits R
// lanes after its dot (quad_perm [2,3,2,3] for R = 2, [1,1,3,3] for R = 1).
template <int R>
__device__ __forceinline__ Score score_from_transposed(double x, double rinv_r, double eps) {
  const double ss = dpp_f64_all<R == 2 ? 0xEE : 0xF5>(x);
  return score_from_sums(x, ss, rinv_r, eps);
}

// Row-local sums for R = 1 or 2 tile rows when the spread key sits in lanes 0..31: the sums of
// the wave's first half are the rows' sums. Lane j (< R) returns row j's score.
template <int R>
__device__ __forceinline__ Score row_scores_rowlocal(const double (&red)[2 * R], int lane,
                                                      double rinv_r,
                                                      double eps) {
  return score_from_transposed<R>(half_sums_transposed<R>(red, lane), rinv_r, eps);
}

// Sums over the whole wave of R = 1 or 2 rows' (q . k, k . k) pairs: the halves' transposed
// sums added through the lane crossbar (a lane-xor-32 exchange, which is not a vector ALU
// instruction). About 20 (R = 1) or 31 (R = 2) vector instructions instead of the 40 or 80 of
// a full butterfly per value. Lane l < 2R returns the sum of red[transposed_index<R>(l)];
// lanes past 2R repeat those values.
template <int R>
__device__ __forceinline__ double wave_sums_transposed(const double (&red)[2 * R], int lane) {
  const double x = half_sums_transposed<R>(red, lane);
  return x + shfl_xor_f64(x, 32);
}

// Sums over the whole wave of 16 values: two transposed butterfly steps leave each lane of a
// quad 4 of the 16 values summed over the quad (lane l: values 8 (l & 1) + 4 ((l >> 1) & 1) +
// k, k = 0..3), and those 4 are then added over the quads of each DPP row, over the rows of
// each half (lane-xor-16 swizzle) and over the two halves (lane-xor-32 exchange). About 90
// vector instructions instead of about 300 for a butterfly per value.
__device__ __forceinline__ void wave_sums_transposed16(const double (&v)[16], int lane,
                                                       double (&u)[4]) {
  constexpr int kRor4 = 0x124, kRor8 = 0x128;
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  double w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const double keep = b0 ? v[8 + k] : v[k], send = b0 ? v[k] : v[8 + k];
    w[k] = keep + dpp_f64_all<kDppXor1>(send);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double keep = b1 ? w[4 + k] : w[k], send = b1 ? w[k] : w[4 + k];
    u[k] = keep + dpp_f64_all<kDppXor2>(send);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] += dpp_f64_all<kRor4>(u[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] += dpp_f64_all<kRor8>(u[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] += swizzle_xor16_f64(u[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] += shfl_xor_f64(u[k], 32);
}

// The index into red[] (dot0, ss0, dot1, ss1) of the sum that lane l < 2R holds after
// wave_sums_transposed.
template <int R>
__device__ __forceinline__ int transposed_index(int lane) {
  return R == 2 ? 2 * (lane & 1) + ((lane >> 1) & 1) : (lane & 1);
}

// Scores of R = 1 or 2 rows whose key sits in the row units of one wave, from
// wave_sums_transposed. Lane j (< R) returns row j's score; other lanes return values of no
// meaning.
template <int R>
__device__ __forceinline__ Score row_scores_wave(const double (&red)[2 * R], int lane,
                                                  double rinv_r,
                                                  double eps) {
  return score_from_transposed<R>(wave_sums_transposed<R>(red, lane), rinv_r, eps);
}

// Scores of the R rows of a tile from their reduced (q . k, k . k) pairs, one row per lane:
// lane j < R returns z of row j (lanes >= R return row 0's), so the square root and the
// division run once for all rows.
template <int R>
__device__ __forceinline__ Score row_scores_to_lanes(const double (&red)[2 * R], int lane,
                                                      double rinv_r,
                                                      double eps) {
  double dot = red[0], ss = red[1];
#pragma unroll
  for (int j = 1; j < R; ++j) {
    if (lane == j) {
      dot = red[2 * j];
      ss = red[2 * j + 1];
    }
  }
  return score_from_sums(dot, ss, rinv_r, eps);
}

template <typename IO, int VEC, int NU>
__device__ __forceinline__ void fma_row(float (&acc)[NU][VEC], float w,
                                        const Unit<IO, VEC> (&row)[NU]) {
#pragma unroll
  for (int k = 0; k < NU; ++k) {
    float x[VEC];
    row[k].get(x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[k][e] = fmaf(w, x[e], acc[k][e]);
  }
}

constexpr int ks_slots(int ks) { return ks > 0 ? ks : 1; }

// The spread query values a lane keeps: float64 for pieces of up to 4 elements, float32 (and
// widened on use) for larger pieces, which would otherwise take 16 or 32 registers.
template <int KS>
using SpreadQ = typename std::conditional<(KS > 4), float, double>::type;

}  // namespace lrar
