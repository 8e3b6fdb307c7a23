// Device-side building blocks of liblrattnres (internal; not installed).
//
// Layout conventions shared by the kernels:
//   * A row is cut into "units" of VEC consecutive elements, 16 bytes on the vector path
//     (8 bf16 or 4 fp32) and one element on the element path. Within a chunk of 64 units the
//     lanes of a wave hold consecutive units, so each load instruction of a wave covers one
//     contiguous 1 KiB stretch of the row.
//   * Rows go to wavefronts either one row per wave at a time (the one-wave-per-row kernels)
//     or as register tiles of a few rows, a row's chunks possibly shared by the four waves of
//     a workgroup (the tile kernels; see lrar_tile_impl.h).
//   * The key slice is the columns [d - r, d). Units that straddle d - r mask their leading
//     elements out of the key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lrar {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kMaxSources = 64;
constexpr int kMaxQueries = 64;

// Index of the calling wave within its workgroup, as a wave-uniform (scalar) value, so that
// row indices and row pointers derived from it stay in scalar registers and global accesses
// take the scalar-base + 32-bit lane-offset form instead of per-lane 64-bit address math.
__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

// Source pointer table, passed by value in the kernel arguments (1 KiB).
struct SrcList {
  const void* ptr[kMaxSources];
  int64_t ld[kMaxSources];
};

// Gradient destinations (float32 or bf16 rows, by the entry point's gradient type).
struct DstList {
  void* ptr[kMaxSources];
  int64_t ld[kMaxSources];
};

using bf16_bits = uint16_t;

// Native 16-byte vector types (accepted by the non-temporal load/store builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- loads with a predicate and no branch ---------------------------------------------------
// A raw buffer resource over [base, base + bytes) (CDNA resource word 3: 32-bit data format,
// no stride). A load through it at a byte offset at or past `bytes` returns zero and reads no
// memory: the hardware's range check. A lane with nothing to load passes kNoLoad, and a whole
// load is switched off with an empty span; either way the instruction is still issued. Loads
// taken under branches would leave the compiler unsure how many loads are in flight, and its
// wait for one of them would then wait for all.
constexpr uint32_t kNoLoad = 0x80000000u;  // past every span used here (each < 2^31 bytes)
constexpr int kCachePolicyNT = 2;          // the nontemporal bit of the buffer load's policy
// base and bytes must be the same in every lane of the wave: the resource lives in scalar
// registers, and they are read from the first active lane (else the compiler, unable to prove
// them uniform, would wrap each load in a loop over the distinct values).
struct Span {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ Span(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(ub, 0, static_cast<int>(n), 0x00020000);
  }
  template <bool NT>
  __device__ __forceinline__ u32x4 b128(uint32_t off) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rsrc, static_cast<int>(off), 0, NT ? kCachePolicyNT : 0));
  }
  template <bool NT>
  __device__ __forceinline__ u32x2 b64(uint32_t off) const {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                         rsrc, static_cast<int>(off), 0, NT ? kCachePolicyNT : 0));
  }
  template <bool NT>
  __device__ __forceinline__ uint32_t b32(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, static_cast<int>(off), 0,
                                                NT ? kCachePolicyNT : 0);
  }
  template <bool NT>
  __device__ __forceinline__ uint16_t b16(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b16(rsrc, static_cast<int>(off), 0,
                                                NT ? kCachePolicyNT : 0);
  }
};

// ---- scalar conversions ------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN. gfx950 converts in
// hardware (v_cvt_pk_bf16_f32, two values per instruction).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_bits, static_cast<__bf16>(f));
}

// Two floats as two bfloat16 in one 32-bit word, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_bits>(bf16_bits v) { return bf16_to_f32(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_bits from_f32<bf16_bits>(float v) { return f32_to_bf16(v); }

// Store of one output unit (16, 8 or 4 bytes), nontemporal: outputs are written once and not
// read back by the kernel, and streaming them out keeps dirty lines from waiting in L2 and the
// memory-side cache, whose later write-back would fall outside the kernel's own time.
template <typename V>
__device__ __forceinline__ void out_store(V v, V* p) {
  __builtin_nontemporal_store(v, p);
}

// ---- unit loads and stores ------------------------------------------------------------------

// A unit of VEC elements of type T held in raw (undecoded) form.
template <typename T, int VEC>
struct Unit;

template <>
struct Unit<bf16_bits, 8> {
  u32x4 raw;
  __device__ __forceinline__ void load(const bf16_bits* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void load_cached(const bf16_bits* p) {
    raw = *reinterpret_cast<const u32x4*>(p);
  }
  template <bool NT = true>
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    raw = s.b128<NT>(off);
  }
  __device__ __forceinline__ void zero() { raw = u32x4{0u, 0u, 0u, 0u}; }
  // Encodes 8 floats (round to nearest even) / writes the raw unit with a streaming store.
  __device__ __forceinline__ void set(const float (&x)[8]) {
    raw.x = pack_bf16x2(x[0], x[1]);
    raw.y = pack_bf16x2(x[2], x[3]);
    raw.z = pack_bf16x2(x[4], x[5]);
    raw.w = pack_bf16x2(x[6], x[7]);
  }
  __device__ __forceinline__ void store(bf16_bits* p) const {
    out_store(raw, reinterpret_cast<u32x4*>(p));
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = __uint_as_float(raw.x << 16);
    x[1] = __uint_as_float(raw.x & 0xffff0000u);
    x[2] = __uint_as_float(raw.y << 16);
    x[3] = __uint_as_float(raw.y & 0xffff0000u);
    x[4] = __uint_as_float(raw.z << 16);
    x[5] = __uint_as_float(raw.z & 0xffff0000u);
    x[6] = __uint_as_float(raw.w << 16);
    x[7] = __uint_as_float(raw.w & 0xffff0000u);
  }
};

template <>
struct Unit<float, 4> {
  f32x4 raw;
  __device__ __forceinline__ void load(const float* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ void load_cached(const float* p) {
    raw = *reinterpret_cast<const f32x4*>(p);
  }
  template <bool NT = true>
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    raw = __builtin_bit_cast(f32x4, s.b128<NT>(off));
  }
  __device__ __forceinline__ void zero() { raw = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void set(const float (&x)[4]) { raw = f32x4{x[0], x[1], x[2], x[3]}; }
  __device__ __forceinline__ void store(float* p) const {
    out_store(raw, reinterpret_cast<f32x4*>(p));
  }
  __device__ __forceinline__ void get(float (&x)[4]) const {
    x[0] = raw.x;
    x[1] = raw.y;
    x[2] = raw.z;
    x[3] = raw.w;
  }
};

template <typename T>
struct Unit<T, 1> {
  T raw;
  __device__ __forceinline__ void load(const T* p) { raw = *p; }
  __device__ __forceinline__ void load_cached(const T* p) { raw = *p; }
  template <bool NT = false>
  __device__ __forceinline__ void load_span(const Span& s, uint32_t off) {
    if constexpr (sizeof(T) == 2) raw = __builtin_bit_cast(T, s.b16<NT>(off));
    else raw = __builtin_bit_cast(T, s.b32<NT>(off));
  }
  __device__ __forceinline__ void zero() { raw = T(0); }
  __device__ __forceinline__ void set(const float (&x)[1]) { raw = from_f32<T>(x[0]); }
  __device__ __forceinline__ void store(T* p) const { *p = raw; }
  __device__ __forceinline__ void get(float (&x)[1]) const { x[0] = to_f32<T>(raw); }
};

// Store VEC floats as VEC elements of T at p (16-byte aligned on the vector path).
template <typename T, int VEC>
__device__ __forceinline__ void store_unit(T* p, const float (&x)[VEC]);

template <>
__device__ __forceinline__ void store_unit<bf16_bits, 8>(bf16_bits* p, const float (&x)[8]) {
  u32x4 v;
  v.x = pack_bf16x2(x[0], x[1]);
  v.y = pack_bf16x2(x[2], x[3]);
  v.z = pack_bf16x2(x[4], x[5]);
  v.w = pack_bf16x2(x[6], x[7]);
  out_store(v, reinterpret_cast<u32x4*>(p));
}

template <>
__device__ __forceinline__ void store_unit<float, 4>(float* p, const float (&x)[4]) {
  out_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
}

template <>
__device__ __forceinline__ void store_unit<float, 8>(float* p, const float (&x)[8]) {
  out_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
  out_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p) + 1);
}

template <>
__device__ __forceinline__ void store_unit<float, 1>(float* p, const float (&x)[1]) { *p = x[0]; }

template <>
__device__ __forceinline__ void store_unit<bf16_bits, 1>(bf16_bits* p, const float (&x)[1]) {
  *p = f32_to_bf16(x[0]);
}

// Load VEC float32 values (16-byte aligned on the vector path).
template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float (&x)[VEC]) {
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int v = 0; v < VEC / 4; ++v) {
      const f32x4 t = reinterpret_cast<const f32x4*>(p)[v];
      x[4 * v + 0] = t.x;
      x[4 * v + 1] = t.y;
      x[4 * v + 2] = t.z;
      x[4 * v + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) x[v] = p[v];
  }
}

// Load VEC accumulator values of type A (float or bf16) as floats.
template <typename A, int VEC>
__device__ __forceinline__ void load_acc(const A* p, float (&x)[VEC]) {
  if constexpr (sizeof(A) == 4) {
    load_f32<VEC>(reinterpret_cast<const float*>(p), x);
  } else if constexpr (VEC == 8) {
    Unit<bf16_bits, 8> u;
    u.load(reinterpret_cast<const bf16_bits*>(p));
    u.get(x);
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) x[v] = to_f32<A>(p[v]);
  }
}

template <typename A, int VEC>
__device__ __forceinline__ void store_acc(A* p, const float (&x)[VEC]) {
  if constexpr (sizeof(A) == 4 && VEC % 4 == 0) {
    store_unit<float, VEC>(reinterpret_cast<float*>(p), x);
  } else if constexpr (sizeof(A) == 2 && VEC == 8) {
    store_unit<bf16_bits, 8>(reinterpret_cast<bf16_bits*>(p), x);
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) p[v] = from_f32<A>(x[v]);
  }
}

// VEC gradient values of type G (float32 or bf16) as floats, and back with round to nearest
// even; on the vector path a row's units start at multiples of 4 * VEC (float32) or 2 * VEC
// (bf16) bytes.

template <typename G, int VEC>
__device__ __forceinline__ void load_grad(const G* p, float (&x)[VEC]) {
  if constexpr (std::is_same<G, float>::value) {
    load_f32<VEC>(p, x);
  } else if constexpr (VEC == 8) {
    Unit<bf16_bits, 8> u;
    u.load_cached(p);
    u.get(x);
  } else if constexpr (VEC == 4) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xffff0000u);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[e] = bf16_to_f32(p[e]);
  }
}

template <typename G, int VEC>
__device__ __forceinline__ void store_grad(G* p, const float (&x)[VEC]) {
  if constexpr (std::is_same<G, float>::value) {
    store_unit<float, VEC>(p, x);
  } else if constexpr (VEC == 8) {
    store_unit<bf16_bits, 8>(p, x);
  } else if constexpr (VEC == 4) {
    u32x2 v;
    v.x = pack_bf16x2(x[0], x[1]);
    v.y = pack_bf16x2(x[2], x[3]);
    out_store(v, reinterpret_cast<u32x2*>(p));
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) p[e] = f32_to_bf16(x[e]);
  }
}

// Lane l holds floats 8l..8l+7 of a run of 512 (one 16-byte bf16 unit's worth of float32
// values per lane). Returns in lo the floats 4l..4l+3 and in hi the floats 256+4l..256+4l+3 of
// the run, so that a 16-byte store of lo, then of hi, by every lane writes 1 KiB contiguously
// each time instead of two half-filled 2 KiB spans. Every lane of the wave must take part.
__device__ __forceinline__ void run_halves(const float (&v)[8], int lane, float (&lo)[4],
                                           float (&hi)[4]) {
  const int a1 = (lane >> 1) << 2;         // byte address of the holder lane l / 2
  const int a2 = ((lane >> 1) + 32) << 2;  // and of 32 + l / 2
  const bool odd = (lane & 1) != 0;        // which half of the holder's 8 floats
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int x0 = __builtin_amdgcn_ds_bpermute(a1, __float_as_int(v[e]));
    const int x1 = __builtin_amdgcn_ds_bpermute(a1, __float_as_int(v[4 + e]));
    lo[e] = __int_as_float(odd ? x1 : x0);
    const int y0 = __builtin_amdgcn_ds_bpermute(a2, __float_as_int(v[e]));
    const int y1 = __builtin_amdgcn_ds_bpermute(a2, __float_as_int(v[4 + e]));
    hi[e] = __int_as_float(odd ? y1 : y0);
  }
}

// The site query staged in LDS for the key units, in VEC-element units v = u - ub counted
// from the first key unit (columns of that unit before the key hold zero). On the vector path
// the units are stored "transposed": elements 4j..4j+3 of unit v are the float4 at index
// j * nv + v, so the lanes of a wave, which hold consecutive units, read consecutive 16-byte
// words (no bank conflicts); on the element path unit v is element v.
struct QStage {
  using value_type = float;
  float* base;
  int nv;  // staged units
  // Stages the query (all threads of the workgroup; call __syncthreads afterwards).
  template <int VEC>
  __device__ __forceinline__ void fill(const float* __restrict__ q, int ub, int c0, int tid,
                                       int nthreads) {
    for (int idx = tid; idx < nv * VEC; idx += nthreads) {
      const int col = ub * VEC + idx;
      const float v = col >= c0 ? q[col - c0] : 0.f;
      const int unit = idx / VEC, e = idx - unit * VEC;
      if constexpr (VEC % 4 == 0) base[((e / 4) * nv + unit) * 4 + (e % 4)] = v;
      else base[idx] = v;
    }
  }
  template <int VEC>
  __device__ __forceinline__ void get(int v, float (&q)[VEC]) const {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
      for (int j = 0; j < VEC / 4; ++j) {
        const f32x4 t = reinterpret_cast<const f32x4*>(base)[j * nv + v];
        q[4 * j + 0] = t.x;
        q[4 * j + 1] = t.y;
        q[4 * j + 2] = t.z;
        q[4 * j + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[e] = base[v * VEC + e];
    }
  }
};

// The same staging in float64 (two values per 16-byte word, transposed likewise), so the
// scoring needs no per-element conversion of q.
struct QStageD {
  using value_type = double;
  double* base;
  int nv;
  template <int VEC>
  __device__ __forceinline__ void fill(const float* __restrict__ q, int ub, int c0, int tid,
                                       int nthreads) {
    for (int idx = tid; idx < nv * VEC; idx += nthreads) {
      const int col = ub * VEC + idx;
      const double v = col >= c0 ? static_cast<double>(q[col - c0]) : 0.0;
      const int unit = idx / VEC, e = idx - unit * VEC;
      if constexpr (VEC % 2 == 0) base[((e / 2) * nv + unit) * 2 + (e % 2)] = v;
      else base[idx] = v;
    }
  }
  template <int VEC>
  __device__ __forceinline__ void get(int v, double (&q)[VEC]) const {
    if constexpr (VEC % 2 == 0) {
      typedef double f64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int j = 0; j < VEC / 2; ++j) {
        const f64x2 t = reinterpret_cast<const f64x2*>(base)[j * nv + v];
        q[2 * j + 0] = t.x;
        q[2 * j + 1] = t.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[e] = base[v * VEC + e];
    }
  }
};

// ---- cross-lane reductions -------------------------------------------------------------------
// Butterfly (xor) reductions: every lane ends with the same, bitwise identical result because
// each step adds the same two operands on both partners.

__device__ __forceinline__ double shfl_xor_f64(double v, int mask) { return __shfl_xor(v, mask, kWave); }

__device__ __forceinline__ double group_sum(double v, int group) {
  for (int o = group >> 1; o >= 1; o >>= 1) v += shfl_xor_f64(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_f64(v, o);
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, shfl_xor_f64(v, o));
  return v;
}

// ---- DPP reductions ----------------------------------------------------------------------------
// Cross-lane data movement through the DPP modifier of VALU moves: no LDS crossbar, a few
// cycles per step. A float64 moves as its two 32-bit halves. `OLD` is what lanes of disabled
// rows keep.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double v, double old) {
  const int64_t b = __double_as_longlong(v);
  const int64_t o = __double_as_longlong(old);
  const int lo = __builtin_amdgcn_update_dpp(static_cast<int>(o), static_cast<int>(b), CTRL,
                                             ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(static_cast<int>(o >> 32), static_cast<int>(b >> 32),
                                             CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// dpp_f64 for patterns that give every lane a source lane inside its own row (quad permutes,
// row rotations and mirrors) with all rows enabled: no lane keeps an old value, so none is
// set up (two moves fewer per step).
template <int CTRL>
__device__ __forceinline__ double dpp_f64_all(double v) {
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each row of 16
constexpr int kDppBcast15 = 0x142;     // lane 15 of each row -> the next row
constexpr int kDppBcast31 = 0x143;     // lane 31 -> rows 2 and 3

// Sum over the 64 lanes, returned wave-uniform. The order of the additions is fixed, so the
// result is reproducible; it is the value that accumulates in lane 63.
__device__ __forceinline__ double wave_sum_dpp(double v) {
  v += dpp_f64_all<kDppXor1>(v);
  v += dpp_f64_all<kDppXor2>(v);
  v += dpp_f64_all<kDppHalfMirror>(v);
  v += dpp_f64_all<kDppMirror>(v);
  v += dpp_f64<kDppBcast15, 0xa>(v, 0.0);
  v += dpp_f64<kDppBcast31, 0xc>(v, 0.0);
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// N independent sums reduced together: the DPP chains interleave, so their latencies
// overlap. Each result is wave-uniform and added in the same fixed order as wave_sum_dpp.
template <int N>
__device__ __forceinline__ void wave_sums_dpp(double (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppXor1>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppXor2>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppHalfMirror>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppMirror>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f64<kDppBcast15, 0xa>(v[k], 0.0);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f64<kDppBcast31, 0xc>(v[k], 0.0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int64_t b = __double_as_longlong(v[k]);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
    v[k] = __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
  }
}

// N sums over lanes [0, gp) (gp a power of two in [1, 64], wave-uniform), each returned
// wave-uniform. Lanes from gp up are not read, and every lane must hold its own value.
template <int N>
__device__ __forceinline__ void lanes_sums_dpp(double (&v)[N], int gp) {
  if (gp >= 2) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppXor1>(v[k]);
  }
  if (gp >= 4) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppXor2>(v[k]);
  }
  if (gp >= 8) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppHalfMirror>(v[k]);
  }
  if (gp >= 16) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_f64_all<kDppMirror>(v[k]);
  }
  if (gp >= 32) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_f64<kDppBcast15, 0xa>(v[k], 0.0);
  }
  if (gp >= 64) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += dpp_f64<kDppBcast31, 0xc>(v[k], 0.0);
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int64_t b = __double_as_longlong(v[k]);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), gp - 1);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), gp - 1);
    v[k] = __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
  }
}

// Maximum over the 64 lanes, wave-uniform (NaN lanes are ignored, as by fmax).
__device__ __forceinline__ double wave_max_dpp(double v) {
  v = fmax(v, dpp_f64_all<kDppXor1>(v));
  v = fmax(v, dpp_f64_all<kDppXor2>(v));
  v = fmax(v, dpp_f64_all<kDppHalfMirror>(v));
  v = fmax(v, dpp_f64_all<kDppMirror>(v));
  v = fmax(v, dpp_f64<kDppBcast15, 0xa>(v, v));
  v = fmax(v, dpp_f64<kDppBcast31, 0xc>(v, v));
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// Value of a float held in lane `lane` (lane must be wave-uniform).
__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ double lane_f64(double v, int lane) {
  const int64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<int64_t>(hi) << 32) | static_cast<uint32_t>(lo));
}

// ---- key-slice geometry ----------------------------------------------------------------------

struct KeyGeom {
  int c0;      // first key column, d - r
  int ub;      // first unit touching the key
  int nur;     // units per row
  int group;   // lanes that cooperate on one source's key (a power of two <= 64)
  int per_it;  // sources handled per iteration of the key pass (64 / group)
};

template <int VEC>
__device__ __forceinline__ KeyGeom key_geom(int d, int r) {
  KeyGeom g;
  g.c0 = d - r;
  g.ub = g.c0 / VEC;
  g.nur = (d + VEC - 1) / VEC;
  const int nut = g.nur - g.ub;
  int G = 1;
  while (G < nut && G < kWave) G <<= 1;
  g.group = G;
  g.per_it = kWave / G;
  return g;
}

// The query value of key column `col` (>= c0), or 0 for a column outside the key.
__device__ __forceinline__ double q_at(const float* __restrict__ q, int col, int c0) {
  return col >= c0 ? static_cast<double>(q[col - c0]) : 0.0;
}

// How a one-wave-per-row kernel forms each source's key and its RMS.
enum RowKeyMode : int {
  kKeySlice = 0,    // the last r columns of the row, RMS over those r columns
  kKeyFullRms = 1,  // the last r columns of the row, RMS over the whole row (the control)
  kKeySeparate = 2  // the first r columns of the source's own key row, RMS over those
};

// Scores of the n sources of one row. On return lane i (< n) holds z_i and rho_i of source i;
// other lanes hold unspecified values. float64 throughout: each bf16 x fp32 product is exact in
// float64, so the only rounding is in the sums. The lanes are cut into groups, one source per
// group per iteration; a group walks its source's key units (KM = kKeySlice), every unit of the
// row (kKeyFullRms: the square sum covers the row, the dot product the key columns), or the
// elements of the source's key row K->ptr[i] (kKeySeparate: single elements, so key rows need
// no alignment).
template <typename IO, int VEC, int KM = kKeySlice>
__device__ __forceinline__ void row_scores(const SrcList& S, int n, int64_t row, int d, int r,
                                           double eps, const float* __restrict__ q, int lane,
                                           double& z_mine, double& rho_mine,
                                           const SrcList* K = nullptr) {
  const KeyGeom g = key_geom<VEC>(d, r);
  // the range each group walks, in units of VEC elements (single elements for separate keys)
  const int w_begin = KM == kKeySlice ? g.ub : 0;
  const int w_end = KM == kKeySeparate ? r : g.nur;
  int group = 1;
  while (group < w_end - w_begin && group < kWave) group <<= 1;
  const int per_it = kWave / group;
  const int slot = lane / group;
  const int sub = lane % group;
  const int iters = (n + per_it - 1) / per_it;
  const int nrm = KM == kKeyFullRms ? d : r;
  z_mine = 0.0;
  rho_mine = 1.0;
  for (int it = 0; it < iters; ++it) {
    // The source of this lane's group; the pointer table is indexed with a uniform index
    // per candidate and selected per lane, so the table stays in scalar registers.
    const int i = it * per_it + slot;
    const IO* base = nullptr;
    int64_t ld = 0;
    for (int c = 0; c < per_it; ++c) {
      const int ic = it * per_it + c;
      if (ic < n && c == slot) {
        if constexpr (KM == kKeySeparate) {
          base = static_cast<const IO*>(K->ptr[ic]);
          ld = K->ld[ic];
        } else {
          base = static_cast<const IO*>(S.ptr[ic]);
          ld = S.ld[ic];
        }
      }
    }
    double dot = 0.0, ss = 0.0;
    if (i < n) {
      const IO* rowp = base + row * ld;
      if constexpr (KM == kKeySeparate) {
        for (int j = w_begin + sub; j < w_end; j += group) {
          const double k = static_cast<double>(to_f32<IO>(rowp[j]));
          dot = fma(static_cast<double>(q[j]), k, dot);
          ss = fma(k, k, ss);
        }
      } else {
        for (int u = w_begin + sub; u < w_end; u += group) {
          Unit<IO, VEC> un;
          un.load_cached(rowp + u * VEC);
          float x[VEC];
          un.get(x);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const int col = u * VEC + e;
            const double v = static_cast<double>(x[e]);
            const double k = (col >= g.c0) ? v : 0.0;
            dot = fma(q_at(q, col, g.c0), k, dot);
            // the control's RMS covers every column of the row, the slice RMS the key alone
            ss = KM == kKeyFullRms ? fma(v, v, ss) : fma(k, k, ss);
          }
        }
      }
    }
    dot = group_sum(dot, group);
    ss = group_sum(ss, group);
    const double rho = sqrt(ss / nrm + eps);
    const double z = dot / rho;
    const int src_lane = (lane % per_it) * group;
    const double zt = __shfl(z, src_lane, kWave);
    const double rt = __shfl(rho, src_lane, kWave);
    if (lane / per_it == it) {
      z_mine = zt;
      rho_mine = rt;
    }
  }
}

}  // namespace lrar
