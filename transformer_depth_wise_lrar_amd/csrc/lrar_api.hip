// The C-ABI entry points of liblrattnres: argument validation, path selection and launch.
// Every check runs before any device work; nothing here allocates, frees or synchronises.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/lrattnres.h"
#include "lrar_device.h"
#include "lrar_launch.h"

// Device scratch of lrar_backward_noalloc: the query-gradient partials, for callers that cannot
// allocate. Each GPU the library runs on holds its own copy until the process ends; host code
// never uses this name as an address (it is a host-side stand-in), only the per-device address
// that hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

namespace {

thread_local std::string g_last_error;

lrar_status fail(lrar_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lrar_status fail(lrar_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

lrar_status device_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return LRAR_OK;
  return fail(LRAR_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(lrar_dtype t) { return t == LRAR_BF16 ? 2 : 4; }

// Elements per 16-byte unit, or 0 for an unknown type.
int vec_of(lrar_dtype t) { return t == LRAR_BF16 ? 8 : (t == LRAR_F32 ? 4 : 0); }

bool dtype_ok(lrar_dtype t) { return t == LRAR_BF16 || t == LRAR_F32; }

lrar_status check_shape(const char* fn, int64_t T, int32_t d, int32_t r, double eps,
                        lrar_dtype io) {
  if (T < 0) return fail(LRAR_ERR_INVALID, "%s: T = %lld < 0", fn, (long long)T);
  if (d < 1) return fail(LRAR_ERR_INVALID, "%s: d = %d < 1", fn, d);
  if (r < 1 || r > d) return fail(LRAR_ERR_INVALID, "%s: r = %d outside [1, d = %d]", fn, r, d);
  if (!(eps >= 0.0) || !std::isfinite(eps))
    return fail(LRAR_ERR_INVALID, "%s: eps = %g must be finite and >= 0", fn, eps);
  if (!dtype_ok(io)) return fail(LRAR_ERR_INVALID, "%s: unknown io dtype %d", fn, (int)io);
  return LRAR_OK;
}

// The read kernels address a tile's rows through 32-bit byte offsets from the tile's first
// row (at most 4 rows, under 2^31 bytes), so a row stride may not exceed 256 MiB.
constexpr int64_t kMaxRowBytes = int64_t(1) << 28;
bool stride_ok(int64_t ld, size_t es) { return ld <= kMaxRowBytes / static_cast<int64_t>(es); }
lrar_status stride_fail(const char* fn, const char* what, int64_t ld) {
  return fail(LRAR_ERR_UNSUPPORTED, "%s: %s = %lld elements is a row stride above 256 MiB",
              fn, what, (long long)ld);
}

// Fills the source table; also reports whether every row start is 16-byte aligned.
lrar_status check_sources(const char* fn, int64_t T, int32_t d, lrar_dtype io, int32_t n,
                          int32_t n_min, const void* const* src, const int64_t* src_ld,
                          lrar::SrcList& S, bool& vec_ok) {
  if (n < n_min || n > LRAR_MAX_SOURCES)
    return fail(LRAR_ERR_INVALID, "%s: n = %d outside [%d, %d]", fn, n, n_min, LRAR_MAX_SOURCES);
  std::memset(&S, 0, sizeof(S));
  if (n == 0) return LRAR_OK;
  if (src == nullptr || src_ld == nullptr)
    return fail(LRAR_ERR_INVALID, "%s: null source table", fn);
  const int vec = vec_of(io);
  for (int i = 0; i < n; ++i) {
    if (src[i] == nullptr && T > 0) return fail(LRAR_ERR_INVALID, "%s: src[%d] is null", fn, i);
    if (src_ld[i] < d)
      return fail(LRAR_ERR_INVALID, "%s: src_ld[%d] = %lld < d = %d", fn, i, (long long)src_ld[i], d);
    if (!stride_ok(src_ld[i], esize(io))) return stride_fail(fn, "src_ld", src_ld[i]);
    S.ptr[i] = src[i];
    S.ld[i] = src_ld[i];
    if (!aligned16(src[i]) || (src_ld[i] % vec) != 0) vec_ok = false;
  }
  if (d % vec != 0) vec_ok = false;
  return LRAR_OK;
}

// ---- aliasing --------------------------------------------------------------------------------
// A buffer an entry point touches, as `rows` rows of `width` bytes every `ld` bytes from `base`
// (a plain span is one row). Outputs may overlap no other buffer of the call; inputs may overlap
// each other (repeated or strided sources are legal).
struct Region {
  uintptr_t base;
  int64_t rows, ld, width;
  const char* name;
  int index;     // for tables of buffers (-1 for a single buffer)
  // An output and an input that both carry this flag may be the same buffer (same start, row
  // stride and shape): an in-place update.
  bool inplace;
};

Region rows_region(const void* p, int64_t T, int64_t ld, int64_t d, size_t es, const char* name,
                   int index = -1) {
  Region g{reinterpret_cast<uintptr_t>(p), p == nullptr ? 0 : T, ld * static_cast<int64_t>(es),
           d * static_cast<int64_t>(es), name, index, false};
  return g;
}

Region span_region(const void* p, int64_t bytes, const char* name, int index = -1) {
  Region g{reinterpret_cast<uintptr_t>(p), (p == nullptr || bytes <= 0) ? 0 : 1, bytes, bytes,
           name, index, false};
  return g;
}

int64_t floor_div(int64_t a, int64_t b) {  // b > 0
  const int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

// Whether two regions share a byte: exact when both use one row stride (or one is a span),
// else by their bounding ranges.
bool regions_overlap(Region a, Region b) {
  if (a.rows <= 0 || b.rows <= 0 || a.width <= 0 || b.width <= 0) return false;
  const auto end = [](const Region& g) {
    return g.base + static_cast<uintptr_t>((g.rows - 1) * g.ld + g.width);
  };
  if (end(a) <= b.base || end(b) <= a.base) return false;
  if (a.rows == 1) a.ld = b.ld;
  if (b.rows == 1) b.ld = a.ld;
  if (a.ld != b.ld || a.width > a.ld || b.width > b.ld) return true;
  // row i of a meets row j of b iff -wb < delta + (j - i) L < wa, delta = b.base - a.base
  const int64_t L = a.ld;
  const int64_t delta = static_cast<int64_t>(b.base - a.base);
  const int64_t k_lo = floor_div(-b.width - delta, L) + 1;
  const int64_t k_hi = -floor_div(-(a.width - delta), L) - 1;  // ceil((wa - delta) / L) - 1
  const int64_t lo = k_lo > -(a.rows - 1) ? k_lo : -(a.rows - 1);
  const int64_t hi = k_hi < b.rows - 1 ? k_hi : b.rows - 1;
  return lo <= hi;
}

constexpr int kMaxRegions = 4 * LRAR_MAX_SOURCES + 16;

struct Regions {
  Region in[kMaxRegions];
  Region out[kMaxRegions / 2];
  int n_in = 0, n_out = 0;
  void input(const Region& g) {
    if (n_in < kMaxRegions) in[n_in++] = g;
  }
  void output(const Region& g) {
    if (n_out < kMaxRegions / 2) out[n_out++] = g;
  }
};

void region_label(const Region& g, char* buf, size_t len) {
  if (g.index >= 0) snprintf(buf, len, "%s[%d]", g.name, g.index);
  else snprintf(buf, len, "%s", g.name);
}

// Every output against every input and every other output.
lrar_status check_disjoint(const char* fn, const Regions& R) {
  char a[48], b[48];
  for (int i = 0; i < R.n_out; ++i) {
    const Region& w = R.out[i];
    for (int j = 0; j < R.n_in; ++j) {
      const Region& x = R.in[j];
      const bool same = w.base == x.base && w.ld == x.ld && w.width == x.width && w.rows == x.rows;
      if (same && x.inplace && w.inplace) continue;
      if (regions_overlap(w, x)) {
        region_label(w, a, sizeof(a));
        region_label(x, b, sizeof(b));
        return fail(LRAR_ERR_INVALID, "%s: %s overlaps %s", fn, a, b);
      }
    }
    for (int j = 0; j < i; ++j) {
      if (regions_overlap(w, R.out[j])) {
        region_label(w, a, sizeof(a));
        region_label(R.out[j], b, sizeof(b));
        return fail(LRAR_ERR_INVALID, "%s: %s overlaps %s", fn, a, b);
      }
    }
  }
  return LRAR_OK;
}

void add_sources(Regions& R, const lrar::SrcList& S, int n, int64_t T, int64_t d, size_t es,
                 const char* name) {
  for (int i = 0; i < n; ++i) R.input(rows_region(S.ptr[i], T, S.ld[i], d, es, name, i));
}

// Checks the arguments every forward read shares and fills the parameter block; use_vec is
// the unit width the sources and out allow (16-byte units, or single elements).
lrar_status check_read(const char* fn, int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                       int32_t n, const void* const* src, const int64_t* src_ld, const float* q,
                       void* out, int64_t out_ld, float* alpha, int64_t alpha_ld,
                       lrar::ReadParams& p, int& use_vec) {
  lrar_status st = check_shape(fn, T, d, r, eps, io);
  if (st != LRAR_OK) return st;
  std::memset(&p, 0, sizeof(p));
  bool vec_ok = true;
  st = check_sources(fn, T, d, io, n, 1, src, src_ld, p.src, vec_ok);
  if (st != LRAR_OK) return st;
  if (q == nullptr && T > 0) return fail(LRAR_ERR_INVALID, "%s: q is null", fn);
  if (out == nullptr && T > 0) return fail(LRAR_ERR_INVALID, "%s: out is null", fn);
  if (out_ld < d) return fail(LRAR_ERR_INVALID, "%s: out_ld = %lld < d", fn, (long long)out_ld);
  if (alpha != nullptr && alpha_ld < n)
    return fail(LRAR_ERR_INVALID, "%s: alpha_ld = %lld < n = %d", fn, (long long)alpha_ld, n);
  const int vec = vec_of(io);
  if (!aligned16(out) || out_ld % vec != 0) vec_ok = false;
  use_vec = vec_ok ? vec : 1;
  p.n = n;
  p.d = d;
  p.r = r;
  p.T = T;
  p.eps = eps;
  p.q = q;
  p.out = out;
  p.out_ld = out_ld;
  p.alpha = alpha;
  p.alpha_ld = alpha_ld;
  return LRAR_OK;
}

// The buffers of a forward read: the sources and q read, out and alpha written.
void read_regions(Regions& R, const lrar::ReadParams& p, lrar_dtype io) {
  add_sources(R, p.src, p.n, p.T, p.d, esize(io), "src");
  R.input(span_region(p.q, static_cast<int64_t>(p.r) * 4, "q"));
  R.output(rows_region(p.out, p.T, p.out_ld, p.d, esize(io), "out"));
  if (p.alpha != nullptr) R.output(rows_region(p.alpha, p.T, p.alpha_ld, p.n, 4, "alpha"));
}

// A row fits a register tile when it has at most tile_max_chunks() chunks of 64 units.
bool row_fits_tile(int32_t d, int use_vec) {
  const int nur = (d + use_vec - 1) / use_vec;
  return (nur + lrar::kWave - 1) / lrar::kWave <= lrar::tile_max_chunks();
}

}  // namespace

namespace {

// lrar_forward, and with saved != nullptr lrar_forward_save.
lrar_status forward_impl(const char* fn, int64_t T, int32_t d, int32_t r, double eps,
                         lrar_dtype io, int32_t n, const void* const* src, const int64_t* src_ld,
                         const float* q, void* out, int64_t out_ld, float* alpha,
                         int64_t alpha_ld, double* saved, int64_t saved_ld, int32_t variant,
                         void* stream) {
  lrar::ReadParams p;
  int use_vec = 1;
  lrar_status st = check_read(fn, T, d, r, eps, io, n, src, src_ld, q, out, out_ld, alpha,
                              alpha_ld, p, use_vec);
  if (st != LRAR_OK) return st;
  if (saved != nullptr && saved_ld < 2 * static_cast<int64_t>(n))
    return fail(LRAR_ERR_INVALID, "%s: saved_ld = %lld < 2 n = %d", fn, (long long)saved_ld,
                2 * n);
  p.saved = saved;
  p.saved_ld = saved_ld;
  if (variant < LRAR_VARIANT_AUTO || variant > LRAR_VARIANT_ONLINE)
    return fail(LRAR_ERR_INVALID, "%s: unknown variant %d", fn, variant);
  const bool tile_fits = row_fits_tile(d, use_vec);
  lrar::ReadKind kind;
  if (variant == LRAR_VARIANT_ONLINE) {
    if (!tile_fits)
      return fail(LRAR_ERR_UNSUPPORTED, "%s: the online variant holds a whole row in registers; "
                  "d = %d is too wide on this path", fn, d);
    kind = lrar::ReadKind::kOnline;
  } else if (variant == LRAR_VARIANT_TWO_PASS) {
    kind = lrar::ReadKind::kTwoPass;
  } else {
    // Reading every byte once (online) is the cheapest whenever the row fits a tile.
    kind = tile_fits ? lrar::ReadKind::kOnline : lrar::ReadKind::kTwoPass;
  }
  if (T == 0) return LRAR_OK;
  Regions R;
  read_regions(R, p, io);
  if (saved != nullptr) R.output(rows_region(saved, T, saved_ld, 2 * n, 8, "saved"));
  st = check_disjoint(fn, R);
  if (st != LRAR_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = tile_fits ? lrar::launch_tile(p, kind, io == LRAR_BF16, use_vec, 0, hs)
                                 : lrar::launch_read(p, kind, io == LRAR_BF16, use_vec, 0, hs);
  return device_status(e, fn);
}

}  // namespace

extern "C" {

lrar_status lrar_forward(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io, int32_t n,
                         const void* const* src, const int64_t* src_ld, const float* q, void* out,
                         int64_t out_ld, float* alpha, int64_t alpha_ld, int32_t variant,
                         void* stream) {
  return forward_impl("lrar_forward", T, d, r, eps, io, n, src, src_ld, q, out, out_ld, alpha,
                      alpha_ld, nullptr, 0, variant, stream);
}

lrar_status lrar_forward_save(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                              int32_t n, const void* const* src, const int64_t* src_ld,
                              const float* q, void* out, int64_t out_ld, double* saved,
                              int64_t saved_ld, int32_t variant, void* stream) {
  if (saved == nullptr && T > 0)
    return fail(LRAR_ERR_INVALID, "lrar_forward_save: saved is null");
  return forward_impl("lrar_forward_save", T, d, r, eps, io, n, src, src_ld, q, out, out_ld,
                      nullptr, 0, saved, saved_ld, variant, stream);
}

lrar_status lrar_forward_fullrms(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                                 int32_t n, const void* const* src, const int64_t* src_ld,
                                 const float* q, void* out, int64_t out_ld, float* alpha,
                                 int64_t alpha_ld, void* stream) {
  const char* fn = "lrar_forward_fullrms";
  lrar::ReadParams p;
  int use_vec = 1;
  lrar_status st = check_read(fn, T, d, r, eps, io, n, src, src_ld, q, out, out_ld, alpha,
                              alpha_ld, p, use_vec);
  if (st != LRAR_OK) return st;
  if (T == 0) return LRAR_OK;
  Regions R;
  read_regions(R, p, io);
  st = check_disjoint(fn, R);
  if (st != LRAR_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // rows too wide for a register tile: key pass over the whole rows, then the values
  if (!row_fits_tile(d, use_vec))
    return device_status(lrar::launch_read(p, lrar::ReadKind::kTwoPass, io == LRAR_BF16, use_vec,
                                           0, hs, lrar::kKeyFullRms),
                         fn);
  return device_status(lrar::launch_tile_fullrms(p, io == LRAR_BF16, use_vec, hs), fn);
}

lrar_status lrar_forward_keys(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                              int32_t n, const void* const* src, const int64_t* src_ld,
                              const void* const* key, const int64_t* key_ld, const float* q,
                              void* out, int64_t out_ld, float* alpha, int64_t alpha_ld,
                              void* stream) {
  const char* fn = "lrar_forward_keys";
  lrar::ReadParams p;
  int use_vec = 1;
  lrar_status st = check_read(fn, T, d, r, eps, io, n, src, src_ld, q, out, out_ld, alpha,
                              alpha_ld, p, use_vec);
  if (st != LRAR_OK) return st;
  if (key == nullptr || key_ld == nullptr) return fail(LRAR_ERR_INVALID, "%s: null key table", fn);
  lrar::SrcList keys;
  std::memset(&keys, 0, sizeof(keys));
  // Largest power of two (up to 16 bytes) that every key row start is a multiple of.
  uintptr_t align = 16;
  for (int i = 0; i < n; ++i) {
    if (key[i] == nullptr && T > 0) return fail(LRAR_ERR_INVALID, "%s: key[%d] is null", fn, i);
    if (key_ld[i] < r)
      return fail(LRAR_ERR_INVALID, "%s: key_ld[%d] = %lld < r = %d", fn, i,
                  (long long)key_ld[i], r);
    if (!stride_ok(key_ld[i], esize(io))) return stride_fail(fn, "key_ld", key_ld[i]);
    const uintptr_t bits = reinterpret_cast<uintptr_t>(key[i]) |
                           static_cast<uintptr_t>(key_ld[i]) * esize(io);
    while (align > 1 && (bits & (align - 1)) != 0) align >>= 1;
    keys.ptr[i] = key[i];
    keys.ld[i] = key_ld[i];
  }
  if (T == 0) return LRAR_OK;
  Regions R;
  read_regions(R, p, io);
  for (int i = 0; i < n; ++i) R.input(rows_region(key[i], T, key_ld[i], r, esize(io), "key", i));
  st = check_disjoint(fn, R);
  if (st != LRAR_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  // One pass on register tiles when the row fits one and a spread key piece serves this key;
  // otherwise the key pass reads the key rows element by element, then the values.
  p.key_piece = row_fits_tile(d, use_vec)
                    ? lrar::tile_keys_piece(r, static_cast<int>(align),
                                            static_cast<int>(esize(io)), use_vec)
                    : 0;
  if (p.key_piece == 0)
    return device_status(lrar::launch_read(p, lrar::ReadKind::kTwoPass, io == LRAR_BF16, use_vec,
                                           0, hs, lrar::kKeySeparate, &keys),
                         fn);
  return device_status(lrar::launch_tile_keys(p, keys, io == LRAR_BF16, use_vec, hs), fn);
}

lrar_status lrar_forward_stats(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                               int32_t n, const void* const* src, const int64_t* src_ld,
                               int32_t nq, const float* q, int64_t q_ld, float* m, float* l,
                               int64_t ml_ld, void* acc, lrar_dtype acc_dtype, int64_t acc_ld,
                               int64_t acc_qstride, void* stream) {
  const char* fn = "lrar_forward_stats";
  lrar_status st = check_shape(fn, T, d, r, eps, io);
  if (st != LRAR_OK) return st;
  lrar::StatsParams p;
  std::memset(&p, 0, sizeof(p));
  bool vec_ok = true;
  st = check_sources(fn, T, d, io, n, 1, src, src_ld, p.src, vec_ok);
  if (st != LRAR_OK) return st;
  if (nq < 1 || nq > LRAR_MAX_QUERIES)
    return fail(LRAR_ERR_INVALID, "%s: nq = %d outside [1, %d]", fn, nq, LRAR_MAX_QUERIES);
  if (q_ld < r) return fail(LRAR_ERR_INVALID, "%s: q_ld = %lld < r", fn, (long long)q_ld);
  if (ml_ld < T) return fail(LRAR_ERR_INVALID, "%s: ml_ld = %lld < T", fn, (long long)ml_ld);
  if (!dtype_ok(acc_dtype)) return fail(LRAR_ERR_INVALID, "%s: unknown acc dtype", fn);
  if (acc_ld < d) return fail(LRAR_ERR_INVALID, "%s: acc_ld = %lld < d", fn, (long long)acc_ld);
  if (nq > 1 && acc_qstride < T * acc_ld)
    return fail(LRAR_ERR_INVALID, "%s: acc_qstride = %lld < T * acc_ld", fn, (long long)acc_qstride);
  if (T > 0 && (q == nullptr || m == nullptr || l == nullptr || acc == nullptr))
    return fail(LRAR_ERR_INVALID, "%s: null q, m, l or acc", fn);
  const int vec = vec_of(io);
  // acc units are VEC elements of acc_dtype; rows must start 16-byte aligned when acc is fp32
  // and units are 8 wide (two 16-byte halves), or whenever acc is written 16 bytes at a time.
  const int acc_elems_per_16 = acc_dtype == LRAR_BF16 ? 8 : 4;
  const bool acc_vec_needed = (esize(acc_dtype) * vec) % 16 == 0;
  if (acc_vec_needed &&
      (!aligned16(acc) || acc_ld % acc_elems_per_16 != 0 || acc_qstride % acc_elems_per_16 != 0))
    vec_ok = false;
  if (T == 0) return LRAR_OK;
  {
    Regions R;
    add_sources(R, p.src, n, T, d, esize(io), "src");
    R.input(rows_region(q, nq, q_ld, r, 4, "q"));
    R.output(rows_region(m, nq, ml_ld, T, 4, "m"));
    R.output(rows_region(l, nq, ml_ld, T, 4, "l"));
    // the accumulators as nq * T rows when the query blocks follow each other, else as one span
    if (nq == 1 || acc_qstride == T * acc_ld)
      R.output(rows_region(acc, nq * T, acc_ld, d, esize(acc_dtype), "acc"));
    else
      R.output(span_region(acc, ((nq - 1) * acc_qstride + (T - 1) * acc_ld + d) *
                                    static_cast<int64_t>(esize(acc_dtype)), "acc"));
    st = check_disjoint(fn, R);
    if (st != LRAR_OK) return st;
  }
  p.n = n;
  p.d = d;
  p.r = r;
  p.T = T;
  p.eps = eps;
  p.nq = nq;
  p.q = q;
  p.q_ld = q_ld;
  p.m = m;
  p.l = l;
  p.ml_ld = ml_ld;
  p.acc = acc;
  p.acc_ld = acc_ld;
  p.acc_qstride = acc_qstride;
  return device_status(lrar::launch_stats(p, io == LRAR_BF16, vec_ok ? vec : 1,
                                          acc_dtype == LRAR_BF16,
                                          static_cast<hipStream_t>(stream)),
                       fn);
}

lrar_status lrar_merge(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                       const float* m, const float* l, const void* acc, lrar_dtype acc_dtype,
                       int64_t acc_ld, int32_t n, const void* const* src, const int64_t* src_ld,
                       const float* q, void* out, int64_t out_ld, float* m_out, float* l_out,
                       void* stream) {
  const char* fn = "lrar_merge";
  lrar_status st = check_shape(fn, T, d, r, eps, io);
  if (st != LRAR_OK) return st;
  lrar::ReadParams p;
  std::memset(&p, 0, sizeof(p));
  bool vec_ok = true;
  st = check_sources(fn, T, d, io, n, 0, src, src_ld, p.src, vec_ok);
  if (st != LRAR_OK) return st;
  if (!dtype_ok(acc_dtype)) return fail(LRAR_ERR_INVALID, "%s: unknown acc dtype", fn);
  if (acc_ld < d) return fail(LRAR_ERR_INVALID, "%s: acc_ld = %lld < d", fn, (long long)acc_ld);
  if (!stride_ok(acc_ld, esize(acc_dtype))) return stride_fail(fn, "acc_ld", acc_ld);
  if (T > 0 && (m == nullptr || l == nullptr || acc == nullptr || out == nullptr))
    return fail(LRAR_ERR_INVALID, "%s: null m, l, acc or out", fn);
  if (T > 0 && n > 0 && q == nullptr) return fail(LRAR_ERR_INVALID, "%s: q is null", fn);
  if (out_ld < d) return fail(LRAR_ERR_INVALID, "%s: out_ld = %lld < d", fn, (long long)out_ld);
  const int vec = vec_of(io);
  if (!aligned16(out) || out_ld % vec != 0) vec_ok = false;
  const int acc_elems_per_16 = acc_dtype == LRAR_BF16 ? 8 : 4;
  if ((esize(acc_dtype) * vec) % 16 == 0 && (!aligned16(acc) || acc_ld % acc_elems_per_16 != 0))
    vec_ok = false;
  if (T == 0) return LRAR_OK;
  {
    Regions R;
    add_sources(R, p.src, n, T, d, esize(io), "src");
    if (n > 0) R.input(span_region(q, static_cast<int64_t>(r) * 4, "q"));
    R.input(span_region(m, T * 4, "m"));
    R.input(span_region(l, T * 4, "l"));
    R.input(rows_region(acc, T, acc_ld, d, esize(acc_dtype), "acc"));
    R.output(rows_region(out, T, out_ld, d, esize(io), "out"));
    R.output(span_region(m_out, T * 4, "m_out"));
    R.output(span_region(l_out, T * 4, "l_out"));
    st = check_disjoint(fn, R);
    if (st != LRAR_OK) return st;
  }
  p.n = n;
  p.d = d;
  p.r = r;
  p.T = T;
  p.eps = eps;
  p.q = q;
  p.out = out;
  p.out_ld = out_ld;
  p.m_in = m;
  p.l_in = l;
  p.acc = acc;
  p.acc_ld = acc_ld;
  p.m_out = m_out;
  p.l_out = l_out;
  const int use_vec = vec_ok ? vec : 1;
  const int nur = (d + use_vec - 1) / use_vec;
  const bool tile_fits = (nur + lrar::kWave - 1) / lrar::kWave <= lrar::tile_max_chunks();
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e =
      tile_fits ? lrar::launch_tile(p, lrar::ReadKind::kMerge, io == LRAR_BF16, use_vec,
                                    acc_dtype == LRAR_BF16, hs)
                : lrar::launch_read(p, lrar::ReadKind::kMerge, io == LRAR_BF16, use_vec,
                                    acc_dtype == LRAR_BF16, hs);
  return device_status(e, fn);
}

size_t lrar_backward_workspace_size(int64_t T, int32_t d, int32_t r, int32_t n) {
  (void)d;
  (void)n;
  if (T <= 0 || r < 1) return 0;
  return lrar::backward_workspace(T, r);
}

lrar_status lrar_merge_accumulate(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                                  const float* m, const float* l, const void* acc,
                                  lrar_dtype acc_dtype, int64_t acc_ld, const void* b,
                                  int64_t b_ld, const void* o, int64_t o_ld, void* b_out,
                                  int64_t b_out_ld, const float* q, void* out, int64_t out_ld,
                                  float* m_out, float* l_out, void* stream) {
  const char* fn = "lrar_merge_accumulate";
  lrar_status st = check_shape(fn, T, d, r, eps, io);
  if (st != LRAR_OK) return st;
  if (!dtype_ok(acc_dtype)) return fail(LRAR_ERR_INVALID, "%s: unknown acc dtype", fn);
  if (acc_ld < d) return fail(LRAR_ERR_INVALID, "%s: acc_ld = %lld < d", fn, (long long)acc_ld);
  if (o_ld < d) return fail(LRAR_ERR_INVALID, "%s: o_ld = %lld < d", fn, (long long)o_ld);
  if (b != nullptr && b_ld < d)
    return fail(LRAR_ERR_INVALID, "%s: b_ld = %lld < d", fn, (long long)b_ld);
  if (b_out_ld < d)
    return fail(LRAR_ERR_INVALID, "%s: b_out_ld = %lld < d", fn, (long long)b_out_ld);
  if (!stride_ok(acc_ld, esize(acc_dtype))) return stride_fail(fn, "acc_ld", acc_ld);
  if (!stride_ok(o_ld, esize(io))) return stride_fail(fn, "o_ld", o_ld);
  if (b != nullptr && !stride_ok(b_ld, esize(io))) return stride_fail(fn, "b_ld", b_ld);
  if (out_ld < d) return fail(LRAR_ERR_INVALID, "%s: out_ld = %lld < d", fn, (long long)out_ld);
  if (T > 0 && (m == nullptr || l == nullptr || acc == nullptr || o == nullptr ||
                b_out == nullptr || q == nullptr || out == nullptr))
    return fail(LRAR_ERR_INVALID, "%s: null m, l, acc, o, b_out, q or out", fn);
  if (m_out != nullptr && m_out == l_out)
    return fail(LRAR_ERR_INVALID, "%s: m_out and l_out alias", fn);
  const int vec = vec_of(io);
  bool vec_ok = d % vec == 0;
  for (const auto& [ptr, ld] : {std::pair<const void*, int64_t>{o, o_ld}, {b, b_ld},
                                {b_out, b_out_ld}, {out, out_ld}})
    if (ptr != nullptr && (!aligned16(ptr) || ld % vec != 0)) vec_ok = false;
  const int acc_elems_per_16 = acc_dtype == LRAR_BF16 ? 8 : 4;
  if ((esize(acc_dtype) * vec) % 16 == 0 && (!aligned16(acc) || acc_ld % acc_elems_per_16 != 0))
    vec_ok = false;
  const int use_vec = vec_ok ? vec : 1;
  if (T == 0) return LRAR_OK;
  {
    // b_out may replace b or o in place (same start and row stride) but overlap nothing else
    const size_t es = esize(io);
    Regions R;
    Region rb = rows_region(b, T, b_ld, d, es, "b");
    Region ro = rows_region(o, T, o_ld, d, es, "o");
    rb.inplace = ro.inplace = true;
    R.input(rb);
    R.input(ro);
    R.input(span_region(q, static_cast<int64_t>(r) * 4, "q"));
    R.input(span_region(m, T * 4, "m"));
    R.input(span_region(l, T * 4, "l"));
    R.input(rows_region(acc, T, acc_ld, d, esize(acc_dtype), "acc"));
    Region rbo = rows_region(b_out, T, b_out_ld, d, es, "b_out");
    rbo.inplace = true;
    R.output(rbo);
    R.output(rows_region(out, T, out_ld, d, es, "out"));
    R.output(span_region(m_out, T * 4, "m_out"));
    R.output(span_region(l_out, T * 4, "l_out"));
    lrar_status st2 = check_disjoint(fn, R);
    if (st2 != LRAR_OK) return st2;
  }
  lrar::ReadParams p;
  std::memset(&p, 0, sizeof(p));
  p.src.ptr[0] = o;
  p.src.ld[0] = o_ld;
  p.n = 1;
  p.d = d;
  p.r = r;
  p.T = T;
  p.eps = eps;
  p.q = q;
  p.out = out;
  p.out_ld = out_ld;
  p.m_in = m;
  p.l_in = l;
  p.acc = acc;
  p.acc_ld = acc_ld;
  p.m_out = m_out;
  p.l_out = l_out;
  p.b_prev = b;
  p.b_prev_ld = b_ld;
  p.b_out = b_out;
  p.b_out_ld = b_out_ld;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!row_fits_tile(d, use_vec)) {
    // rows too wide for a register tile: b_out = b + o first, then the merge reads b_out
    hipError_t e = lrar::launch_add_rows(b, b_ld, o, o_ld, b_out, b_out_ld, T, d, io == LRAR_BF16,
                                         use_vec, hs);
    if (e == hipSuccess) {
      p.src.ptr[0] = b_out;
      p.src.ld[0] = b_out_ld;
      e = lrar::launch_read(p, lrar::ReadKind::kMerge, io == LRAR_BF16, use_vec,
                            acc_dtype == LRAR_BF16, hs);
    }
    return device_status(e, fn);
  }
  return device_status(lrar::launch_tile(p, lrar::ReadKind::kMergeAccumulate, io == LRAR_BF16,
                                         use_vec, acc_dtype == LRAR_BF16, hs),
                       fn);
}

}  // extern "C"

namespace {

// The backward with gradients (dout, dsrc) of type grad; shared by both entry points.
// The no-allocation backward's scratch: at most kScratchBytes of dq partials. The workspace
// entry point's grid is kept when its rows fit; otherwise fewer workgroups (at least
// kScratchMinGrid, or as many as the rows need) share the rows.
constexpr int kScratchMinGrid = 256;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the calling thread's current device's copy of `scratch`, looked up once per device.
lrar_status device_scratch(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LRAR_ERR_UNSUPPORTED, "%s: device %d beyond the %d the scratch table covers", fn,
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, fn);
    if (ptr == nullptr) return fail(LRAR_ERR_DEVICE, "%s: no scratch address on device %d", fn, dev);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LRAR_OK;
}

// workspace == nullptr with use_scratch: the partials go to the device scratch.
lrar_status backward_impl(const char* fn, int64_t T, int32_t d, int32_t r, double eps,
                          lrar_dtype io, int32_t n, const void* const* src,
                          const int64_t* src_ld, const float* q, lrar_dtype grad,
                          const void* dout, int64_t dout_ld, void* const* dsrc,
                          const int64_t* dsrc_ld, int32_t accumulate, float* dq, void* workspace,
                          size_t workspace_bytes, void* stream, bool use_scratch = false,
                          const double* saved = nullptr, int64_t saved_ld = 0) {
  lrar_status st = check_shape(fn, T, d, r, eps, io);
  if (st != LRAR_OK) return st;
  if (!dtype_ok(grad)) return fail(LRAR_ERR_INVALID, "%s: unknown gradient dtype %d", fn, (int)grad);
  // a gradient row's 16-byte units must start 16-byte aligned on the vector path
  const int64_t grad_per_16 = 16 / static_cast<int64_t>(esize(grad));
  lrar::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  bool vec_ok = true;
  st = check_sources(fn, T, d, io, n, 1, src, src_ld, p.src, vec_ok);
  if (st != LRAR_OK) return st;
  if (accumulate != 0 && accumulate != 1)
    return fail(LRAR_ERR_INVALID, "%s: accumulate must be 0 or 1", fn);
  if (saved != nullptr && saved_ld < 2 * static_cast<int64_t>(n))
    return fail(LRAR_ERR_INVALID, "%s: saved_ld = %lld < 2 n = %d", fn, (long long)saved_ld,
                2 * n);
  if (dout_ld < d) return fail(LRAR_ERR_INVALID, "%s: dout_ld = %lld < d", fn, (long long)dout_ld);
  if (dsrc == nullptr || dsrc_ld == nullptr) return fail(LRAR_ERR_INVALID, "%s: null dsrc table", fn);
  if (T > 0 && (q == nullptr || dout == nullptr || dq == nullptr))
    return fail(LRAR_ERR_INVALID, "%s: null q, dout or dq", fn);
  const int vec = vec_of(io);
  if (!aligned16(dout) || dout_ld % grad_per_16 != 0) vec_ok = false;
  for (int i = 0; i < n; ++i) {
    if (dsrc[i] == nullptr && T > 0) return fail(LRAR_ERR_INVALID, "%s: dsrc[%d] is null", fn, i);
    if (dsrc_ld[i] < d)
      return fail(LRAR_ERR_INVALID, "%s: dsrc_ld[%d] = %lld < d", fn, i, (long long)dsrc_ld[i]);
    if (!aligned16(dsrc[i]) || dsrc_ld[i] % grad_per_16 != 0) vec_ok = false;
    p.dsrc.ptr[i] = dsrc[i];
    p.dsrc.ld[i] = dsrc_ld[i];
  }
  const int use_vec = vec_ok ? vec : 1;
  if (!lrar::backward_supported(d, r, use_vec))
    return fail(LRAR_ERR_UNSUPPORTED, "%s: the key of r = %d columns at d = %d spans more "
                "chunks of 64 units than the %s path keeps query-gradient partials for", fn, r,
                d, use_vec > 1 ? "vector" : "scalar");
  size_t need = lrar::backward_workspace(T, r);
  int ws_grid = 0;
  if (use_scratch) {
    // the workspace entry point's grid when its rows fit the scratch, else fewer workgroups
    const int full = T > 0 ? lrar::backward_grid(T) : 0;
    const int64_t fit = static_cast<int64_t>(kScratchBytes / (sizeof(double) * r)) - 32;
    const int floor_grid = full < kScratchMinGrid ? full : kScratchMinGrid;
    if (T > 0 && fit < floor_grid)
      return fail(LRAR_ERR_UNSUPPORTED, "%s: r = %d needs more than the %zu bytes of scratch "
                  "(its query-gradient partials of %d workgroups at r = %d)", fn, r,
                  kScratchBytes, floor_grid, r);
    ws_grid = static_cast<int>(fit < full ? fit : full);
    need = T > 0 ? lrar::backward_workspace_rows(ws_grid, r) : 0;
  } else {
    if (T > 0 && (workspace == nullptr || workspace_bytes < need))
      return fail(LRAR_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace_bytes);
    if (T > 0 && (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
      return fail(LRAR_ERR_INVALID, "%s: workspace must be 8-byte aligned", fn);
  }
  if (T == 0) return LRAR_OK;
  {
    Regions R;
    add_sources(R, p.src, n, T, d, esize(io), "src");
    R.input(span_region(q, static_cast<int64_t>(r) * 4, "q"));
    R.input(rows_region(dout, T, dout_ld, d, esize(grad), "dout"));
    if (saved != nullptr) R.input(rows_region(saved, T, saved_ld, 2 * n, 8, "saved"));
    for (int i = 0; i < n; ++i)
      R.output(rows_region(dsrc[i], T, dsrc_ld[i], d, esize(grad), "dsrc", i));
    R.output(span_region(dq, static_cast<int64_t>(r) * 4, "dq"));
    if (!use_scratch) R.output(span_region(workspace, static_cast<int64_t>(need), "workspace"));
    st = check_disjoint(fn, R);
    if (st != LRAR_OK) return st;
  }
  if (use_scratch) {
    st = device_scratch(fn, &workspace);
    if (st != LRAR_OK) return st;
  }
  p.n = n;
  p.d = d;
  p.r = r;
  p.T = T;
  p.eps = eps;
  p.q = q;
  p.dout = dout;
  p.dout_ld = dout_ld;
  p.saved = saved;
  p.saved_ld = saved_ld;
  p.accumulate = accumulate;
  p.dq = dq;
  p.workspace = workspace;
  return device_status(lrar::launch_backward(p, io == LRAR_BF16, grad == LRAR_BF16, use_vec,
                                             static_cast<hipStream_t>(stream), ws_grid),
                       fn);
}

}  // namespace

extern "C" {

lrar_status lrar_backward(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io, int32_t n,
                          const void* const* src, const int64_t* src_ld, const float* q,
                          const float* dout, int64_t dout_ld, float* const* dsrc,
                          const int64_t* dsrc_ld, int32_t accumulate, float* dq, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return backward_impl("lrar_backward", T, d, r, eps, io, n, src, src_ld, q, LRAR_F32, dout,
                       dout_ld, reinterpret_cast<void* const*>(dsrc), dsrc_ld, accumulate, dq,
                       workspace, workspace_bytes, stream);
}

lrar_status lrar_backward_grad(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                               int32_t n, const void* const* src, const int64_t* src_ld,
                               const float* q, lrar_dtype grad_dtype, const void* dout,
                               int64_t dout_ld, void* const* dsrc, const int64_t* dsrc_ld,
                               int32_t accumulate, float* dq, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return backward_impl("lrar_backward_grad", T, d, r, eps, io, n, src, src_ld, q, grad_dtype,
                       dout, dout_ld, dsrc, dsrc_ld, accumulate, dq, workspace, workspace_bytes,
                       stream);
}

lrar_status lrar_backward_saved(int64_t T, int32_t d, int32_t r, lrar_dtype io, int32_t n,
                                const void* const* src, const int64_t* src_ld, const float* q,
                                const double* saved, int64_t saved_ld, lrar_dtype grad_dtype,
                                const void* dout, int64_t dout_ld, void* const* dsrc,
                                const int64_t* dsrc_ld, int32_t accumulate, float* dq,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (saved == nullptr && T > 0)
    return fail(LRAR_ERR_INVALID, "lrar_backward_saved: saved is null");
  // eps only enters through the saved reciprocal RMS; 0 passes the shape check
  return backward_impl("lrar_backward_saved", T, d, r, 0.0, io, n, src, src_ld, q, grad_dtype,
                       dout, dout_ld, dsrc, dsrc_ld, accumulate, dq, workspace, workspace_bytes,
                       stream, false, saved, saved_ld);
}

lrar_status lrar_backward_noalloc(int64_t T, int32_t d, int32_t r, double eps, lrar_dtype io,
                                  int32_t n, const void* const* src, const int64_t* src_ld,
                                  const float* q, lrar_dtype grad_dtype, const void* dout,
                                  int64_t dout_ld, void* const* dsrc, const int64_t* dsrc_ld,
                                  int32_t accumulate, float* dq, void* stream) {
  return backward_impl("lrar_backward_noalloc", T, d, r, eps, io, n, src, src_ld, q, grad_dtype,
                       dout, dout_ld, dsrc, dsrc_ld, accumulate, dq, nullptr, 0, stream, true);
}

lrar_status lrar_copy(void* dst, const void* src, size_t bytes, void* stream) {
  const char* fn = "lrar_copy";
  if (bytes == 0) return LRAR_OK;
  if (dst == nullptr || src == nullptr) return fail(LRAR_ERR_INVALID, "%s: null pointer", fn);
  if (!aligned16(dst) || !aligned16(src) || bytes % 16 != 0)
    return fail(LRAR_ERR_INVALID, "%s: pointers and size must be 16-byte multiples", fn);
  const uintptr_t a = reinterpret_cast<uintptr_t>(dst), b = reinterpret_cast<uintptr_t>(src);
  if (a < b + bytes && b < a + bytes) return fail(LRAR_ERR_INVALID, "%s: buffers overlap", fn);
  return device_status(lrar::launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream)), fn);
}

size_t lrar_read_stream_sink_bytes(void) {
  return static_cast<size_t>(lrar::kCalibBlocks) * lrar::kBlock * sizeof(uint32_t);
}

lrar_status lrar_read_stream(const void* src, size_t bytes, void* sink, void* stream) {
  const char* fn = "lrar_read_stream";
  if (bytes == 0) return LRAR_OK;
  if (src == nullptr || sink == nullptr) return fail(LRAR_ERR_INVALID, "%s: null pointer", fn);
  if (!aligned16(src) || bytes % 16 != 0)
    return fail(LRAR_ERR_INVALID, "%s: src and size must be 16-byte multiples", fn);
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return fail(LRAR_ERR_INVALID, "%s: sink must be 4-byte aligned", fn);
  const uintptr_t a = reinterpret_cast<uintptr_t>(sink), b = reinterpret_cast<uintptr_t>(src);
  const size_t sb = lrar_read_stream_sink_bytes();
  if (a < b + bytes && b < a + sb) return fail(LRAR_ERR_INVALID, "%s: sink overlaps src", fn);
  return device_status(lrar::launch_read_stream(src, bytes, sink, static_cast<hipStream_t>(stream)),
                       fn);
}

lrar_status lrar_mix_stream(int64_t T, int32_t d, int32_t n, const void* const* src,
                            const int64_t* src_ld, int32_t nout, void* const* out,
                            const int64_t* out_ld, lrar_dtype out_dtype, int32_t waves_per_cu,
                            int32_t waves_per_row, int32_t depth, int32_t slots,
                            int32_t rows_per_wave, int32_t lockstep, void* stream) {
  const char* fn = "lrar_mix_stream";
  if (T < 0) return fail(LRAR_ERR_INVALID, "%s: T = %lld < 0", fn, (long long)T);
  if (d < 8 || d % 8 != 0)
    return fail(LRAR_ERR_INVALID, "%s: d = %d must be a positive multiple of 8", fn, d);
  if (waves_per_cu < 4 || waves_per_cu > 32 || waves_per_cu % 4 != 0)
    return fail(LRAR_ERR_INVALID, "%s: waves_per_cu = %d must be 4, 8, ..., 32", fn, waves_per_cu);
  if (waves_per_row != 1 && waves_per_row != 2 && waves_per_row != 4)
    return fail(LRAR_ERR_INVALID, "%s: waves_per_row = %d must be 1, 2 or 4", fn, waves_per_row);
  if (depth != 1 && depth != 2 && depth != 4)
    return fail(LRAR_ERR_INVALID, "%s: depth = %d must be 1, 2 or 4", fn, depth);
  if (slots != 2 && slots != 4 && slots != 8 && slots != 16)
    return fail(LRAR_ERR_INVALID, "%s: slots = %d must be 2, 4, 8 or 16", fn, slots);
  if (depth * slots > 16)
    return fail(LRAR_ERR_INVALID, "%s: depth x slots = %d exceeds 16 units a lane", fn,
                depth * slots);
  if (rows_per_wave < 0)
    return fail(LRAR_ERR_INVALID, "%s: rows_per_wave = %d < 0", fn, rows_per_wave);
  if (lockstep < 0 || lockstep > 2)
    return fail(LRAR_ERR_INVALID, "%s: lockstep = %d must be 0, 1 or 2", fn, lockstep);
  if (nout < 1 || nout > LRAR_MAX_SOURCES)
    return fail(LRAR_ERR_INVALID, "%s: nout = %d outside [1, %d]", fn, nout, LRAR_MAX_SOURCES);
  if (!dtype_ok(out_dtype)) return fail(LRAR_ERR_INVALID, "%s: unknown out dtype", fn);
  lrar::SrcList S;
  bool vec_ok = true;
  lrar_status st = check_sources(fn, T, d, LRAR_BF16, n, 1, src, src_ld, S, vec_ok);
  if (st != LRAR_OK) return st;
  if (T == 0) return LRAR_OK;
  if (out == nullptr || out_ld == nullptr)
    return fail(LRAR_ERR_INVALID, "%s: null out table", fn);
  const size_t oe = esize(out_dtype);
  const int64_t per16 = static_cast<int64_t>(16 / oe);
  lrar::DstList O;
  Regions R;
  add_sources(R, S, n, T, d, 2, "src");
  for (int j = 0; j < nout; ++j) {
    if (out[j] == nullptr) return fail(LRAR_ERR_INVALID, "%s: out[%d] is null", fn, j);
    if (out_ld[j] < d)
      return fail(LRAR_ERR_INVALID, "%s: out_ld[%d] = %lld < d", fn, j, (long long)out_ld[j]);
    if (!stride_ok(out_ld[j], oe)) return stride_fail(fn, "out_ld", out_ld[j]);
    if (!aligned16(out[j]) || out_ld[j] % per16 != 0) vec_ok = false;
    O.ptr[j] = out[j];
    O.ld[j] = out_ld[j];
    R.output(rows_region(out[j], T, out_ld[j], d, oe, "out", j));
  }
  if (!vec_ok)
    return fail(LRAR_ERR_INVALID,
                "%s: every row start must be 16-byte aligned (pointers, and strides in 16 bytes)",
                fn);
  st = check_disjoint(fn, R);
  if (st != LRAR_OK) return st;
  return device_status(lrar::launch_mix_stream(S, n, T, d, O, nout, out_dtype == LRAR_F32,
                                               waves_per_cu, waves_per_row, depth, slots,
                                               rows_per_wave, lockstep,
                                               static_cast<hipStream_t>(stream)),
                       fn);
}

const char* lrar_status_string(lrar_status s) {
  switch (s) {
    case LRAR_OK: return "ok";
    case LRAR_ERR_INVALID: return "invalid argument";
    case LRAR_ERR_UNSUPPORTED: return "unsupported shape or variant";
    case LRAR_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* lrar_last_error(void) { return g_last_error.c_str(); }

const char* lrar_version(void) { return "0.1.0"; }

}  // extern "C"

// ---- the calibration kernels --------------------------------------------------------------------
// Plain streams that set the bandwidth ceilings the read is measured against. Each lane keeps
// U independent 16-byte loads in flight, and the workgroups walk the buffer in one shared
// window (workgroup b takes the U * kBlock units from b * U * kBlock, then jumps by the grid):
// on MI355X a grid of 1024 workgroups with two (copy) or four (read) loads per lane measured
// fastest in a sweep of 1024-8192 workgroups and 1-8 loads per lane.

namespace lrar {

__global__ __launch_bounds__(kBlock) void k_copy(u32x4* __restrict__ dst,
                                                 const u32x4* __restrict__ src, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock * kCopyUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kBlock * kCopyUnroll + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) {
      const int64_t i = base + static_cast<int64_t>(k) * kBlock;
      v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) {
      const int64_t i = base + static_cast<int64_t>(k) * kBlock;
      if (i < n16) __builtin_nontemporal_store(v[k], dst + i);
    }
  }
}

// Reads n16 units and folds them into one 32-bit word per thread (written to sink, so the
// loads cannot be dropped): the traffic is the read alone, plus 4 bytes per thread.
__global__ __launch_bounds__(kBlock) void k_read_stream(const u32x4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock * kReadUnroll;
  uint32_t x = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kBlock * kReadUnroll + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) {
      const int64_t i = base + static_cast<int64_t>(k) * kBlock;
      v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  sink[static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x] = x;
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  int64_t blocks = (n16 + kBlock * kCopyUnroll - 1) / (kBlock * kCopyUnroll);
  if (blocks > kCalibBlocks) blocks = kCalibBlocks;
  hipLaunchKernelGGL(k_copy, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

// A kernel's traffic with next to no arithmetic: for the rows [r0, r1), the n bf16 source rows
// are read and their mean (float32 sums in source order) written to each of the nout output
// rows, as float32 (F32OUT) or rounded to nearest-even bf16. A row goes to wpr waves of one
// workgroup (1, 2 or 4; the row group g of the launch takes rows r0 + g + k * groups, as the
// read's tiles), which take its chunks of 64 16-byte units in turn, NU chunks a wave per
// pass (NU units a lane, chunk k * wpr + w of the pass to wave w of the row); DEPTH sources
// are loaded before any is added, and the loads are waited for together. One bf16 output is a
// read's traffic; more outputs, or float32 ones, give the write-heavy mixes of Phase 1 and the
// backward. lock = 1 or 2: the workgroup's waves
// meet at a barrier once per row or once per group of DEPTH sources, as the reads keep their
// waves in lockstep, in the steps where every wave of the workgroup has a row (a condition all
// of them compute alike, so they meet the same barriers).
template <int DEPTH, int NU, bool F32OUT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(NU >= 16 ? 2 : 1)))
void k_mix_stream(SrcList src, int n, int64_t r0, int64_t r1, int nur, DstList out, int nout,
                  float w, int wpr, int lock) {
  const int lane = threadIdx.x & (kWave - 1);
  // wpr divides the workgroup's 4 waves, so a row group never spans two workgroups
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_in_block();
  const int64_t group = wave / wpr;
  const int wr = static_cast<int>(wave % wpr);
  const int64_t groups = static_cast<int64_t>(gridDim.x) * (kWavesPerBlock / wpr);
  const int64_t last_group =
      (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + kWavesPerBlock - 1) / wpr;
  for (int64_t row = r0 + group; row < r1; row += groups) {
    const bool all_rows = (row - group) + last_group < r1;
    if (lock == 1 && all_rows) __syncthreads();
    for (int g = 0; g < nur; g += NU * kWave * wpr) {
      float acc[NU][8];
#pragma unroll
      for (int k = 0; k < NU; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
      for (int i0 = 0; i0 < n; i0 += DEPTH) {
        if (lock == 2 && all_rows) __syncthreads();
        Unit<bf16_bits, 8> v[DEPTH][NU];
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) {
          const int i = i0 + b < n ? i0 + b : n - 1;
          const bf16_bits* rp = static_cast<const bf16_bits*>(src.ptr[i]) + row * src.ld[i];
#pragma unroll
          for (int k = 0; k < NU; ++k) {
            if constexpr (F32OUT) {
              // two runs of 4 columns, 256 apart: each 16-byte float32 store then lands next
              // to its neighbour lanes' (1 KiB a store instruction). d is a multiple of 8, so
              // a run lies wholly inside the row or wholly past it.
              const int c0 = (g + (k * wpr + wr) * kWave) * 8 + 4 * lane;
              const u32x2 lo = c0 < nur * 8
                  ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rp + c0))
                  : u32x2{0u, 0u};
              const u32x2 hi = c0 + 256 < nur * 8
                  ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rp + c0 + 256))
                  : u32x2{0u, 0u};
              v[b][k].raw = u32x4{lo.x, lo.y, hi.x, hi.y};
            } else {
              const int u = g + (k * wpr + wr) * kWave + lane;
              if (u < nur) v[b][k].load(rp + static_cast<int64_t>(u) * 8);
              else v[b][k].zero();
            }
          }
        }
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) {
          const float wb = i0 + b < n ? w : 0.f;
#pragma unroll
          for (int k = 0; k < NU; ++k) {
            float x[8];
            v[b][k].get(x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][e] = fmaf(wb, x[e], acc[k][e]);
          }
        }
      }
      for (int j = 0; j < nout; ++j) {
#pragma unroll
        for (int k = 0; k < NU; ++k) {
          if constexpr (F32OUT) {
            const int c0 = (g + (k * wpr + wr) * kWave) * 8 + 4 * lane;
            float* op = static_cast<float*>(out.ptr[j]) + row * out.ld[j] + c0;
            if (c0 < nur * 8)
              out_store(f32x4{acc[k][0], acc[k][1], acc[k][2], acc[k][3]},
                        reinterpret_cast<f32x4*>(op));
            if (c0 + 256 < nur * 8)
              out_store(f32x4{acc[k][4], acc[k][5], acc[k][6], acc[k][7]},
                        reinterpret_cast<f32x4*>(op + 256));
          } else {
            const int u = g + (k * wpr + wr) * kWave + lane;
            if (u < nur) {
              Unit<bf16_bits, 8> y;
              y.set(acc[k]);
              y.store(static_cast<bf16_bits*>(out.ptr[j]) + row * out.ld[j] +
                      static_cast<int64_t>(u) * 8);
            }
          }
        }
      }
    }
  }
}

template <int DEPTH, int NU>
void launch_mix_stream_t(const SrcList& src, int n, int64_t r0, int64_t r1, int nur,
                         const DstList& out, int nout, bool f32_out, float w, int wpr, int lock,
                         unsigned blocks, hipStream_t s) {
  if (f32_out)
    hipLaunchKernelGGL((k_mix_stream<DEPTH, NU, true>), dim3(blocks), dim3(kBlock), 0, s, src, n,
                       r0, r1, nur, out, nout, w, wpr, lock);
  else
    hipLaunchKernelGGL((k_mix_stream<DEPTH, NU, false>), dim3(blocks), dim3(kBlock), 0, s, src,
                       n, r0, r1, nur, out, nout, w, wpr, lock);
}

hipError_t launch_mix_stream(const SrcList& src, int n, int64_t T, int d, const DstList& out,
                             int nout, bool f32_out, int waves_per_cu, int waves_per_row,
                             int depth, int slots, int rows_per_wave, int lockstep,
                             hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t blocks = static_cast<int64_t>(cus) * waves_per_cu / kWavesPerBlock;
  // rows_per_wave rows for each row group of the launch
  const int64_t span =
      rows_per_wave > 0 ? blocks * (kWavesPerBlock / waves_per_row) * rows_per_wave : T;
  const int nur = d / 8;
  const float w = 1.0f / static_cast<float>(n);
  const unsigned g = static_cast<unsigned>(blocks);
  for (int64_t r0 = 0; r0 < T; r0 += span) {
    const int64_t r1 = r0 + span < T ? r0 + span : T;
    const int key = 10 * depth + slots;
#define LRAR_MIX(D, U) \
  launch_mix_stream_t<D, U>(src, n, r0, r1, nur, out, nout, f32_out, w, waves_per_row, lockstep, \
                            g, s)
    switch (key) {
      case 12: LRAR_MIX(1, 2); break;
      case 14: LRAR_MIX(1, 4); break;
      case 18: LRAR_MIX(1, 8); break;
      case 26: LRAR_MIX(1, 16); break;
      case 22: LRAR_MIX(2, 2); break;
      case 24: LRAR_MIX(2, 4); break;
      case 28: LRAR_MIX(2, 8); break;
      case 42: LRAR_MIX(4, 2); break;
      case 44: LRAR_MIX(4, 4); break;
      default: return hipErrorInvalidValue;
    }
#undef LRAR_MIX
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_read_stream(const void* src, size_t bytes, void* sink, hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  hipLaunchKernelGGL(k_read_stream, dim3(kCalibBlocks), dim3(kBlock), 0, s,
                     static_cast<const u32x4*>(src), n16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace lrar
