// LR-AttnRes depth-mix read: the oracle.
//
// TEST INFRASTRUCTURE ONLY. This file is a plain, slow, obviously correct fp64 CPU
// statement of what the read computes. Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg may load it. It shares no code, header, table or helper
// with the HIP library, and the HIP library never calls it.
//
// Sources cited (titles of the public pages this was written from):
//   [Explainer]  "Low-Rank Attention Residuals", the author's explainer page.
//   [Paper]      "Low-Rank Attention Residuals" (J. Su), the paper's HTML version.
//   [AttnRes-TR] "Attention Residuals (AttnRes / Block AttnRes) - Technical Report",
//                a summary page of the predecessor report.
//
// Conventions shared by every entry point below:
//   * A source is a row-major [T, d] array of doubles. src[i] points at its row 0 and
//     ld[i] is its row stride in elements. The caller decodes bf16/fp32 inputs to
//     double first (the decode is exact).
//   * q is the site's query, r doubles. Every token uses the same q.
//   * All arithmetic is IEEE double, evaluated in the order the formulas are written.
//     Nothing is blocked, fused or reordered.
//   * Functions return 0 on success, -1 on an invalid argument.
//
// Readings taken where the pages are silent or garbled (each also listed in the design notes):
//   * The RMS denominator is sqrt(mean(k^2) + eps): the square root is lost in the
//     paper's printed Eq. 13, but the explainer's code takes rsqrt and its worked example
//     maps the key (1,0) to (sqrt 2, 0).
//   * No affine gain in the key norm and no score temperature ([Paper] App. I calls the
//     norm parameter-free; the worked example's score is exactly q . k-bar).
//   * Softmax is evaluated as exp(z_i - max z) / sum_j exp(z_j - max z), which is the
//     same function as exp(z_i) / sum_j exp(z_j) and does not overflow.

#include <cmath>
#include <cstdint>
#include <cstddef>
#include <limits>
#include <vector>

namespace {

bool bad_common(int64_t T, int d, int r, double eps, int n, int n_min) {
  return T < 0 || d < 1 || r < 1 || r > d || !(eps >= 0.0) || n < n_min;
}

const double* row_of(const double* base, int64_t ld, int64_t t) { return base + t * ld; }

// The routing key of a source is its last r coordinates, a view into the value
// ([Paper] §3.3 "Routing keys": k = tail_r(o) = o_{d-r+1..d}, 1-based).
// Its RMS is sqrt((1/r) * sum_j k_j^2 + eps)
// ([Explainer] "The mechanism in PyTorch-style code", function rms; [Paper] §3.3).
double slice_rms(const double* o_row, int d, int r, double eps) {
  double sum_sq = 0.0;
  for (int j = d - r; j < d; ++j) sum_sq += o_row[j] * o_row[j];
  return std::sqrt(sum_sq / r + eps);
}

// Score of one source at one read: z = q . RMSNorm(tail_r(o))
// ([Paper] §3.1 routing equation with the key of §3.3; [Explainer] "A short description
// chooses a full-width value").
double slice_score(const double* o_row, int d, int r, double eps, const double* q) {
  const double rho = slice_rms(o_row, d, r, eps);
  double z = 0.0;
  for (int j = 0; j < r; ++j) z += q[j] * (o_row[d - r + j] / rho);
  return z;
}

// Softmax over the sources of one read ([Paper] §3.1; [Explainer] "softmax converts
// scores into positive weights summing to one").
void softmax(const std::vector<double>& z, std::vector<double>& alpha) {
  const size_t n = z.size();
  alpha.assign(n, 0.0);
  double m = -std::numeric_limits<double>::infinity();
  for (size_t i = 0; i < n; ++i) m = (z[i] > m || std::isnan(z[i])) ? z[i] : m;
  double l = 0.0;
  for (size_t i = 0; i < n; ++i) {
    alpha[i] = std::exp(z[i] - m);
    l += alpha[i];
  }
  for (size_t i = 0; i < n; ++i) alpha[i] /= l;
}

}  // namespace

extern "C" {

// Per-token slice statistics, exposed so tests can pin the intermediate values:
// z[t*n + i] = score of source i at token t, rho[t*n + i] = its slice RMS. Either may be null.
int orc_scores(int64_t T, int d, int r, double eps, int n, const double* const* src,
               const int64_t* ld, const double* q, double* z, double* rho) {
  if (bad_common(T, d, r, eps, n, 1) || !src || !ld || !q) return -1;
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      if (z) z[t * n + i] = slice_score(o, d, r, eps, q);
      if (rho) rho[t * n + i] = slice_rms(o, d, r, eps);
    }
  }
  return 0;
}

// The depth-mix read ([Paper] §3.1 and §3.3; [Explainer] "A short description chooses a
// full-width value"): for every token t,
//   alpha_i = softmax_i(q . RMSNorm(tail_r(o_i)))   over the n sources,
//   h       = sum_i alpha_i o_i                       over all d coordinates.
// out is [T, out_ld]; alpha (nullable) is [T, n].
int orc_forward(int64_t T, int d, int r, double eps, int n, const double* const* src,
                const int64_t* ld, const double* q, double* out, int64_t out_ld,
                double* alpha) {
  if (bad_common(T, d, r, eps, n, 1) || !src || !ld || !q || !out || out_ld < d) return -1;
  std::vector<double> z(n), a(n);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) z[i] = slice_score(row_of(src[i], ld[i], t), d, r, eps, q);
    softmax(z, a);
    double* h = out + t * out_ld;
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];
      h[j] = s;
    }
    if (alpha)
      for (int i = 0; i < n; ++i) alpha[t * n + i] = a[i];
  }
  return 0;
}

// Standard AttnRes, written separately from the sliced read: the key is the whole value,
// RMS-normalised over all d coordinates, and q has d entries ([Paper] §3.1,
// "alpha = softmax(q^T RMSNorm(o_i))"; [Explainer]: setting r = d recovers standard AttnRes).
int orc_attnres_standard(int64_t T, int d, double eps, int n, const double* const* src,
                         const int64_t* ld, const double* q, double* out, int64_t out_ld,
                         double* alpha) {
  if (bad_common(T, d, d, eps, n, 1) || !src || !ld || !q || !out || out_ld < d) return -1;
  std::vector<double> z(n), a(n);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      double ms = 0.0;
      for (int j = 0; j < d; ++j) ms += o[j] * o[j];
      ms /= d;
      const double inv = 1.0 / std::sqrt(ms + eps);
      double zi = 0.0;
      for (int j = 0; j < d; ++j) zi += q[j] * (o[j] * inv);
      z[i] = zi;
    }
    softmax(z, a);
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];
      out[t * out_ld + j] = s;
    }
    if (alpha)
      for (int i = 0; i < n; ++i) alpha[t * n + i] = a[i];
  }
  return 0;
}

// Full-width-RMS control read ([Paper] §4.4 Eq. 13 "control"; App. B.1): the key is
// normalised by the RMS of all d coordinates and then sliced,
//   k-bar = P_r o / sqrt(||o||^2 / d + eps).
int orc_forward_fullrms(int64_t T, int d, int r, double eps, int n, const double* const* src,
                        const int64_t* ld, const double* q, double* out, int64_t out_ld,
                        double* alpha) {
  if (bad_common(T, d, r, eps, n, 1) || !src || !ld || !q || !out || out_ld < d) return -1;
  std::vector<double> z(n), a(n);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      double sum_sq = 0.0;
      for (int j = 0; j < d; ++j) sum_sq += o[j] * o[j];
      const double rho_d = std::sqrt(sum_sq / d + eps);
      double zi = 0.0;
      for (int j = 0; j < r; ++j) zi += q[j] * (o[d - r + j] / rho_d);
      z[i] = zi;
    }
    softmax(z, a);
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];
      out[t * out_ld + j] = s;
    }
    if (alpha)
      for (int i = 0; i < n; ++i) alpha[t * n + i] = a[i];
  }
  return 0;
}

// Separate-key read, the read side of Projected LR-AttnRes ([Paper] App. C.1: each source
// has its own r-wide key, RMS-normalised; App. C.2: a source then carries d + r elements).
// Source i supplies a value row o_i (d wide, from src) and a key row k_i (r wide, from key);
// for every token t,
//   alpha_i = softmax_i(q . k_i / sqrt(||k_i||^2 / r + eps)),   h = sum_i alpha_i o_i.
// key[i] is a [T, key_ld[i]] array of which the first r columns are the key.
int orc_forward_keys(int64_t T, int d, int r, double eps, int n, const double* const* src,
                     const int64_t* ld, const double* const* key, const int64_t* key_ld,
                     const double* q, double* out, int64_t out_ld, double* alpha) {
  if (bad_common(T, d, r, eps, n, 1) || !src || !ld || !key || !key_ld || !q || !out ||
      out_ld < d)
    return -1;
  for (int i = 0; i < n; ++i)
    if (!key[i] || key_ld[i] < r) return -1;
  std::vector<double> z(n), a(n);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const double* k = row_of(key[i], key_ld[i], t);
      double sum_sq = 0.0;
      for (int j = 0; j < r; ++j) sum_sq += k[j] * k[j];
      const double rho = std::sqrt(sum_sq / r + eps);
      double zi = 0.0;
      for (int j = 0; j < r; ++j) zi += q[j] * (k[j] / rho);
      z[i] = zi;
    }
    softmax(z, a);
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];
      out[t * out_ld + j] = s;
    }
    if (alpha)
      for (int i = 0; i < n; ++i) alpha[t * n + i] = a[i];
  }
  return 0;
}

// Phase 1 of the two-phase block schedule ([AttnRes-TR] Method, "two-phase inference":
// the block's static queries are batched against the cached block representations;
// [Paper] §3.4: the inter- and intra-block results merge by an online-softmax update).
// For each query s and token t, over the n sources:
//   m = max_i z_i,  l = sum_i exp(z_i - m),  acc = sum_i exp(z_i - m) o_i  (not normalised).
// q is [nq, r] (row s at q + s*r); m and l are [nq, T]; acc is [nq, T, d].
int orc_stats(int64_t T, int d, int r, double eps, int n, const double* const* src,
              const int64_t* ld, int nq, const double* q, double* m, double* l, double* acc) {
  if (bad_common(T, d, r, eps, n, 1) || nq < 1 || !src || !ld || !q || !m || !l || !acc)
    return -1;
  std::vector<double> z(n), e(n);
  for (int s = 0; s < nq; ++s) {
    const double* qs = q + (int64_t)s * r;
    for (int64_t t = 0; t < T; ++t) {
      double mx = -std::numeric_limits<double>::infinity();
      for (int i = 0; i < n; ++i) {
        z[i] = slice_score(row_of(src[i], ld[i], t), d, r, eps, qs);
        mx = (z[i] > mx || std::isnan(z[i])) ? z[i] : mx;
      }
      double sum = 0.0;
      for (int i = 0; i < n; ++i) {
        e[i] = std::exp(z[i] - mx);
        sum += e[i];
      }
      m[(int64_t)s * T + t] = mx;
      l[(int64_t)s * T + t] = sum;
      double* a = acc + ((int64_t)s * T + t) * d;
      for (int j = 0; j < d; ++j) {
        double v = 0.0;
        for (int i = 0; i < n; ++i) v += e[i] * row_of(src[i], ld[i], t)[j];
        a[j] = v;
      }
    }
  }
  return 0;
}

// Phase 2: merge one site's Phase-1 statistics (m, l, acc) with n >= 0 further sources
// (normally the intra-block partial sum) by the online-softmax update ([AttnRes-TR] Method;
// [Paper] §3.4):
//   m' = max(m, max_b z_b),
//   l' = l e^{m-m'} + sum_b e^{z_b-m'},
//   h  = (acc e^{m-m'} + sum_b e^{z_b-m'} o_b) / l'.
// m, l are [T]; acc is [T, d]; out is [T, out_ld]; m_out, l_out (nullable) are [T].
int orc_merge(int64_t T, int d, int r, double eps, const double* m, const double* l,
              const double* acc, int n, const double* const* src, const int64_t* ld,
              const double* q, double* out, int64_t out_ld, double* m_out, double* l_out) {
  if (bad_common(T, d, r, eps, n, 0) || !m || !l || !acc || !out || out_ld < d) return -1;
  if (n > 0 && (!src || !ld || !q)) return -1;
  std::vector<double> z(n > 0 ? n : 1);
  for (int64_t t = 0; t < T; ++t) {
    double m_new = m[t];
    for (int i = 0; i < n; ++i) {
      z[i] = slice_score(row_of(src[i], ld[i], t), d, r, eps, q);
      m_new = (z[i] > m_new || std::isnan(z[i])) ? z[i] : m_new;
    }
    const double scale_old = std::exp(m[t] - m_new);
    double l_new = l[t] * scale_old;
    for (int i = 0; i < n; ++i) l_new += std::exp(z[i] - m_new);
    for (int j = 0; j < d; ++j) {
      double v = acc[t * d + j] * scale_old;
      for (int i = 0; i < n; ++i) v += std::exp(z[i] - m_new) * row_of(src[i], ld[i], t)[j];
      out[t * out_ld + j] = v / l_new;
    }
    if (m_out) m_out[t] = m_new;
    if (l_out) l_out[t] = l_new;
  }
  return 0;
}

// Rounds x to the nearest number with a p-bit significand, ties to even, in a binary format
// whose normal range starts at 2^-126 (below it the spacing stays 2^(-126 - p + 1), as for
// subnormals): p = 24 is IEEE float32, p = 8 is bfloat16, p = 53 leaves a double of
// magnitude >= 2^-126 unchanged.
// Overflow is not modelled (the values here stay far below the formats' maxima).
static double round_to_format(double x, int p) {
  if (x == 0.0 || !std::isfinite(x)) return x;
  int e = 0;
  std::frexp(x, &e);  // x = f 2^e with 1/2 <= |f| < 1: the leading bit is worth 2^(e-1)
  int lead = e - 1;
  if (lead < -126) lead = -126;
  const double spacing = std::ldexp(1.0, lead - (p - 1));
  return std::nearbyint(x / spacing) * spacing;  // the default mode: nearest, ties to even
}

// Phase 2 with the partial-sum update fused in ([Paper] §3.3 "Partial-block routing": the
// block's running sum is kept at full width, a new sub-layer output is added into it before
// the next read, and that read keys the sum by its last r columns after the addition;
// [AttnRes-TR] Method, Phase 2 merges the intra-block lookback). The
// updated sum is stored in the sources' element type with a p-bit significand,
//   b' = round_to_format(b + o, p)      (b null: the block's first write, b' = round(o)),
// and the site merges its Phase-1 statistics with the single source b' as orc_merge does.
// b, o are [T, *_ld]; b_out is [T, d] (row stride d) and receives b'.
int orc_merge_accumulate(int64_t T, int d, int r, double eps, int p, const double* m,
                         const double* l, const double* acc, const double* b, int64_t b_ld,
                         const double* o, int64_t o_ld, const double* q, double* b_out,
                         double* out, int64_t out_ld, double* m_out, double* l_out) {
  if (bad_common(T, d, r, eps, 1, 1) || p < 2 || p > 53 || !o || o_ld < d || !b_out || !q)
    return -1;
  if (b && b_ld < d) return -1;
  for (int64_t t = 0; t < T; ++t) {
    for (int j = 0; j < d; ++j) {
      const double prev = b ? row_of(b, b_ld, t)[j] : 0.0;
      b_out[t * d + j] = round_to_format(prev + row_of(o, o_ld, t)[j], p);
    }
  }
  const double* srcs[1] = {b_out};
  const int64_t lds[1] = {d};
  return orc_merge(T, d, r, eps, m, l, acc, 1, srcs, lds, q, out, out_ld, m_out, l_out);
}

// Exposes round_to_format so tests can pin it against library conversions.
int orc_round_to_format(int64_t count, const double* x, int p, double* y) {
  if (count < 0 || p < 2 || p > 53 || (count > 0 && (!x || !y))) return -1;
  for (int64_t k = 0; k < count; ++k) y[k] = round_to_format(x[k], p);
  return 0;
}

// Backward of one read, treating every source slot as an independent input
// ([Paper] App. B.3). With g = dL/dh for token t:
//   Lemma 2 / §4.7:  dL/do_i = alpha_i g + alpha_i <g, o_i - h> grad_{o_i} z_i,
//   Cor. 2.1:        grad_{o_i} z_i = P_r^T [ q / rho_i - (q . k_i) k_i / (r rho_i^3) ],
//   and, since z_i = q . k-bar_i,  dL/dq = sum_t sum_i alpha_i <g, o_i - h> k-bar_i.
// dout is [T, dout_ld]; dsrc[i] is [T, d] (row stride d), overwritten; dq is [r], overwritten.
int orc_backward(int64_t T, int d, int r, double eps, int n, const double* const* src,
                 const int64_t* ld, const double* q, const double* dout, int64_t dout_ld,
                 double* const* dsrc, double* dq) {
  if (bad_common(T, d, r, eps, n, 1) || !src || !ld || !q || !dout || dout_ld < d || !dsrc ||
      !dq)
    return -1;
  for (int j = 0; j < r; ++j) dq[j] = 0.0;
  std::vector<double> z(n), a(n), rho(n), h(d);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      rho[i] = slice_rms(o, d, r, eps);
      z[i] = slice_score(o, d, r, eps, q);
    }
    softmax(z, a);
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];
      h[j] = s;
    }
    const double* g = dout + t * dout_ld;
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      double g_dot_diff = 0.0;  // <g, o_i - h>
      for (int j = 0; j < d; ++j) g_dot_diff += g[j] * (o[j] - h[j]);
      const double dz = a[i] * g_dot_diff;  // dL/dz_i (Lemma 2)
      double q_dot_k = 0.0;
      for (int j = 0; j < r; ++j) q_dot_k += q[j] * o[d - r + j];
      double* gi = dsrc[i] + t * d;
      for (int j = 0; j < d; ++j) gi[j] = a[i] * g[j];
      const double rho3 = rho[i] * rho[i] * rho[i];
      for (int j = 0; j < r; ++j) {
        const double k = o[d - r + j];
        gi[d - r + j] += dz * (q[j] / rho[i] - q_dot_k * k / (r * rho3));
        dq[j] += dz * (k / rho[i]);
      }
    }
  }
  return 0;
}

// Backward of the full-width-RMS control read ([Paper] App. B.3, Cor. 2.2):
//   grad_{o_i} z_i = P_r^T q / rho_d(o_i) - z_i o_i / (d rho_d(o_i)^2),
// combined with Lemma 2 as in orc_backward. dq = sum_t sum_i dL/dz_i P_r o_i / rho_d(o_i).
int orc_backward_fullrms(int64_t T, int d, int r, double eps, int n, const double* const* src,
                         const int64_t* ld, const double* q, const double* dout,
                         int64_t dout_ld, double* const* dsrc, double* dq) {
  if (bad_common(T, d, r, eps, n, 1) || !src || !ld || !q || !dout || dout_ld < d || !dsrc ||
      !dq)
    return -1;
  for (int j = 0; j < r; ++j) dq[j] = 0.0;
  std::vector<double> z(n), a(n), rho(n), h(d);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      double sum_sq = 0.0;
      for (int j = 0; j < d; ++j) sum_sq += o[j] * o[j];
      rho[i] = std::sqrt(sum_sq / d + eps);
      double zi = 0.0;
      for (int j = 0; j < r; ++j) zi += q[j] * (o[d - r + j] / rho[i]);
      z[i] = zi;
    }
    softmax(z, a);
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];
      h[j] = s;
    }
    const double* g = dout + t * dout_ld;
    for (int i = 0; i < n; ++i) {
      const double* o = row_of(src[i], ld[i], t);
      double g_dot_diff = 0.0;
      for (int j = 0; j < d; ++j) g_dot_diff += g[j] * (o[j] - h[j]);
      const double dz = a[i] * g_dot_diff;
      double* gi = dsrc[i] + t * d;
      for (int j = 0; j < d; ++j) gi[j] = a[i] * g[j] - dz * z[i] * o[j] / (d * rho[i] * rho[i]);
      for (int j = 0; j < r; ++j) {
        gi[d - r + j] += dz * q[j] / rho[i];
        dq[j] += dz * (o[d - r + j] / rho[i]);
      }
    }
  }
  return 0;
}

}  // extern "C"
