// Host side of libaatc: calibration statistics, rotations, integer reverse water-filling,
// quantizer tables and the calibration artefact.  Pure C++17, fp64 throughout.
//
// Method sources: page "KV Cache Compression Through the Lens of Transform Coding"
// (Key points, Full text: transform coding + reverse water-filling over a calibration set);
// page "SPECTRA: Pushing the KV Cache Beyond the 2-Bit Cliff via Spectral Transform Coding"
// (Abstract: a coordinate system computed from the cache's own statistics removes the
// channel correlations; the budget goes to the few channels carrying the signal); page
// "Ablation, Statistical Inference, and Validation for KV-Cache Compression" (first
// abstract: Walsh-Hadamard transform + scalar MSE quantizer).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "aatc_internal.h"

namespace aatc {

static thread_local char g_err[512] = "";

aatc_status fail(aatc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

uint64_t blob_checksum(const aatc_calib* c) {
  const unsigned char* p = reinterpret_cast<const unsigned char*>(c);
  const size_t off = offsetof(aatc_calib, checksum);
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < sizeof(aatc_calib); ++i) {
    unsigned char b = (i >= off && i < off + sizeof(uint64_t)) ? 0 : p[i];
    h ^= b;
    h *= 1099511628211ull;
  }
  return h;
}

// Plane, field and channel->field tables from bits[].
void build_layout(aatc_calib* c) {
  const int d = AATC_D;
  int p = 0, coded = 0;
  std::memset(c->plane_channel, 0, sizeof(c->plane_channel));
  std::memset(c->plane_bit, 0, sizeof(c->plane_bit));
  for (int i = 0; i < d; ++i) {
    if (c->bits[i]) ++coded;
    for (int k = 0; k < c->bits[i]; ++k) {
      c->plane_channel[p] = static_cast<uint8_t>(i);
      c->plane_bit[p] = static_cast<uint8_t>(k);
      ++p;
    }
  }
  struct F { int ch, shift, w; };
  std::vector<F> f;
  for (int i = 0; i < d; ++i) {
    int rest = c->bits[i], shift = 0;
    for (int w : {4, 2, 1})
      while (rest >= w) { f.push_back({i, shift, w}); shift += w; rest -= w; }
  }
  std::stable_sort(f.begin(), f.end(), [](const F& a, const F& b) {
    if (a.w != b.w) return a.w > b.w;
    if (a.ch != b.ch) return a.ch < b.ch;
    return a.shift < b.shift;
  });
  std::memset(c->field_channel, 0, sizeof(c->field_channel));
  std::memset(c->field_shift, 0, sizeof(c->field_shift));
  std::memset(c->field_width, 0, sizeof(c->field_width));
  std::memset(c->field_word, 0, sizeof(c->field_word));
  for (int i = 0; i < d * 3; ++i) c->channel_field[i] = -1;
  int word = 0, n4 = 0, n2 = 0, n1 = 0;
  for (size_t k = 0; k < f.size(); ++k) {
    c->field_channel[k] = static_cast<uint16_t>(f[k].ch);
    c->field_shift[k] = static_cast<uint8_t>(f[k].shift);
    c->field_width[k] = static_cast<uint8_t>(f[k].w);
    c->field_word[k] = static_cast<uint16_t>(word);
    word += 2 * f[k].w;
    (f[k].w == 4 ? n4 : f[k].w == 2 ? n2 : n1)++;
    int16_t* cf = c->channel_field + 3 * f[k].ch;
    int slot = 0;
    while (cf[slot] >= 0) ++slot;
    cf[slot] = static_cast<int16_t>(k);
  }
  // channel_field in increasing shift order
  for (int i = 0; i < d; ++i) {
    int16_t* cf = c->channel_field + 3 * i;
    std::sort(cf, cf + 3, [&](int16_t a, int16_t b) {
      if (a < 0) return false;
      if (b < 0) return true;
      return c->field_shift[a] < c->field_shift[b];
    });
  }
  c->n_coded = coded;
  c->n_fields = static_cast<int32_t>(f.size());
  c->n_fields4 = n4;
  c->n_fields2 = n2;
  c->n_fields1 = n1;
}

namespace {

// ---- statistics ------------------------------------------------------------------------
template <class T>
double load_elem(const void* x, int64_t i);
template <>
double load_elem<float>(const void* x, int64_t i) { return static_cast<const float*>(x)[i]; }
template <>
double load_elem<double>(const void* x, int64_t i) { return static_cast<const double*>(x)[i]; }
struct bf16_tag {};
template <>
double load_elem<bf16_tag>(const void* x, int64_t i) {
  uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(x)[i]) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

template <class T>
bool read_rows(const void* x, int64_t n, int64_t stride, std::vector<double>& out) {
  out.resize(static_cast<size_t>(n) * AATC_D);
  for (int64_t r = 0; r < n; ++r)
    for (int j = 0; j < AATC_D; ++j) {
      double v = load_elem<T>(x, r * stride + j);
      if (!std::isfinite(v)) return false;
      out[static_cast<size_t>(r) * AATC_D + j] = v;
    }
  return true;
}

// Mean and centred covariance with 1/M (two passes).
void mean_cov(const std::vector<double>& x, int64_t m, double* mu, std::vector<double>& cov) {
  const int d = AATC_D;
  for (int j = 0; j < d; ++j) mu[j] = 0.0;
  for (int64_t r = 0; r < m; ++r)
    for (int j = 0; j < d; ++j) mu[j] += x[r * d + j];
  for (int j = 0; j < d; ++j) mu[j] /= static_cast<double>(m);
  cov.assign(d * d, 0.0);
  std::vector<double> c(d);
  for (int64_t r = 0; r < m; ++r) {
    for (int j = 0; j < d; ++j) c[j] = x[r * d + j] - mu[j];
    for (int a = 0; a < d; ++a) {
      const double ca = c[a];
      double* row = &cov[a * d];
      for (int b = a; b < d; ++b) row[b] += ca * c[b];
    }
  }
  for (int a = 0; a < d; ++a)
    for (int b = a; b < d; ++b) {
      cov[a * d + b] /= static_cast<double>(m);
      cov[b * d + a] = cov[a * d + b];
    }
}

// ---- cyclic Jacobi eigensolver (Golub & Van Loan, Matrix Computations, sec. 8.5) -------
// On return a holds the eigenvalues on its diagonal and v's columns the eigenvectors.
bool jacobi_eig(std::vector<double>& a, std::vector<double>& v, int n) {
  v.assign(n * n, 0.0);
  for (int i = 0; i < n; ++i) v[i * n + i] = 1.0;
  double fro = 0.0;
  for (double e : a) fro += e * e;
  fro = std::sqrt(fro);
  if (fro == 0.0) return true;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += 2.0 * a[p * n + q] * a[p * n + q];
    if (std::sqrt(off) <= 1e-17 * fro) return true;
    for (int p = 0; p < n - 1; ++p)
      for (int q = p + 1; q < n; ++q) {
        const double apq = a[p * n + q];
        if (apq == 0.0) continue;
        const double app = a[p * n + p], aqq = a[q * n + q];
        // skip negligible entries once they are below the diagonal's rounding level
        if (sweep > 3 && std::fabs(apq) < 1e-18 * (std::fabs(app) + std::fabs(aqq))) {
          a[p * n + q] = a[q * n + p] = 0.0;
          continue;
        }
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(1.0 + theta * theta));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < n; ++k) {
          const double akp = a[k * n + p], akq = a[k * n + q];
          a[k * n + p] = c * akp - s * akq;
          a[k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {
          const double apk = a[p * n + k], aqk = a[q * n + k];
          a[p * n + k] = c * apk - s * aqk;
          a[q * n + k] = s * apk + c * aqk;
        }
        a[p * n + q] = a[q * n + p] = 0.0;
        for (int k = 0; k < n; ++k) {
          const double vkp = v[k * n + p], vkq = v[k * n + q];
          v[k * n + p] = c * vkp - s * vkq;
          v[k * n + q] = s * vkp + c * vkq;
        }
      }
  }
  return false;
}

// ---- quantizer step g(b) ----------------------------------------------------------------
// Mid-rise uniform quantizer with 2^b levels (k - 2^(b-1) + 1/2) * step on Z ~ N(0,1).
// dMSE/dstep = -2 sum_k a_k int_bin(k) (z - r_k) phi(z) dz  (threshold terms cancel),
// evaluated on the positive half and doubled.  g(b) is its root, found by bisection.
double phi(double z) { return std::exp(-0.5 * z * z) * 0.39894228040143267794; }
double upper_tail(double z) { return 0.5 * std::erfc(z * 0.70710678118654752440); }

double mse_deriv(int b, double step) {
  const int half = 1 << (b - 1);
  double s = 0.0;
  for (int k = 0; k < half; ++k) {
    const double lo = k * step;
    const bool last = (k == half - 1);
    const double hi = (k + 1) * step;
    const double pl = phi(lo), ph = last ? 0.0 : phi(hi);
    const double ql = upper_tail(lo), qh = last ? 0.0 : upper_tail(hi);
    const double r = (k + 0.5) * step;
    s += (k + 0.5) * ((pl - ph) - r * (ql - qh));
  }
  return -4.0 * s;
}

double optimal_step(int b) {
  double lo = 1e-4, hi = 4.0;  // derivative < 0 at lo (overload), > 0 at hi (granular)
  for (int it = 0; it < 2000; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (mse_deriv(b, mid) < 0.0) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// ---- Lloyd-Max quantizer of N(0,1) ----------------------------------------------------------
// Page "SPHERICAL KV ..." (NOVA-KV abstract) and page "Ablation ..." (OCTOPUS abstract).  The
// 2^b-level MSE-optimal quantizer is the solution of Lloyd's conditions: each level the mean of
// N(0,1) over its cell, each threshold the midpoint of its two levels.  The quantizer is
// symmetric, so the h = 2^(b-1) positive levels are solved with cells [t_(k-1), t_k), t_0 = 0,
// t_k = (y_k + y_(k+1)) / 2, the last cell unbounded: Lloyd iterations from a uniform start,
// then Newton steps on y - centroid(y) = 0 (tridiagonal Jacobian, Thomas algorithm).
void lm_centroids(const std::vector<double>& y, std::vector<double>& c, std::vector<double>& dl,
                  std::vector<double>& dr) {
  const int h = static_cast<int>(y.size());
  c.assign(h, 0.0);
  dl.assign(h, 0.0);
  dr.assign(h, 0.0);
  for (int k = 0; k < h; ++k) {
    const double lo = k == 0 ? 0.0 : 0.5 * (y[k - 1] + y[k]);
    const bool last = k == h - 1;
    const double hi = last ? 0.0 : 0.5 * (y[k] + y[k + 1]);
    const double plo = phi(lo), phi_hi = last ? 0.0 : phi(hi);
    const double mass = upper_tail(lo) - (last ? 0.0 : upper_tail(hi));
    c[k] = (plo - phi_hi) / mass;
    // d centroid / d lower edge and d centroid / d upper edge
    dl[k] = k == 0 ? 0.0 : plo * (c[k] - lo) / mass;
    dr[k] = last ? 0.0 : phi_hi * (hi - c[k]) / mass;
  }
}

void lloyd_max_half(int b, std::vector<double>& y) {
  const int h = 1 << (b - 1);
  y.assign(h, 0.0);
  if (h == 1) {
    y[0] = std::sqrt(2.0 / 3.14159265358979323846);
    return;
  }
  for (int k = 0; k < h; ++k) y[k] = (k + 0.5) * (1.0 + 0.5 * b) / h;
  std::vector<double> c, dl, dr;
  for (int it = 0; it < 200; ++it) {
    lm_centroids(y, c, dl, dr);
    y = c;
  }
  std::vector<double> a(h), bd(h), cu(h), rhs(h);
  for (int it = 0; it < 60; ++it) {
    lm_centroids(y, c, dl, dr);
    // row k of J = I - d c / d y: sub (y_(k-1)) = -dl_k / 2, diag = 1 - (dl_k + dr_k) / 2,
    // sup (y_(k+1)) = -dr_k / 2
    for (int k = 0; k < h; ++k) {
      a[k] = -0.5 * dl[k];
      bd[k] = 1.0 - 0.5 * (dl[k] + dr[k]);
      cu[k] = -0.5 * dr[k];
      rhs[k] = c[k] - y[k];
    }
    for (int k = 1; k < h; ++k) {        // forward elimination
      const double m = a[k] / bd[k - 1];
      bd[k] -= m * cu[k - 1];
      rhs[k] -= m * rhs[k - 1];
    }
    double mx = 0.0;
    for (int k = h - 1; k >= 0; --k) {   // back substitution
      const double st = (rhs[k] - (k + 1 < h ? cu[k] * rhs[k + 1] : 0.0)) / bd[k];
      rhs[k] = st;
      mx = std::max(mx, std::fabs(st));
    }
    for (int k = 0; k < h; ++k) y[k] += rhs[k];
    if (mx <= 1e-17 * y[h - 1]) break;
  }
}

// Standardized levels (and Lloyd-Max thresholds) of b = 1..8 bits into the blob's tables.
void fill_levels(aatc_calib* c) {
  for (int b = 1; b <= AATC_MAX_BITS; ++b) {
    const int n = 1 << b, h = n >> 1, off = n - 2;
    if (c->quantizer == AATC_QUANT_LLOYD_MAX) {
      std::vector<double> y;
      lloyd_max_half(b, y);
      for (int k = 0; k < h; ++k) {
        c->level[off + h + k] = y[k];
        c->level[off + h - 1 - k] = -y[k];
      }
      for (int k = 0; k + 1 < n; ++k) c->thresh[off + k] = 0.5 * (c->level[off + k] + c->level[off + k + 1]);
      c->thresh[off + h - 1] = 0.0;
    } else {
      for (int k = 0; k < n; ++k) c->level[off + k] = k - h + 0.5;
    }
  }
  for (int k = 0; k < AATC_LEVELS; ++k) c->level32[k] = static_cast<float>(c->level[k]);
}

// ---- integer reverse water-filling ---------------------------------------------------------
// The B largest candidates sigma_i^2 4^-k (k < max_bits) in the order (value desc,
// channel asc, bit asc); exact in fp64 (ldexp).
// KLT of a symmetric d x d matrix: rows of r = eigenvectors in descending eigenvalue order
// (stable), the largest-magnitude entry of each row made positive (first index on ties);
// s2 = the eigenvalues, clamped at 0.
bool klt_rows(const std::vector<double>& sym, int d, double* r, double* s2) {
  std::vector<double> a = sym, v;
  if (!jacobi_eig(a, v, d)) return false;
  std::vector<int> order(d);
  for (int i = 0; i < d; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int i, int j) { return a[i * d + i] > a[j * d + j]; });
  for (int row = 0; row < d; ++row) {
    const int col = order[row];
    int jmax = 0;
    for (int k = 1; k < d; ++k)
      if (std::fabs(v[k * d + col]) > std::fabs(v[jmax * d + col])) jmax = k;
    const double sg = v[jmax * d + col] < 0 ? -1.0 : 1.0;
    for (int k = 0; k < d; ++k) r[row * d + k] = sg * v[k * d + col];
    s2[row] = std::max(a[col * d + col], 0.0);
  }
  return true;
}

// Eigenvalues of the query second moment below this fraction of the largest are raised to it.
constexpr double kNovaEigFloor = 1e-6;

void waterfill_impl(const double* s2, int d, int total, int max_bits, uint8_t* bits) {
  struct C { double v; int i, k; };
  std::vector<C> c;
  c.reserve(d * max_bits);
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < max_bits; ++k) c.push_back({std::ldexp(s2[i], -2 * k), i, k});
  std::sort(c.begin(), c.end(), [](const C& a, const C& b) {
    if (a.v != b.v) return a.v > b.v;
    if (a.i != b.i) return a.i < b.i;
    return a.k < b.k;
  });
  for (int i = 0; i < d; ++i) bits[i] = 0;
  for (int j = 0; j < total; ++j) bits[c[j].i]++;
}

}  // namespace

void waterfill(const double* s2, int d, int total, int max_bits, uint8_t* bits) {
  waterfill_impl(s2, d, total, max_bits, bits);
}

}  // namespace aatc

using namespace aatc;

extern "C" {

const char* aatc_status_string(aatc_status s) {
  switch (s) {
    case AATC_OK: return "ok";
    case AATC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case AATC_ERR_UNSUPPORTED: return "unsupported";
    case AATC_ERR_BUDGET: return "bit budget out of range";
    case AATC_ERR_NUMERICAL: return "numerical failure";
    case AATC_ERR_BAD_ARTEFACT: return "bad calibration artefact";
    case AATC_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case AATC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* aatc_last_error(void) { return g_err; }

size_t aatc_calib_bytes(int32_t d) { return d == AATC_D ? sizeof(aatc_calib) : 0; }

int32_t aatc_bits_budget(double bits_per_elem, int32_t d) {
  if (!(bits_per_elem >= 0.0) || d <= 0) return -1;
  const double b = std::floor(bits_per_elem * d + 0.5);
  if (b > 8.0 * d) return -1;
  return static_cast<int32_t>(b);
}

size_t aatc_packed_bytes(int32_t total_bits, int64_t n_tokens) {
  if (total_bits < 0 || n_tokens < 0) return 0;
  return static_cast<size_t>((n_tokens + AATC_TILE - 1) / AATC_TILE) * 8u * static_cast<size_t>(total_bits);
}

aatc_status aatc_calibrate(const aatc_calib_params* p, const void* x, aatc_dtype dt, int64_t n,
                           int64_t stride, void* out, size_t out_bytes) {
  clear_error();
  if (!p || !x || !out) return fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (p->d != AATC_D) return fail(AATC_ERR_UNSUPPORTED, "d=%d (only 128)", p->d);
  if (p->rotation < AATC_ROT_KLT || p->rotation > AATC_ROT_NOVA)
    return fail(AATC_ERR_INVALID_ARGUMENT, "rotation %d", p->rotation);
  if (p->rotation == AATC_ROT_NOVA) {
    if (!p->query_moment) return fail(AATC_ERR_INVALID_ARGUMENT, "NOVA needs query_moment");
    const double* s = p->query_moment;
    for (int i = 0; i < AATC_D * AATC_D; ++i)
      if (!std::isfinite(s[i])) return fail(AATC_ERR_NUMERICAL, "query_moment[%d] is not finite", i);
    for (int i = 0; i < AATC_D; ++i)
      for (int j = i + 1; j < AATC_D; ++j) {
        const double a = s[i * AATC_D + j], b = s[j * AATC_D + i];
        if (std::fabs(a - b) > 1e-12 * (std::fabs(a) + std::fabs(b)) + 1e-300)
          return fail(AATC_ERR_INVALID_ARGUMENT, "query_moment is not symmetric at (%d, %d)", i, j);
      }
  }
  if (p->max_bits < 1 || p->max_bits > AATC_MAX_BITS)
    return fail(AATC_ERR_BUDGET, "max_bits=%d (1..8)", p->max_bits);
  if (p->quantizer != AATC_QUANT_UNIFORM && p->quantizer != AATC_QUANT_LLOYD_MAX)
    return fail(AATC_ERR_INVALID_ARGUMENT, "quantizer %d", p->quantizer);
  const int32_t total = aatc_bits_budget(p->bits_per_elem, p->d);
  if (total < 0 || total > p->max_bits * p->d)
    return fail(AATC_ERR_BUDGET, "bits_per_elem=%g gives B outside [0, %d]", p->bits_per_elem,
                p->max_bits * p->d);
  if (n < 2) return fail(AATC_ERR_INVALID_ARGUMENT, "n_calib=%lld < 2", (long long)n);
  if (stride < AATC_D) return fail(AATC_ERR_INVALID_ARGUMENT, "row_stride < d");
  if (out_bytes < sizeof(aatc_calib)) return fail(AATC_ERR_BUFFER_TOO_SMALL, "calib buffer %zu < %zu",
                                                  out_bytes, sizeof(aatc_calib));
  if (p->channel_weight)
    for (int i = 0; i < AATC_D; ++i) {
      const double w = p->channel_weight[i];
      if (!std::isfinite(w)) return fail(AATC_ERR_NUMERICAL, "channel_weight[%d] is not finite", i);
      if (w < 0.0) return fail(AATC_ERR_INVALID_ARGUMENT, "channel_weight[%d] = %g < 0", i, w);
    }
  std::vector<double> xs;
  bool ok;
  switch (dt) {
    case AATC_F32: ok = read_rows<float>(x, n, stride, xs); break;
    case AATC_BF16: ok = read_rows<bf16_tag>(x, n, stride, xs); break;
    case AATC_F64: ok = read_rows<double>(x, n, stride, xs); break;
    default: return fail(AATC_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  }
  if (!ok) return fail(AATC_ERR_NUMERICAL, "non-finite calibration value");

  auto* c = static_cast<aatc_calib*>(out);
  std::memset(c, 0, sizeof(aatc_calib));
  c->magic = AATC_MAGIC;
  c->version = AATC_VERSION;
  c->d = AATC_D;
  c->rotation = p->rotation;
  c->total_bits = total;
  c->max_bits = p->max_bits;
  c->n_calib = static_cast<int32_t>(n);
  c->quantizer = p->quantizer;
  const int d = AATC_D;
  std::vector<double> cov;
  mean_cov(xs, n, c->mu, cov);

  if (p->rotation == AATC_ROT_KLT) {
    if (!klt_rows(cov, d, c->R, c->sigma2)) return fail(AATC_ERR_NUMERICAL, "Jacobi eigensolver did not converge");
  } else if (p->rotation == AATC_ROT_NOVA) {
    // S = V diag(s) V^T with s floored; S^(+-1/2); KLT U of M = S^(1/2) C S^(1/2);
    // E = U S^(1/2), R = U S^(-1/2)
    std::vector<double> a(p->query_moment, p->query_moment + d * d), v;
    if (!jacobi_eig(a, v, d)) return fail(AATC_ERR_NUMERICAL, "Jacobi eigensolver did not converge");
    double smax = 0.0;
    for (int i = 0; i < d; ++i) smax = std::max(smax, a[i * d + i]);
    if (!(smax > 0.0)) return fail(AATC_ERR_NUMERICAL, "query moment has no positive eigenvalue");
    std::vector<double> sh(d * d, 0.0), sih(d * d, 0.0), ev(d);
    for (int k = 0; k < d; ++k) ev[k] = std::max(a[k * d + k], kNovaEigFloor * smax);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double h = 0.0, ih = 0.0;
        for (int k = 0; k < d; ++k) {
          const double vv = v[i * d + k] * v[j * d + k];
          h += vv * std::sqrt(ev[k]);
          ih += vv / std::sqrt(ev[k]);
        }
        sh[i * d + j] = h;
        sih[i * d + j] = ih;
      }
    std::vector<double> tmp(d * d, 0.0), m(d * d, 0.0);
    for (int i = 0; i < d; ++i)          // tmp = S^(1/2) C
      for (int k = 0; k < d; ++k) {
        const double sik = sh[i * d + k];
        for (int j = 0; j < d; ++j) tmp[i * d + j] += sik * cov[k * d + j];
      }
    for (int i = 0; i < d; ++i)          // m = tmp S^(1/2)
      for (int k = 0; k < d; ++k) {
        const double tik = tmp[i * d + k];
        for (int j = 0; j < d; ++j) m[i * d + j] += tik * sh[k * d + j];
      }
    for (int i = 0; i < d; ++i)
      for (int j = i + 1; j < d; ++j) m[i * d + j] = m[j * d + i] = 0.5 * (m[i * d + j] + m[j * d + i]);
    std::vector<double> u(d * d);
    if (!klt_rows(m, d, u.data(), c->sigma2)) return fail(AATC_ERR_NUMERICAL, "Jacobi eigensolver did not converge");
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double e = 0.0, r = 0.0;
        for (int k = 0; k < d; ++k) {
          e += u[i * d + k] * sh[k * d + j];
          r += u[i * d + k] * sih[k * d + j];
        }
        c->E[i * d + j] = e;
        c->R[i * d + j] = r;
      }
  } else {
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        if (p->rotation == AATC_ROT_WHT) {
          const double s = (__builtin_popcount(i & j) & 1) ? -1.0 : 1.0;
          c->R[i * d + j] = s / std::sqrt(static_cast<double>(d));
        } else {
          c->R[i * d + j] = (i == j) ? 1.0 : 0.0;
        }
      }
    for (int i = 0; i < d; ++i) {  // sigma2_i = (R C R^T)_ii
      double s = 0.0;
      for (int j = 0; j < d; ++j) {
        double t = 0.0;
        for (int k = 0; k < d; ++k) t += cov[j * d + k] * c->R[i * d + k];
        s += c->R[i * d + j] * t;
      }
      c->sigma2[i] = s;
    }
  }
  if (p->rotation != AATC_ROT_NOVA) std::memcpy(c->E, c->R, sizeof(c->R));
  if (p->channel_weight) {
    // attention-aware: the candidates are w_i sigma_i^2 4^-k
    double ws2[AATC_D];
    for (int i = 0; i < d; ++i) ws2[i] = p->channel_weight[i] * c->sigma2[i];
    waterfill_impl(ws2, d, total, p->max_bits, c->bits);
  } else {
    waterfill_impl(c->sigma2, d, total, p->max_bits, c->bits);
  }

  double smax = 0.0;
  for (int i = 0; i < d; ++i) smax = std::max(smax, std::sqrt(std::max(c->sigma2[i], 0.0)));
  const double ref = smax > 0 ? smax : 1.0;
  for (int i = 0; i < d; ++i) {
    double o = 0.0;
    for (int j = 0; j < d; ++j) o += c->E[i * d + j] * c->mu[j];
    c->o[i] = o;
    if (c->bits[i]) {
      const double sg = std::sqrt(std::max(c->sigma2[i], 0.0));
      const double s0 = sg > 0 ? sg : std::ldexp(ref, -40);
      c->delta[i] = s0 * optimal_step(c->bits[i]);
      c->inv_delta[i] = 1.0 / c->delta[i];
      c->scale[i] = c->quantizer == AATC_QUANT_LLOYD_MAX ? s0 : c->delta[i];
      c->inv_scale[i] = 1.0 / c->scale[i];
    }
    c->o32[i] = static_cast<float>(c->o[i]);
    c->delta32[i] = static_cast<float>(c->delta[i]);
    c->scale32[i] = static_cast<float>(c->scale[i]);
  }
  for (int i = 0; i < d * d; ++i) c->R32[i] = static_cast<float>(c->R[i]);
  fill_levels(c);
  build_layout(c);
  c->checksum = blob_checksum(c);
  return AATC_OK;
}

aatc_status aatc_calib_validate(const void* blob, size_t bytes) {
  clear_error();
  if (!blob) return fail(AATC_ERR_INVALID_ARGUMENT, "null blob");
  if (bytes < sizeof(aatc_calib)) return fail(AATC_ERR_BUFFER_TOO_SMALL, "blob %zu < %zu", bytes, sizeof(aatc_calib));
  const auto* c = static_cast<const aatc_calib*>(blob);
  if (c->magic != AATC_MAGIC || c->version != AATC_VERSION) return fail(AATC_ERR_BAD_ARTEFACT, "magic/version");
  if (c->d != AATC_D) return fail(AATC_ERR_BAD_ARTEFACT, "d=%d", c->d);
  if (c->checksum != blob_checksum(c)) return fail(AATC_ERR_BAD_ARTEFACT, "checksum mismatch");
  if (c->quantizer != AATC_QUANT_UNIFORM && c->quantizer != AATC_QUANT_LLOYD_MAX)
    return fail(AATC_ERR_BAD_ARTEFACT, "quantizer %d", c->quantizer);
  int sum = 0;
  for (int i = 0; i < AATC_D; ++i) {
    if (c->bits[i] > AATC_MAX_BITS) return fail(AATC_ERR_BAD_ARTEFACT, "bits[%d]=%d", i, c->bits[i]);
    sum += c->bits[i];
    if (c->bits[i] && !(c->delta[i] > 0.0)) return fail(AATC_ERR_BAD_ARTEFACT, "delta[%d]", i);
    if (c->bits[i] && !(c->scale[i] > 0.0)) return fail(AATC_ERR_BAD_ARTEFACT, "scale[%d]", i);
  }
  for (int b = 1; b <= AATC_MAX_BITS; ++b)          // level tables strictly increasing
    for (int k = (1 << b) - 2; k + 1 < (1 << (b + 1)) - 2; ++k)
      if (!(c->level[k] < c->level[k + 1])) return fail(AATC_ERR_BAD_ARTEFACT, "level table of %d bits", b);
  if (sum != c->total_bits) return fail(AATC_ERR_BAD_ARTEFACT, "bits sum %d != %d", sum, c->total_bits);
  aatc_calib tmp;
  std::memcpy(&tmp, c, sizeof(tmp));
  build_layout(&tmp);
  if (std::memcmp(&tmp, c, sizeof(tmp)) != 0) return fail(AATC_ERR_BAD_ARTEFACT, "layout tables");
  return AATC_OK;
}

aatc_status aatc_query_channel_weights(const void* blob, size_t bytes, const void* q, aatc_dtype dt, int64_t n,
                                       int64_t stride, double* w) {
  const aatc_status st = aatc_calib_validate(blob, bytes);   // clears the error, or sets it
  if (st != AATC_OK) return st;
  if (!q || !w) return fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (n < 1) return fail(AATC_ERR_INVALID_ARGUMENT, "n=%lld < 1", (long long)n);
  if (stride < AATC_D) return fail(AATC_ERR_INVALID_ARGUMENT, "row_stride < d");
  std::vector<double> qs;
  bool ok;
  switch (dt) {
    case AATC_F32: ok = read_rows<float>(q, n, stride, qs); break;
    case AATC_BF16: ok = read_rows<bf16_tag>(q, n, stride, qs); break;
    case AATC_F64: ok = read_rows<double>(q, n, stride, qs); break;
    default: return fail(AATC_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  }
  if (!ok) return fail(AATC_ERR_NUMERICAL, "non-finite query value");
  const auto* c = static_cast<const aatc_calib*>(blob);
  const int d = AATC_D;
  std::vector<double> acc(d, 0.0);
  for (int64_t r = 0; r < n; ++r) {
    const double* qr = qs.data() + r * d;
    for (int i = 0; i < d; ++i) {
      double y = 0.0;
      for (int k = 0; k < d; ++k) y += c->R[i * d + k] * qr[k];
      acc[i] += y * y;
    }
  }
  for (int i = 0; i < d; ++i) w[i] = acc[i] / static_cast<double>(n);
  return AATC_OK;
}

aatc_status aatc_query_moment(const void* q, aatc_dtype dt, int64_t n, int64_t stride, double* out) {
  clear_error();
  if (!q || !out) return fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (n < 1) return fail(AATC_ERR_INVALID_ARGUMENT, "n=%lld < 1", (long long)n);
  if (stride < AATC_D) return fail(AATC_ERR_INVALID_ARGUMENT, "row_stride < d");
  std::vector<double> qs;
  bool ok;
  switch (dt) {
    case AATC_F32: ok = read_rows<float>(q, n, stride, qs); break;
    case AATC_BF16: ok = read_rows<bf16_tag>(q, n, stride, qs); break;
    case AATC_F64: ok = read_rows<double>(q, n, stride, qs); break;
    default: return fail(AATC_ERR_UNSUPPORTED, "dtype %d", (int)dt);
  }
  if (!ok) return fail(AATC_ERR_NUMERICAL, "non-finite query value");
  const int d = AATC_D;
  std::vector<double> acc(d * d, 0.0);
  for (int64_t r = 0; r < n; ++r) {
    const double* qr = qs.data() + r * d;
    for (int i = 0; i < d; ++i)
      for (int j = i; j < d; ++j) acc[i * d + j] += qr[i] * qr[j];
  }
  for (int i = 0; i < d; ++i)
    for (int j = i; j < d; ++j) out[i * d + j] = out[j * d + i] = acc[i * d + j] / static_cast<double>(n);
  return AATC_OK;
}

aatc_status aatc_joint_kv_split(const void* kblobs, const void* vblobs, int32_t n_heads, const double* kw,
                                float scale, int32_t total, int32_t* bk_out, int32_t* bv_out) {
  clear_error();
  if (!kblobs || !vblobs || !bk_out || !bv_out) return fail(AATC_ERR_INVALID_ARGUMENT, "null pointer");
  if (n_heads < 1) return fail(AATC_ERR_INVALID_ARGUMENT, "n_heads=%d < 1", n_heads);
  const auto* kc = static_cast<const aatc_calib*>(kblobs);
  const auto* vc = static_cast<const aatc_calib*>(vblobs);
  const int d = AATC_D;
  int max_k = AATC_MAX_BITS, max_v = AATC_MAX_BITS;
  for (int h = 0; h < n_heads; ++h) {
    aatc_status st = aatc_calib_validate(kc + h, sizeof(aatc_calib));
    if (st == AATC_OK) st = aatc_calib_validate(vc + h, sizeof(aatc_calib));
    if (st != AATC_OK) return st;
    max_k = std::min(max_k, static_cast<int>(kc[h].max_bits));
    max_v = std::min(max_v, static_cast<int>(vc[h].max_bits));
  }
  if (kw)
    for (int64_t i = 0; i < static_cast<int64_t>(n_heads) * d; ++i) {
      if (!std::isfinite(kw[i])) return fail(AATC_ERR_NUMERICAL, "k_weight[%lld] is not finite", (long long)i);
      if (kw[i] < 0.0) return fail(AATC_ERR_INVALID_ARGUMENT, "k_weight[%lld] < 0", (long long)i);
    }
  // each tensor stays on the summed-code cache pass of decode attention (AATC_MAX_ATTN_BITS per vector)
  const int cap_k = std::min(d * max_k, AATC_MAX_ATTN_BITS), cap_v = std::min(d * max_v, AATC_MAX_ATTN_BITS);
  if (total < 0 || total > cap_k + cap_v)
    return fail(AATC_ERR_BUDGET, "total_bits %d outside [0, %d] (each tensor at most %d bits per vector)", total,
                cap_k + cap_v, AATC_MAX_ATTN_BITS);
  const double sc = scale > 0.f ? static_cast<double>(scale) : 1.0 / std::sqrt(static_cast<double>(d));
  std::vector<double> ks(static_cast<size_t>(n_heads) * d), lam(n_heads);
  for (int h = 0; h < n_heads; ++h) {
    double tr = 0.0;
    for (int i = 0; i < d; ++i) {
      ks[h * d + i] = kw ? kw[h * d + i] * kc[h].sigma2[i] : kc[h].sigma2[i];
      tr += vc[h].sigma2[i];
    }
    lam[h] = sc * sc * tr;
  }
  auto dist = [&](const double* s2, int budget, int max_bits) {
    uint8_t bits[AATC_D];
    waterfill_impl(s2, d, budget, max_bits, bits);
    double t = 0.0;
    for (int i = 0; i < d; ++i) t += std::ldexp(s2[i], -2 * bits[i]);
    return t;
  };
  const int lo = std::max(0, total - cap_v), hi = std::min(total, cap_k);
  std::vector<double> tot(hi - lo + 1);
  for (int bk = lo; bk <= hi; ++bk) {
    double t = 0.0;
    for (int h = 0; h < n_heads; ++h) {
      t += lam[h] * dist(&ks[h * d], bk, max_k);
      t += dist(vc[h].sigma2, total - bk, max_v);
    }
    tot[bk - lo] = t;
  }
  double best = tot[0];
  for (double t : tot) best = std::min(best, t);
  int pick = 0;
  while (!(tot[pick] <= best * (1.0 + 1e-12))) ++pick;
  *bk_out = lo + pick;
  *bv_out = total - lo - pick;
  return AATC_OK;
}

int32_t aatc_calib_v_tiles(const void* blob) {
  if (!blob) return -1;
  const auto* c = static_cast<const aatc_calib*>(blob);
  if (c->magic != AATC_MAGIC || c->d != AATC_D) return -1;
  return (c->n_fields4 + 15) / 16 + (c->n_fields2 + 15) / 16 + (c->n_fields1 + 15) / 16;
}

}  // extern "C"
