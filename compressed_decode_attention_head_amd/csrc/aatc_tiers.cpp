// Token tiers: a joint token x channel allocation of the bit budget (host, fp64).
//
// Page "SPHERICAL KV ..." (RDKV abstract): a token's width may be anything from uncompressed to
// nothing (eviction), set by reverse water-filling once after prefill.  Page "KV Cache
// Compression Through the Lens of Transform Coding" (Key points): the attention output's
// distortion factors over tokens and channels.
//
// Each token gets a tier tau in {0, 2, 4, 16} bits per element: 0 evicts it, 2 and 4 code it
// with that tier's water-filling (same rotation), 16 keeps it as raw bf16.  A tier costs
// D(tau) = sum over K and V of sum_i sigma_i^2 4^-b_i(tau), with D(0) the total variance and
// D(16) = 0.  Token t weighs a_t^2 (its softmax mass squared: the output error is the
// mass-weighted sum of value errors).  For a multiplier lambda every token takes
// argmin_tau a_t^2 D(tau) + lambda d tau (ties to the lower tier); lambda is bisected to the
// smallest value whose bit total fits avg_bits * n * d.
#include <cmath>
#include <cstdint>
#include <vector>

#include "aatc_internal.h"

namespace {

constexpr int kTiers[4] = {0, 2, 4, 16};

void tiers_at(const std::vector<double>& w, const double* dist, double lam, int d, int8_t* out, int64_t* total) {
  const double ld = lam * d;
  int64_t sum = 0;
  for (size_t t = 0; t < w.size(); ++t) {
    int best = 0;
    double bc = w[t] * dist[0] + ld * kTiers[0];
    for (int j = 1; j < 4; ++j) {
      const double c = w[t] * dist[j] + ld * kTiers[j];
      if (c < bc) {          // strict: ties keep the lower tier
        bc = c;
        best = j;
      }
    }
    if (out) out[t] = static_cast<int8_t>(kTiers[best]);
    sum += kTiers[best];
  }
  *total = sum * d;
}

}  // namespace

extern "C" {

aatc_status aatc_tier_distortions(const double* sigma2, int32_t n_tensors, int32_t d, int32_t max_bits,
                                  double dist_out[4]) {
  aatc::clear_error();
  if (!sigma2 || !dist_out || n_tensors < 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer or no tensor");
  if (d != AATC_D) return aatc::fail(AATC_ERR_UNSUPPORTED, "d=%d (only 128)", d);
  if (max_bits < 4 || max_bits > AATC_MAX_BITS)
    return aatc::fail(AATC_ERR_BUDGET, "max_bits %d: the 4-bit tier needs 4..8", max_bits);
  for (int64_t i = 0; i < static_cast<int64_t>(n_tensors) * d; ++i)
    if (!std::isfinite(sigma2[i]) || sigma2[i] < 0.0) return aatc::fail(AATC_ERR_NUMERICAL, "sigma2[%lld]", (long long)i);
  for (int j = 0; j < 4; ++j) {
    double tot = 0.0;
    for (int s = 0; s < n_tensors; ++s) {
      const double* s2 = sigma2 + static_cast<int64_t>(s) * d;
      if (kTiers[j] == 0) {
        for (int i = 0; i < d; ++i) tot += s2[i];
      } else if (kTiers[j] < 16) {
        uint8_t bits[AATC_D];
        aatc::waterfill(s2, d, kTiers[j] * d, max_bits, bits);
        for (int i = 0; i < d; ++i) tot += s2[i] * std::ldexp(1.0, -2 * bits[i]);
      }
    }
    dist_out[j] = tot;
  }
  return AATC_OK;
}

aatc_status aatc_token_tiers(const double* attn_mass, int64_t n, const double dist[4], int32_t d, double avg_bits,
                             int8_t* tiers_out) {
  aatc::clear_error();
  if (!attn_mass || !dist || !tiers_out || n < 0) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "null pointer or n < 0");
  if (d < 1) return aatc::fail(AATC_ERR_INVALID_ARGUMENT, "d=%d", d);
  if (!(avg_bits >= 0.0 && avg_bits <= 16.0)) return aatc::fail(AATC_ERR_BUDGET, "avg_bits %g outside [0, 16]", avg_bits);
  for (int j = 0; j < 4; ++j)
    if (!std::isfinite(dist[j]) || dist[j] < 0.0) return aatc::fail(AATC_ERR_NUMERICAL, "dist[%d]", j);
  std::vector<double> w(static_cast<size_t>(n));
  for (int64_t t = 0; t < n; ++t) {
    if (!std::isfinite(attn_mass[t]) || attn_mass[t] < 0.0)
      return aatc::fail(AATC_ERR_NUMERICAL, "attn_mass[%lld]", (long long)t);
    w[t] = attn_mass[t] * attn_mass[t];
  }
  const double budget = avg_bits * static_cast<double>(n) * d;
  int64_t tot = 0;
  tiers_at(w, dist, 0.0, d, nullptr, &tot);
  if (static_cast<double>(tot) <= budget) {
    tiers_at(w, dist, 0.0, d, tiers_out, &tot);
    return AATC_OK;
  }
  double lo = 0.0, hi = 1.0;
  for (int it = 0;; ++it) {
    tiers_at(w, dist, hi, d, nullptr, &tot);
    if (static_cast<double>(tot) <= budget) break;
    if (it > 2000) return aatc::fail(AATC_ERR_NUMERICAL, "no multiplier meets the budget");
    hi *= 2.0;
  }
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    tiers_at(w, dist, mid, d, nullptr, &tot);
    if (static_cast<double>(tot) > budget) lo = mid;
    else hi = mid;
  }
  tiers_at(w, dist, hi, d, tiers_out, &tot);
  return AATC_OK;
}

}  // extern "C"
