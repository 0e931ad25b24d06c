// Drives every host-side entry point of the library (calibration, the query statistics, the joint
// K/V split, token tiers, blob validation, sizes and status strings) over ordinary and error
// inputs.  Built from the host sources alone with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitizers.py; any sanitizer report aborts with a non-zero status, and every
// status is checked against the one the header documents.  It checks no numerics: the oracle
// tests do that.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "aatc.h"

namespace {

int g_fail = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s\n", what);
    ++g_fail;
  }
}

void expect(aatc_status got, aatc_status want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d (%s), want %d; %s\n", what, static_cast<int>(got),
                 aatc_status_string(got), static_cast<int>(want), aatc_last_error());
    ++g_fail;
  }
}

// xorshift64* and Box-Muller: a seeded stream of normal deviates for the inputs
struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 2654435761u + 1) {}
  double uniform() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return ((s * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
  }
  double normal() {
    const double u = uniform() + 1e-300, v = uniform();
    return std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v);
  }
};

// rows with a decaying spectrum, some correlation between neighbours and two large coordinates
std::vector<double> make_rows(int n, int d, uint64_t seed) {
  Rng r(seed);
  std::vector<double> x(static_cast<size_t>(n) * d);
  for (int t = 0; t < n; ++t) {
    double prev = 0.0;
    for (int i = 0; i < d; ++i) {
      const double z = r.normal() * std::pow(1.0 + i, -0.75);
      x[static_cast<size_t>(t) * d + i] = z + 0.3 * prev + (i == 5 || i == 77 ? 10.0 * z : 0.0);
      prev = z;
    }
  }
  return x;
}

std::vector<float> to_f32(const std::vector<double>& x) { return std::vector<float>(x.begin(), x.end()); }

std::vector<uint16_t> to_bf16(const std::vector<double>& x) {
  std::vector<uint16_t> y(x.size());
  for (size_t k = 0; k < x.size(); ++k) {
    const float f = static_cast<float>(x[k]);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest even
    y[k] = static_cast<uint16_t>(u >> 16);
  }
  return y;
}

}  // namespace

int main() {
  const int d = AATC_D;
  const size_t cb = aatc_calib_bytes(d);
  if (cb == 0 || aatc_calib_bytes(64) != 0) {
    std::fprintf(stderr, "FAIL aatc_calib_bytes\n");
    return 1;
  }
  check(aatc_bits_budget(1.33, d) == 170 && aatc_bits_budget(-1.0, d) == -1 && aatc_bits_budget(9.0, d) == -1,
        "bits_budget");
  check(aatc_packed_bytes(170, 65) == 2 * 8 * 170u, "packed_bytes");
  for (int s = 0; s <= 8; ++s) (void)std::strlen(aatc_status_string(static_cast<aatc_status>(s)));

  const int n = 600;
  const std::vector<double> x64 = make_rows(n, d, 1);
  const std::vector<float> x32 = to_f32(x64);
  const std::vector<uint16_t> x16 = to_bf16(x64);
  const std::vector<double> q64 = make_rows(300, d, 2);

  std::vector<double> moment(static_cast<size_t>(d) * d);
  expect(aatc_query_moment(q64.data(), AATC_F64, 300, d, moment.data()), AATC_OK, "query_moment");
  expect(aatc_query_moment(nullptr, AATC_F64, 300, d, moment.data()), AATC_ERR_INVALID_ARGUMENT, "query_moment null");
  expect(aatc_query_moment(q64.data(), AATC_F64, 0, d, moment.data()), AATC_ERR_INVALID_ARGUMENT, "query_moment n=0");

  // every rotation, quantizer, dtype and a spread of budgets
  std::vector<uint8_t> blob(cb), kblobs(2 * cb), vblobs(2 * cb);
  const double budgets[] = {0.0, 0.5, 1.33, 2.76, 4.0, 8.0};
  for (int rot = 0; rot < 4; ++rot) {
    for (int qz = 0; qz < 2; ++qz) {
      for (double bpe : budgets) {
        for (int dt = 0; dt < 3; ++dt) {
          aatc_calib_params p{};
          p.d = d;
          p.rotation = rot;
          p.bits_per_elem = bpe;
          p.max_bits = 8;
          p.quantizer = qz;
          p.query_moment = rot == AATC_ROT_NOVA ? moment.data() : nullptr;
          const void* src = dt == 0 ? static_cast<const void*>(x32.data())
                                    : dt == 1 ? static_cast<const void*>(x16.data()) : static_cast<const void*>(x64.data());
          expect(aatc_calibrate(&p, src, static_cast<aatc_dtype>(dt), n, d, blob.data(), cb), AATC_OK, "calibrate");
          expect(aatc_calib_validate(blob.data(), cb), AATC_OK, "validate");
          check(aatc_calib_v_tiles(blob.data()) >= 0, "v_tiles");
        }
      }
    }
  }

  // attention-aware keys: channel weights from a KLT key blob, then the joint split
  aatc_calib_params p{};
  p.d = d;
  p.rotation = AATC_ROT_KLT;
  p.bits_per_elem = 2.76;
  p.max_bits = 8;
  std::vector<double> w(2 * d);
  for (int h = 0; h < 2; ++h) {
    const std::vector<double> xk = make_rows(n, d, 10 + h), xv = make_rows(n, d, 20 + h);
    expect(aatc_calibrate(&p, xk.data(), AATC_F64, n, d, kblobs.data() + h * cb, cb), AATC_OK, "calibrate K");
    expect(aatc_calibrate(&p, xv.data(), AATC_F64, n, d, vblobs.data() + h * cb, cb), AATC_OK, "calibrate V");
    expect(aatc_query_channel_weights(kblobs.data() + h * cb, cb, q64.data(), AATC_F64, 300, d, w.data() + h * d),
           AATC_OK, "query_channel_weights");
  }
  p.channel_weight = w.data();
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb), AATC_OK, "calibrate weighted");
  p.channel_weight = nullptr;
  for (int tb : {0, 1, 170, 340, 706, 1024}) {
    int32_t bk = -1, bv = -1;
    expect(aatc_joint_kv_split(kblobs.data(), vblobs.data(), 2, w.data(), 0.f, tb, &bk, &bv), AATC_OK, "split");
    expect(aatc_joint_kv_split(kblobs.data(), vblobs.data(), 2, nullptr, 0.1f, tb, &bk, &bv), AATC_OK, "split unweighted");
    check(bk >= 0 && bv >= 0 && bk + bv == tb && bk <= AATC_MAX_ATTN_BITS && bv <= AATC_MAX_ATTN_BITS, "split range");
  }
  int32_t bk, bv;
  expect(aatc_joint_kv_split(kblobs.data(), vblobs.data(), 2, nullptr, 0.f, 1025, &bk, &bv), AATC_ERR_BUDGET, "split over");
  expect(aatc_joint_kv_split(kblobs.data(), vblobs.data(), 0, nullptr, 0.f, 100, &bk, &bv), AATC_ERR_INVALID_ARGUMENT,
         "split n_heads");

  // error paths of calibration and validation
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb - 1), AATC_ERR_BUFFER_TOO_SMALL, "small blob");
  expect(aatc_calibrate(&p, nullptr, AATC_F64, n, d, blob.data(), cb), AATC_ERR_INVALID_ARGUMENT, "null rows");
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, 1, d, blob.data(), cb), AATC_ERR_INVALID_ARGUMENT, "one row");
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d - 1, blob.data(), cb), AATC_ERR_INVALID_ARGUMENT, "stride");
  p.quantizer = 2;
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb), AATC_ERR_INVALID_ARGUMENT, "quantizer");
  p.quantizer = 0;
  p.bits_per_elem = 8.5;
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb), AATC_ERR_BUDGET, "budget");
  p.bits_per_elem = 2.0;
  p.rotation = AATC_ROT_NOVA;
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb), AATC_ERR_INVALID_ARGUMENT, "nova no moment");
  p.rotation = AATC_ROT_KLT;
  std::vector<double> bad = x64;
  bad[17] = std::nan("");
  expect(aatc_calibrate(&p, bad.data(), AATC_F64, n, d, blob.data(), cb), AATC_ERR_NUMERICAL, "nan row");
  p.d = 64;
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb), AATC_ERR_UNSUPPORTED, "d");
  p.d = d;
  expect(aatc_calibrate(&p, x64.data(), AATC_F64, n, d, blob.data(), cb), AATC_OK, "calibrate again");
  std::vector<uint8_t> broken = blob;
  broken[cb / 2] ^= 0x5a;
  expect(aatc_calib_validate(broken.data(), cb), AATC_ERR_BAD_ARTEFACT, "checksum");
  expect(aatc_calib_validate(blob.data(), cb - 8), AATC_ERR_BUFFER_TOO_SMALL, "validate size");
  std::vector<uint8_t> nomagic = blob;
  nomagic[0] ^= 1;
  check(aatc_calib_v_tiles(nomagic.data()) == -1 && aatc_calib_v_tiles(nullptr) == -1, "v_tiles of a bad blob");

  // token tiers
  std::vector<double> s2(2 * d);
  for (int i = 0; i < 2 * d; ++i) s2[i] = std::pow(1.0 + (i % d), -1.5);
  double dist[4];
  expect(aatc_tier_distortions(s2.data(), 2, d, 8, dist), AATC_OK, "tier_distortions");
  expect(aatc_tier_distortions(s2.data(), 2, d, 3, dist), AATC_ERR_BUDGET, "tier max_bits");
  Rng r(3);
  for (int64_t nt : {0, 1, 7, 5000}) {
    std::vector<double> mass(static_cast<size_t>(nt) + 1);
    for (int64_t t = 0; t < nt; ++t) mass[t] = std::pow(1.0 + t, -1.1) * (0.5 + r.uniform());
    std::vector<int8_t> tiers(static_cast<size_t>(nt) + 1);
    for (double ab : {0.0, 0.5, 2.76, 16.0}) {
      expect(aatc_token_tiers(mass.data(), nt, dist, d, ab, tiers.data()), AATC_OK, "token_tiers");
      for (int64_t t = 0; t < nt; ++t)
        check(tiers[t] == 0 || tiers[t] == 2 || tiers[t] == 4 || tiers[t] == 16, "tier value");
    }
  }
  std::vector<double> one(1, -1.0);
  std::vector<int8_t> tt(1);
  expect(aatc_token_tiers(one.data(), 1, dist, d, 2.0, tt.data()), AATC_ERR_NUMERICAL, "negative mass");
  expect(aatc_token_tiers(one.data(), 1, dist, d, 17.0, tt.data()), AATC_ERR_BUDGET, "tier budget");

  if (g_fail) {
    std::fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  std::printf("host driver: all checks passed\n");
  return 0;
}
