// Build-time generator of the HLWQ codebook tables.
//
// Prints a C header (to stdout) with, for Q5 (K = 32), Q3 (K = 8) and the
// 2-bit KV variant (K = 4):
//   * the Lloyd-Max centroids for N(0, 1), rounded to fp32, ascending
//     (model card "Qwen3.6-35B-A3B — HLWQ Q5", section "Method", step [4];
//     "Qwopus3.6-27B-v2 · HLWQ Q5", "Methodology notes": centroids computed for a
//     unit Gaussian, 32 for weights, 8 for the 3-bit KV cache);
//   * the decision thresholds: the largest fp32 value not above the exact
//     midpoint of two neighbouring fp32 centroids, so "number of thresholds
//     strictly below y" is the index of the nearest centroid, ties low;
//   * the two tables the kernels use to find a code with one compare;
//   * for Q3, the same two tables for the mirrored search of TQ3 (below).
//
// Bucket search.  For a rotated value y the kernels form, in fp32,
//   u = fma(y, 2^-146, bias)       bias = C * 2^-149, a denormal, C even
// with one rounding.  For every reachable y the exact value 8 y 2^-149 + bias
// lies in the denormal range, whose spacing is 2^-149, so the bit pattern of u
// is the integer k = RN(8 y + C) (ties to even): the index of a bucket of
// width 1/8.  k is used as a byte address with no masking:
//   bucket table  B[k] = 8 * base_k, base_k = number of thresholds below every
//                 y of bucket k;
//   entry table   E[b] = {threshold b (+inf for b = K - 1), b}, 8 bytes each;
//   code          = E[B[k]].b + (y > E[B[k]].threshold).
// The thresholds are further apart than 1/8, so a bucket holds at most one
// threshold, which is then threshold base_k; every other threshold is below
// all of the bucket or not below any of it, and the compare settles the rest.
// This program checks both facts and then verifies the search by brute force
// against the plain count on every fp32 value near every threshold and bucket
// edge, plus a dense sweep, and exits non-zero (failing the build) on any
// disagreement.
//
// Mirrored search (TQ3's output signs).  TQ3 codes -y where its sign vector
// D2 is -1.  The Q3 thresholds T are symmetric (t_k = -t_{K-2-k} exactly, as
// the centroids are), so for every fp32 y
//   #{t in T : t < -y} = #{t in T : t > y} = (K - 1) - #{t in T : t <= y}
//                      = (K - 1) - #{t' in T' : t' < y},  T' = {pred(t)},
// pred(t) the next fp32 value below t (t <= y iff pred(t) < y for fp32 y).
// So the code of -y is K - 1 - (the code of y searched among T'), and K - 1 - c
// = c ^ (K - 1): a bucket search over T' (bias C + number of buckets, its
// tables stored after the plain ones) plus one xor of the packed codes.  This
// program checks the symmetry and verifies that identity by brute force.
//
// Reach.  Let S be the exact squared norm of a block and s the computed one.
// Each of the R roundings of the norm sum (191 for a 128-block, 383 for a
// 256-vector) errs by at most 2^-24 of its result or 2^-150, so with s >= 2^-149
// (the smallest non-zero value) S / s <= (1 + 2^-24 R)(1 + R / 2).  As every
// rotated value obeys |z| <= sqrt(L S), |y| = |z| / s^(1/2) stays below
// sqrt(128 * 96.5) < 112 for weights and sqrt(256 * 192.5) < 222 for KV
// vectors (including the fp32 error of the butterflies), inside the 2048- and
// 4096-bucket tables (|y| < 128 and < 256).  Blocks whose squares underflow are
// exactly where s underestimates S; for the rest |y| <= sqrt(L) (1 + 2e-6).

#include <cinttypes>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

namespace {

const double kInf = std::numeric_limits<double>::infinity();

// Extent of the brute-force checks: ulps probed on each side of every
// threshold and bucket edge, and sweep points on each side of zero.  The build
// uses the full check; HLWQ_GEN_QUICK=1 (the sanitizer test, which runs this
// program under AddressSanitizer and UBSan) a smaller one.  The tables printed
// do not depend on it.
int g_near = 4096;
int64_t g_sweep = 20000000;

double gauss_pdf(double t) {
  if (std::isinf(t)) return 0.0;
  return std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI);
}

// P(X > t), X ~ N(0, 1)
double upper_tail(double t) { return 0.5 * std::erfc(t / std::sqrt(2.0)); }

// P(lo < X < hi), written with the tail that avoids cancellation
double cell_mass(double lo, double hi) {
  if (lo >= 0.0) return upper_tail(lo) - upper_tail(hi);
  return upper_tail(-hi) - upper_tail(-lo);
}

// Lloyd's iteration on the Gaussian density: thresholds at the midpoints,
// centroids at the conditional means of their cells; evenly spread start.
std::vector<double> lloyd_max(int K) {
  std::vector<double> c(K), next(K);
  for (int k = 0; k < K; ++k) c[k] = 3.0 * (2.0 * (k + 0.5) / K - 1.0);
  bool done = false;
  for (int it = 0; it < 1000000 && !done; ++it) {
    double delta = 0.0;
    for (int k = 0; k < K; ++k) {
      const double lo = k == 0 ? -kInf : 0.5 * (c[k - 1] + c[k]);
      const double hi = k == K - 1 ? kInf : 0.5 * (c[k] + c[k + 1]);
      next[k] = (gauss_pdf(lo) - gauss_pdf(hi)) / cell_mass(lo, hi);
      delta = std::fmax(delta, std::fabs(next[k] - c[k]));
    }
    c.swap(next);
    done = delta < 1e-15;
  }
  if (!done) {
    std::fprintf(stderr, "gen_tables: Lloyd iteration for K=%d did not converge\n", K);
    std::exit(1);
  }
  for (int k = 0; k < K / 2; ++k) {  // exact symmetry c_k = -c_{K-1-k}
    const double v = 0.5 * (c[K - 1 - k] - c[k]);
    c[k] = -v;
    c[K - 1 - k] = v;
  }
  return c;
}

uint32_t f2u(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

float u2f(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

constexpr float kScale = 0x1p-146f;  // 8 * 2^-149

struct Tables {
  int K;
  std::vector<float> cent, thr;
  std::vector<uint8_t> bucket;   // B[k] = 8 * base_k
  std::vector<uint32_t> entry;   // E[b] = {threshold bits, b}
  uint32_t bias = 0;             // bits of the denormal bias (= C)
};

// code by definition: number of thresholds strictly below y
uint32_t count_code(const std::vector<float>& thr, float y) {
  uint32_t n = 0;
  for (float t : thr) n += (y > t) ? 1u : 0u;
  return n;
}

// the kernels' search, with the same single-rounding fused multiply-add
uint32_t bucket_code(const Tables& tb, float y) {
  const uint32_t k = f2u(std::fmaf(y, kScale, u2f(tb.bias)));
  if (k >= tb.bucket.size()) {
    std::fprintf(stderr, "gen_tables: bucket index %u out of range at y=%a\n", k, y);
    std::exit(1);
  }
  const uint32_t e = tb.bucket[k] / 4u;
  return tb.entry[e + 1] + ((y > u2f(tb.entry[e])) ? 1u : 0u);
}

Tables make_tables(int K, int buckets) {
  Tables tb;
  tb.K = K;
  const std::vector<double> c = lloyd_max(K);
  for (double v : c) tb.cent.push_back((float)v);
  for (int k = 0; k + 1 < K; ++k) {
    const double m = 0.5 * ((double)tb.cent[k] + (double)tb.cent[k + 1]);  // exact
    float b = (float)m;
    if ((double)b > m) b = std::nextafterf(b, -INFINITY);
    tb.thr.push_back(b);
  }
  for (int k = 0; k + 2 < K; ++k) {
    if (!((double)tb.thr[k + 1] - (double)tb.thr[k] > 0.125)) {
      std::fprintf(stderr, "gen_tables: thresholds closer than one bucket (K=%d)\n", K);
      std::exit(1);
    }
  }
  const int C = buckets / 2;  // even; bucket C holds y = 0
  tb.bias = (uint32_t)C;
  // bucket k holds the y with k - 1/2 <= 8 y + C <= k + 1/2 (ties to even)
  for (int k = 0; k < buckets; ++k) {
    const double lo = (k - C - 0.5) / 8.0, hi = (k - C + 0.5) / 8.0;
    int base = 0, inside = 0;
    for (float t : tb.thr) {
      if ((double)t < lo) ++base;
      else if ((double)t < hi) ++inside;
    }
    if (inside > 1) {
      std::fprintf(stderr, "gen_tables: bucket %d holds %d thresholds\n", k, inside);
      std::exit(1);
    }
    tb.bucket.push_back((uint8_t)(8 * base));
  }
  for (int b = 0; b < K; ++b) {
    tb.entry.push_back(b + 1 < K ? f2u(tb.thr[b]) : f2u(INFINITY));
    tb.entry.push_back((uint32_t)b);
  }
  // brute-force verification over the reachable range |y| < buckets / 16
  const float ymax = (float)(buckets / 16.0 - 0.125);
  std::vector<float> probes;
  for (float t : tb.thr) probes.push_back(t);
  for (int k = 0; k <= buckets; ++k) probes.push_back((float)((k - C - 0.5) / 8.0));
  probes.push_back(0.0f);
  for (float p : probes) {
    float lo = p, hi = p;
    for (int i = 0; i < g_near; ++i) {
      lo = std::nextafterf(lo, -INFINITY);
      hi = std::nextafterf(hi, INFINITY);
      for (float y : {lo, hi, p}) {
        if (!(std::fabs(y) < ymax)) continue;
        if (count_code(tb.thr, y) != bucket_code(tb, y)) {
          std::fprintf(stderr, "gen_tables: bucket search wrong at y=%a\n", y);
          std::exit(1);
        }
      }
    }
  }
  for (int64_t i = -g_sweep; i <= g_sweep; ++i) {
    const float y = (float)((double)i * (ymax / (double)g_sweep));
    if (count_code(tb.thr, y) != bucket_code(tb, y)) {
      std::fprintf(stderr, "gen_tables: bucket search wrong at y=%a\n", y);
      std::exit(1);
    }
  }
  for (float y : {0.0f, -0.0f, 0x1p-149f, -0x1p-149f, 0x1p-126f, -0x1p-126f}) {
    if (count_code(tb.thr, y) != bucket_code(tb, y)) {
      std::fprintf(stderr, "gen_tables: bucket search wrong at y=%a\n", y);
      std::exit(1);
    }
  }
  return tb;
}

// The search tables over T' = {pred(t)} of a symmetric threshold set (see
// "Mirrored search" above), verified against the plain count of -y.
Tables mirror_tables(const Tables& tb) {
  const int K = tb.K;
  for (int k = 0; k + 1 < K; ++k) {
    if (tb.thr[k] != -tb.thr[K - 2 - k]) {
      std::fprintf(stderr, "gen_tables: thresholds not symmetric (K=%d)\n", K);
      std::exit(1);
    }
  }
  Tables m;
  m.K = K;
  m.cent = tb.cent;
  for (float t : tb.thr) m.thr.push_back(std::nextafterf(t, -INFINITY));
  const int buckets = (int)tb.bucket.size(), C = buckets / 2;
  m.bias = tb.bias;
  for (int k = 0; k < buckets; ++k) {
    const double lo = (k - C - 0.5) / 8.0, hi = (k - C + 0.5) / 8.0;
    int base = 0, inside = 0;
    for (float t : m.thr) {
      if ((double)t < lo) ++base;
      else if ((double)t < hi) ++inside;
    }
    if (inside > 1) {
      std::fprintf(stderr, "gen_tables: mirrored bucket %d holds %d thresholds\n", k, inside);
      std::exit(1);
    }
    m.bucket.push_back((uint8_t)(8 * base));
  }
  for (int b = 0; b < K; ++b) {
    m.entry.push_back(b + 1 < K ? f2u(m.thr[b]) : f2u(INFINITY));
    m.entry.push_back((uint32_t)b);
  }
  const float ymax = (float)(buckets / 16.0 - 0.125);
  auto check = [&](float y) {
    if (!(std::fabs(y) < ymax)) return;
    if ((bucket_code(m, y) ^ (uint32_t)(K - 1)) != count_code(tb.thr, -y)) {
      std::fprintf(stderr, "gen_tables: mirrored search wrong at y=%a\n", y);
      std::exit(1);
    }
  };
  std::vector<float> probes;
  for (float t : tb.thr) probes.push_back(t);
  for (int k = 0; k <= buckets; ++k) probes.push_back((float)((k - C - 0.5) / 8.0));
  probes.push_back(0.0f);
  for (float p : probes) {
    float lo = p, hi = p;
    for (int i = 0; i < g_near; ++i) {
      lo = std::nextafterf(lo, -INFINITY);
      hi = std::nextafterf(hi, INFINITY);
      check(lo);
      check(hi);
      check(p);
    }
  }
  for (int64_t i = -g_sweep; i <= g_sweep; ++i) check((float)((double)i * (ymax / (double)g_sweep)));
  for (float y : {0.0f, -0.0f, 0x1p-149f, -0x1p-149f, 0x1p-126f, -0x1p-126f}) check(y);
  return m;
}

void emit_floats(const char* name, const std::vector<float>& v) {
  std::printf("#define %s { \\\n", name);
  for (size_t i = 0; i < v.size(); ++i)
    std::printf("  %af%s\n", (double)v[i], i + 1 < v.size() ? ", \\" : " }");
}

void emit_words(const char* name, const std::vector<uint32_t>& v) {
  std::printf("#define %s { \\\n", name);
  for (size_t i = 0; i < v.size(); i += 2)
    std::printf("  0x%08" PRIx32 "u, %" PRIu32 "u%s\n", v[i], v[i + 1], i + 2 < v.size() ? ", \\" : " }");
}

// bucket bytes packed little-endian into 32-bit words (the kernels copy words)
void emit_bytes(const char* name, const std::vector<uint8_t>& v) {
  std::printf("#define %s { \\\n", name);
  for (size_t i = 0; i < v.size(); i += 16) {
    std::printf(" ");
    for (size_t j = i; j < i + 16; j += 4) {
      const uint32_t w = v[j] | (v[j + 1] << 8) | (v[j + 2] << 16) | ((uint32_t)v[j + 3] << 24);
      std::printf(" 0x%08" PRIx32 "u%s", w, j + 4 < v.size() ? "," : "");
    }
    std::printf("%s\n", i + 16 < v.size() ? " \\" : " }");
  }
}

}  // namespace

int main() {
  const char* quick = std::getenv("HLWQ_GEN_QUICK");
  if (quick && quick[0] == '1') {
    g_near = 64;
    g_sweep = 200000;
  }
  const Tables q5 = make_tables(32, 2048);
  const Tables q3 = make_tables(8, 2048);
  const Tables kv3 = make_tables(8, 4096);
  const Tables kv2 = make_tables(4, 4096);
  Tables q3m = mirror_tables(q3);
  // the mirrored entries follow the plain ones (K entries of 8 bytes)
  for (uint8_t& b : q3m.bucket) b = (uint8_t)(b + 8 * q3.K);
  std::printf("// Generated at build time by gen_tables.cpp: Lloyd-Max tables for N(0,1).\n");
  std::printf("#pragma once\n");
  std::printf("#define HLWQ_SEARCH_SCALE %af\n", (double)kScale);
  std::printf("#define HLWQ_BUCKETS %zu\n#define HLWQ_BUCKET_BIAS %uu\n", q5.bucket.size(), q5.bias);
  std::printf("#define HLWQ_KV_BUCKETS %zu\n#define HLWQ_KV_BUCKET_BIAS %uu\n", kv3.bucket.size(), kv3.bias);
  emit_floats("HLWQ_CENTROIDS_5", q5.cent);
  emit_floats("HLWQ_THRESHOLDS_5", q5.thr);
  emit_bytes("HLWQ_BUCKET_5", q5.bucket);
  emit_words("HLWQ_ENTRY_5", q5.entry);
  emit_floats("HLWQ_CENTROIDS_3", q3.cent);
  emit_floats("HLWQ_THRESHOLDS_3", q3.thr);
  emit_bytes("HLWQ_BUCKET_3", q3.bucket);
  emit_words("HLWQ_ENTRY_3", q3.entry);
  emit_bytes("HLWQ_BUCKET_3M", q3m.bucket);
  emit_words("HLWQ_ENTRY_3M", q3m.entry);
  emit_bytes("HLWQ_KV_BUCKET_3", kv3.bucket);
  emit_floats("HLWQ_CENTROIDS_2", kv2.cent);
  emit_floats("HLWQ_THRESHOLDS_2", kv2.thr);
  emit_words("HLWQ_ENTRY_2", kv2.entry);
  emit_bytes("HLWQ_KV_BUCKET_2", kv2.bucket);
  return 0;
}
