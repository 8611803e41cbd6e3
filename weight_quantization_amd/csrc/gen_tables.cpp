// Build-time generator of the HLWQ codebook tables.
//
// Prints a C header (to stdout) with, for Q5 (K = 32) and Q3 (K = 8):
//   * the Lloyd-Max centroids for N(0, 1), rounded to fp32, ascending
//     (model card "Qwen3.6-35B-A3B — HLWQ Q5", section "Method", step [4];
//     "Qwopus3.6-27B-v2 · HLWQ Q5", "Methodology notes": centroids computed for a
//     unit Gaussian, 32 for weights, 8 for the 3-bit KV cache);
//   * the decision thresholds: the largest fp32 value not above the exact
//     midpoint of two neighbouring fp32 centroids, so "number of thresholds
//     strictly below y" is the index of the nearest centroid, ties low;
//   * the bucket table the kernels use to find a code with one compare.
//
// Bucket search.  For a rotated value y the kernels form, in fp32,
//   u = y + O            (one rounding; O lies in [2^16, 2^17), ulp 1/128)
// and read 8 bytes at LDS byte offset  bits(u) & MASK.  Every u the kernels
// can produce lies in one aligned window of that binade in which mantissa
// bits 4 and up count buckets of width 1/8 (16 ulps), so the masked bits are
// the byte offset of a 16-byte entry with no shift; bit 3 of u (which half of
// its bucket y fell in) picks one of two identical 8-byte copies inside the
// entry, which spreads the reads of a wave over twice as many LDS banks.  The entry is
// {threshold t_k or +inf, base_k} and the code is base_k + (y > t_k).
// Buckets are narrower than the smallest gap between thresholds, so each holds
// at most one threshold; base_k counts the thresholds below the bucket.  The
// add is monotone and the bucket edges are representable, so rounding can only
// move a y lying at most 1/256 below an edge up into the next bucket; the
// result stays exact as long as no threshold lies that close below an edge.
// The phase of the edges (O modulo 1/8) is chosen per table to keep every
// threshold at least 1/128 below the next edge; this program then verifies the
// search by brute force against the plain count on every fp32 value near
// every threshold and edge, plus a dense sweep, and exits non-zero (failing
// the build) on any disagreement.
//
// |y| <= sqrt(128) * (1 + 2e-6) for every finite 128-block (Cauchy-Schwarz on
// the unit-norm rotated block), inside the 32-wide window of the weight
// tables (256 entries, MASK 0xff8); 256-wide KV vectors reach |y| <= 16, so
// their table spans a 64-wide window (512 entries, MASK 0x1ff8).

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

struct Tables {
  int K;
  std::vector<float> cent, thr;
  std::vector<uint32_t> search;  // 16-byte entries {threshold bits, base} x 2
  float offset = 0.0f;           // O
  uint32_t mask = 0;             // byte-offset mask of bits(u)
};

// code by definition: number of thresholds strictly below y
uint32_t count_code(const std::vector<float>& thr, float y) {
  uint32_t n = 0;
  for (float t : thr) n += (y > t) ? 1u : 0u;
  return n;
}

constexpr double kU0 = 98304.0;  // 1.5 * 2^16: start of the window, low 13 mantissa bits zero

uint32_t bucket_code(const Tables& tb, float y) {
  const float u = y + tb.offset;  // one fp32 rounding, as on the device
  uint32_t bits;
  std::memcpy(&bits, &u, 4);
  const uint32_t off = (bits & tb.mask) >> 2;  // word index of the 8-byte copy read
  float t;
  std::memcpy(&t, &tb.search[off], 4);
  return tb.search[off + 1] + ((y > t) ? 1u : 0u);
}

// y-interval [lo, hi) of bucket k for window offset O
void bucket_range(int k, double O, double* lo, double* hi) {
  *lo = kU0 + k / 8.0 - O;
  *hi = kU0 + (k + 1) / 8.0 - O;
}

Tables make_tables(int K, int entries, uint32_t mask) {
  Tables tb;
  tb.K = K;
  tb.mask = mask;
  const std::vector<double> c = lloyd_max(K);
  for (double v : c) tb.cent.push_back((float)v);
  for (int k = 0; k + 1 < K; ++k) {
    const double m = 0.5 * ((double)tb.cent[k] + (double)tb.cent[k + 1]);  // exact
    float b = (float)m;
    if ((double)b > m) b = std::nextafterf(b, -INFINITY);
    tb.thr.push_back(b);
  }
  // window centred on y = 0; the phase (steps of 1/64) is chosen to keep the
  // largest distance between every threshold and the bucket edge above it
  // (only a value just below an edge can be rounded into the next bucket)
  const double half = entries / 16.0;  // half the window width in y
  double best_phase = -1, best_gap = -1;
  for (int j = 0; j < 16; ++j) {
    const double phase = j / 128.0;
    double gap = 1e9;
    for (float t : tb.thr) {
      const double r = std::fmod((double)t + half + phase, 0.125);  // position inside its bucket
      const double rr = r < 0 ? r + 0.125 : r;
      gap = std::fmin(gap, 0.125 - rr);
    }
    if (gap > best_gap) { best_gap = gap; best_phase = phase; }
  }
  if (best_gap < 1.0 / 128.0) {
    std::fprintf(stderr, "gen_tables: no bucket phase keeps thresholds 1/128 below the edges (K=%d)\n", K);
    std::exit(1);
  }
  const double O = kU0 + half + best_phase;
  tb.offset = (float)O;
  if ((double)tb.offset != O) {
    std::fprintf(stderr, "gen_tables: window offset not representable\n");
    std::exit(1);
  }
  for (int k = 0; k < entries; ++k) {
    double lo, hi;
    bucket_range(k, O, &lo, &hi);
    uint32_t base = 0;
    int inside = 0;
    float t_in = INFINITY;
    for (float t : tb.thr) {
      if ((double)t < lo) ++base;
      else if ((double)t < hi) { ++inside; t_in = t; }
    }
    if (inside > 1) {
      std::fprintf(stderr, "gen_tables: bucket %d holds %d thresholds\n", k, inside);
      std::exit(1);
    }
    tb.search.push_back(f2u(t_in));
    tb.search.push_back(base);
    tb.search.push_back(f2u(t_in));
    tb.search.push_back(base);
  }
  // brute-force verification over the reachable range |y| < half - 1/8
  const float ymax = (float)(half - 0.25);
  std::vector<float> probes;
  for (float t : tb.thr) probes.push_back(t);
  for (int k = 0; k <= entries; ++k) {
    double lo, hi;
    bucket_range(k, O, &lo, &hi);
    probes.push_back((float)lo);
  }
  probes.push_back(0.0f);
  for (float p : probes) {
    float lo = p, hi = p;
    for (int i = 0; i < 4096; ++i) {
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
  for (int64_t i = -20000000; i <= 20000000; ++i) {
    const float y = (float)((double)i * (ymax / 20000000.0));
    if (count_code(tb.thr, y) != bucket_code(tb, y)) {
      std::fprintf(stderr, "gen_tables: bucket search wrong at y=%a\n", y);
      std::exit(1);
    }
  }
  for (float y : {0.0f, -0.0f}) {
    if (count_code(tb.thr, y) != bucket_code(tb, y)) {
      std::fprintf(stderr, "gen_tables: bucket search wrong at signed zero\n");
      std::exit(1);
    }
  }
  return tb;
}

void emit_floats(const char* name, const std::vector<float>& v) {
  std::printf("#define %s { \\\n", name);
  for (size_t i = 0; i < v.size(); ++i)
    std::printf("  %af%s\n", (double)v[i], i + 1 < v.size() ? ", \\" : " }");
}

void emit_words(const char* name, const std::vector<uint32_t>& v) {
  std::printf("#define %s { \\\n", name);
  for (size_t i = 0; i < v.size(); i += 4)
    std::printf("  0x%08" PRIx32 "u, %" PRIu32 "u, 0x%08" PRIx32 "u, %" PRIu32 "u%s\n", v[i], v[i + 1], v[i + 2],
                v[i + 3], i + 4 < v.size() ? ", \\" : " }");
}

}  // namespace

int main() {
  const Tables q5 = make_tables(32, 256, 0xff8u);
  const Tables q3 = make_tables(8, 256, 0xff8u);
  const Tables kv3 = make_tables(8, 512, 0x1ff8u);
  std::printf("// Generated at build time by gen_tables.cpp: Lloyd-Max tables for N(0,1).\n");
  std::printf("#pragma once\n");
  std::printf("#define HLWQ_SEARCH_ENTRIES 256\n#define HLWQ_SEARCH_MASK 0xff8u\n");
  std::printf("#define HLWQ_SEARCH_OFFSET_5 %af\n#define HLWQ_SEARCH_OFFSET_3 %af\n", (double)q5.offset,
              (double)q3.offset);
  std::printf("#define HLWQ_KV_SEARCH_ENTRIES 512\n#define HLWQ_KV_SEARCH_MASK 0x1ff8u\n");
  std::printf("#define HLWQ_KV_SEARCH_OFFSET %af\n", (double)kv3.offset);
  emit_floats("HLWQ_CENTROIDS_5", q5.cent);
  emit_floats("HLWQ_THRESHOLDS_5", q5.thr);
  emit_words("HLWQ_SEARCH_5", q5.search);
  emit_floats("HLWQ_CENTROIDS_3", q3.cent);
  emit_floats("HLWQ_THRESHOLDS_3", q3.thr);
  emit_words("HLWQ_SEARCH_3", q3.search);
  emit_words("HLWQ_KV_SEARCH_3", kv3.search);
  return 0;
}
