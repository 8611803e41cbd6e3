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
// Bucket search.  For a rotated value y the kernels form
//   k = (uint32_t) fmaf(y, 8, 96)            (round to nearest, then truncate)
// and read entry k = {threshold t_k or +inf, base_k}; the code is
//   base_k + (y > t_k).
// Bucket k nominally holds y in [(k - 96) / 8, (k - 95) / 8).  Because the
// buckets are narrower than the smallest gap between thresholds, each holds at
// most one threshold; base_k counts the thresholds below the bucket.  Rounding
// in the fma can only move a y that lies just below a bucket edge up into the
// next bucket (rounding is monotone and the edges are representable), so the
// result stays exact as long as no threshold lies within that rounding
// distance below an edge.  This program checks that condition with a wide
// margin and then verifies the search by brute force against the plain count
// on every fp32 value near every threshold and edge, plus a dense sweep; it
// exits non-zero, failing the build, if anything disagrees.
//
// |y| <= sqrt(128) * (1 + 2e-6) for every finite block (Cauchy-Schwarz on the
// unit-norm rotated block), so k stays inside [5, 187) and 192 entries cover
// every reachable bucket; the same bound holds for the 256-wide KV vectors,
// whose values are at most sqrt(256) = 16 in magnitude, so their table is
// indexed with fmaf(y, 8, 136) into 272 entries.

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
  std::vector<uint32_t> search;  // pairs {threshold bits, base}
};

// code by definition: number of thresholds strictly below y
uint32_t count_code(const std::vector<float>& thr, float y) {
  uint32_t n = 0;
  for (float t : thr) n += (y > t) ? 1u : 0u;
  return n;
}

uint32_t bucket_code(const Tables& tb, float y, float offset) {
  const float u = std::fmaf(y, 8.0f, offset);
  const uint32_t k = u > 0.0f ? (uint32_t)u : 0u;  // device: v_cvt_u32_f32 saturates at 0
  float t;
  uint32_t bits = tb.search[2 * k];
  std::memcpy(&t, &bits, 4);
  return tb.search[2 * k + 1] + ((y > t) ? 1u : 0u);
}

Tables make_tables(int K, int entries, int offset) {
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
  // bucket table
  const double margin = std::ldexp(1.0, -18);
  for (int k = 0; k < entries; ++k) {
    const double lo = (k - offset) / 8.0, hi = (k - offset + 1) / 8.0;
    uint32_t base = 0;
    int inside = 0;
    float t_in = INFINITY;
    for (float t : tb.thr) {
      if ((double)t < lo) ++base;
      else if ((double)t < hi) { ++inside; t_in = t; }
      if ((double)t > lo - margin && (double)t < lo) {
        std::fprintf(stderr, "gen_tables: threshold %.9g too close below bucket edge %.9g\n", t, lo);
        std::exit(1);
      }
    }
    if (inside > 1) {
      std::fprintf(stderr, "gen_tables: bucket %d holds %d thresholds\n", k, inside);
      std::exit(1);
    }
    if (k == 0 && inside) {
      std::fprintf(stderr, "gen_tables: lowest bucket must hold no threshold\n");
      std::exit(1);
    }
    tb.search.push_back(f2u(t_in));
    tb.search.push_back(base);
  }
  // brute-force verification of the bucketed search
  const float foff = (float)offset;
  const float ymax = (entries - offset) / 8.0f - 0.25f;
  std::vector<float> probes;
  for (float t : tb.thr) probes.push_back(t);
  for (int k = 0; k <= entries; ++k) probes.push_back((k - offset) / 8.0f);
  for (float p : probes) {
    float lo = p, hi = p;
    for (int i = 0; i < 4096; ++i) {
      lo = std::nextafterf(lo, -INFINITY);
      hi = std::nextafterf(hi, INFINITY);
      for (float y : {lo, hi, p}) {
        if (!(std::fabs(y) < ymax)) continue;
        if (count_code(tb.thr, y) != bucket_code(tb, y, foff)) {
          std::fprintf(stderr, "gen_tables: bucket search wrong at y=%a\n", y);
          std::exit(1);
        }
      }
    }
  }
  for (int64_t i = -20000000; i <= 20000000; ++i) {
    const float y = (float)((double)i * (ymax / 20000000.0));
    if (count_code(tb.thr, y) != bucket_code(tb, y, foff)) {
      std::fprintf(stderr, "gen_tables: bucket search wrong at y=%a\n", y);
      std::exit(1);
    }
  }
  for (float y : {0.0f, -0.0f}) {
    if (count_code(tb.thr, y) != bucket_code(tb, y, foff)) {
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
  for (size_t i = 0; i < v.size(); i += 2)
    std::printf("  0x%08" PRIx32 "u, %" PRIu32 "u%s\n", v[i], v[i + 1], i + 2 < v.size() ? ", \\" : " }");
}

}  // namespace

int main() {
  const Tables q5 = make_tables(32, 192, 96);
  const Tables q3 = make_tables(8, 192, 96);
  const Tables kv3 = make_tables(8, 272, 136);
  std::printf("// Generated at build time by gen_tables.cpp: Lloyd-Max tables for N(0,1).\n");
  std::printf("#pragma once\n");
  std::printf("#define HLWQ_SEARCH_ENTRIES 192\n#define HLWQ_SEARCH_OFFSET 96.0f\n");
  std::printf("#define HLWQ_KV_SEARCH_ENTRIES 272\n#define HLWQ_KV_SEARCH_OFFSET 136.0f\n");
  emit_floats("HLWQ_CENTROIDS_5", q5.cent);
  emit_floats("HLWQ_THRESHOLDS_5", q5.thr);
  emit_words("HLWQ_SEARCH_5", q5.search);
  emit_floats("HLWQ_CENTROIDS_3", q3.cent);
  emit_floats("HLWQ_THRESHOLDS_3", q3.thr);
  emit_words("HLWQ_SEARCH_3", q3.search);
  emit_words("HLWQ_KV_SEARCH_3", kv3.search);
  return 0;
}
