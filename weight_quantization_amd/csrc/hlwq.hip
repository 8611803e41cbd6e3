// hlwq.hip — HLWQ (Hadamard-Lloyd Weight Quantization) quantize / dequantize
// kernels for MI355X (gfx950) and the C ABI declared in include/hlwq.h.
//
// The path is a streaming codec: every 128-weight block (and every 256-wide KV
// head vector) is independent, and the work per byte moved is small, so the
// kernels are bound by HBM bandwidth and by VALU issue, never by a dense
// contraction; no matrix cores are used.
//
// Work mapping.  One work-item owns one whole 128-block: its 128 values live in
// VGPRs, so the norm tree, all 7 butterfly stages, the code search and the bit
// packing are lane-local, and the square root and reciprocal are paid once per
// 128 weights.  A KV head vector (256 values) is split over two adjacent lanes;
// only the last norm level and the last butterfly stage (stride 128) cross
// lanes, through a DPP quad permutation.
//
// Code search.  A rotated value y picks bucket k = (uint32_t) fmaf(y, 8, off)
// of a small LDS table {threshold, base}; the code is base + (y > threshold).
// The table is built and proven exact against the plain count at build time
// (gen_tables.cpp), so the kernels reproduce "number of fp32 thresholds below
// y" bit for bit with one compare.
//
// Rounding.  The file is compiled with -ffp-contract=off: every + and * below
// is one IEEE round-to-nearest operation in the order written, sqrtf and the
// division are correctly rounded, and the only fused multiply-adds are the
// explicit __builtin_fmaf calls whose product is exact (a multiply by 8 or by
// +-1), so no rounding differs from the operation order documented in
// include/hlwq.h.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>
#include <cstring>

#include "hlwq.h"
#include "hlwq_tables.inc"

namespace {

constexpr int kBlock = 128;    // weights per HLWQ block
constexpr int kKvDim = 256;    // KV head vector length
constexpr int kThreads = 256;  // work-items per workgroup (4 wave64)
constexpr int kMaxGroup = 16;  // matrices per grouped launch

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__constant__ float c_cent5[32] = HLWQ_CENTROIDS_5;
__constant__ float c_cent3[8] = HLWQ_CENTROIDS_3;
__constant__ uint32_t c_search5[2 * HLWQ_SEARCH_ENTRIES] = HLWQ_SEARCH_5;
__constant__ uint32_t c_search3[2 * HLWQ_SEARCH_ENTRIES] = HLWQ_SEARCH_3;
__constant__ uint32_t c_kvsearch3[2 * HLWQ_KV_SEARCH_ENTRIES] = HLWQ_KV_SEARCH_3;

const float h_cent5[32] = HLWQ_CENTROIDS_5;
const float h_thr5[31] = HLWQ_THRESHOLDS_5;
const float h_cent3[8] = HLWQ_CENTROIDS_3;
const float h_thr3[7] = HLWQ_THRESHOLDS_3;
const uint32_t h_search5[2 * HLWQ_SEARCH_ENTRIES] = HLWQ_SEARCH_5;
const uint32_t h_search3[2 * HLWQ_SEARCH_ENTRIES] = HLWQ_SEARCH_3;
const uint32_t h_kvsearch3[2 * HLWQ_KV_SEARCH_ENTRIES] = HLWQ_KV_SEARCH_3;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values; the kernels only
// produce finite values for finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// fp32 -> fp16 bits (round to nearest even, overflow to inf) and back (exact)
__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }
__device__ __forceinline__ float f16_value(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

// value of the lane whose id differs in bit 0 (quad permutation [1,0,3,2])
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Unpack 8 bf16 from a 16-byte word into x[8*c .. 8*c+7].
template <int N>
__device__ __forceinline__ void unpack8(u32x4 v, float (&x)[N], int c) {
  x[8 * c + 0] = bf16_lo(v.x);
  x[8 * c + 1] = bf16_hi(v.x);
  x[8 * c + 2] = bf16_lo(v.y);
  x[8 * c + 3] = bf16_hi(v.y);
  x[8 * c + 4] = bf16_lo(v.z);
  x[8 * c + 5] = bf16_hi(v.z);
  x[8 * c + 6] = bf16_lo(v.w);
  x[8 * c + 7] = bf16_hi(v.w);
}

// Load 128 bf16 starting at p, of which the first n (1..128) are real; the
// rest is zero (step [1]: the last block of a row is zero-padded).
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ p, int n, float (&x)[kBlock]) {
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(p) & 15u) == 0);
  if (vec_ok && n == kBlock) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 16; ++c) unpack8(__builtin_nontemporal_load(q + c), x, c);
  } else if (vec_ok && (n & 7) == 0) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (8 * c < n) v = __builtin_nontemporal_load(q + c);
      unpack8(v, x, c);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kBlock; ++j) x[j] = j < n ? __uint_as_float(static_cast<uint32_t>(p[j]) << 16) : 0.0f;
  }
}

// Store 128 values as bf16 to p, only the first n (1..128).
__device__ __forceinline__ void store_block(uint16_t* __restrict__ p, int n, const float (&w)[kBlock]) {
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(p) & 15u) == 0);
  if (vec_ok && (n & 7) == 0) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (8 * c < n) {
        u32x4 v;
        v.x = pack_bf16x2(w[8 * c + 0], w[8 * c + 1]);
        v.y = pack_bf16x2(w[8 * c + 2], w[8 * c + 3]);
        v.z = pack_bf16x2(w[8 * c + 4], w[8 * c + 5]);
        v.w = pack_bf16x2(w[8 * c + 6], w[8 * c + 7]);
        __builtin_nontemporal_store(v, q + c);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kBlock; ++j)
      if (j < n) p[j] = static_cast<uint16_t>(bf16_rne(w[j]));
  }
}

// Sum of squares by the adjacent-pair tree: level 0 forms x[2i]^2 + x[2i+1]^2,
// every further level adds neighbouring partial sums.
template <int L>
__device__ __forceinline__ float sumsq_tree(const float (&x)[L]) {
  float s[L / 2];
#pragma unroll
  for (int i = 0; i < L / 2; ++i) s[i] = x[2 * i] * x[2 * i] + x[2 * i + 1] * x[2 * i + 1];
#pragma unroll
  for (int w = L / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) s[i] = s[2 * i] + s[2 * i + 1];
  return s[0];
}

// Unnormalised Walsh-Hadamard butterflies, strides 1, 2, ..., L/2 (natural order).
template <int L>
__device__ __forceinline__ void fwht(float (&v)[L]) {
#pragma unroll
  for (int h = 1; h < L; h <<= 1)
#pragma unroll
    for (int i = 0; i < L; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

// Norm, fp16 norm and reciprocal of a block whose squared norm is s.
struct NormInfo {
  float r;
  uint16_t n16;
};
__device__ __forceinline__ NormInfo norm_info(float s) {
  const float n = sqrtf(s);
  NormInfo ni;
  ni.n16 = f16_bits(n);
  ni.r = (n >= FLT_MIN) ? 1.0f / n : 0.0f;
  return ni;
}

// y = z * r, code by bucket search, 8 codes of BITS bits per group packed
// little-endian into W words (code j occupies bits [BITS*j, BITS*j + BITS)).
template <int BITS, int L>
__device__ __forceinline__ void encode(const float (&z)[L], float r, const uint2* __restrict__ tab, float offset,
                                       uint32_t (&w)[L * BITS / 32]) {
#pragma unroll
  for (int i = 0; i < L * BITS / 32; ++i) w[i] = 0u;
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const float y = z[j] * r;
    const uint32_t k = static_cast<uint32_t>(__builtin_fmaf(y, 8.0f, offset));
    const uint2 e = tab[k];
    const uint32_t code = e.y + ((y > __uint_as_float(e.x)) ? 1u : 0u);
    const int p = j * BITS;
    w[p >> 5] |= code << (p & 31);
    if ((p & 31) + BITS > 32) w[(p >> 5) + 1] |= code >> (32 - (p & 31));
  }
}

// Unpack L codes of BITS bits and look up their centroids.
template <int BITS, int L>
__device__ __forceinline__ void decode(const uint32_t (&w)[L * BITS / 32], const float* __restrict__ cent,
                                       float (&v)[L]) {
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int p = j * BITS;
    uint32_t code = w[p >> 5] >> (p & 31);
    if ((p & 31) + BITS > 32) code |= w[(p >> 5) + 1] << (32 - (p & 31));
    v[j] = cent[code & ((1u << BITS) - 1u)];
  }
}

// ---------------------------------------------------------------------------
// weight kernels (grouped: up to kMaxGroup matrices per launch)
// ---------------------------------------------------------------------------

struct WeightGroup {
  int32_t n;                        // matrices in this launch
  int32_t wg_start[kMaxGroup + 1];  // first workgroup of every matrix (prefix sum)
  uint32_t nblocks[kMaxGroup];      // rows * nb
  uint32_t nb[kMaxGroup];           // blocks per row
  int64_t in[kMaxGroup];            // columns
  uint16_t* w[kMaxGroup];
  uint8_t* packed[kMaxGroup];
  uint16_t* norms[kMaxGroup];
};

// matrix owning this workgroup (uniform across the workgroup)
__device__ __forceinline__ int group_of(const WeightGroup& g) {
  int d = 0;
  for (int i = 1; i < g.n; ++i) d = (static_cast<int>(blockIdx.x) >= g.wg_start[i]) ? i : d;
  return d;
}

template <int BITS>
__global__ void __launch_bounds__(kThreads) hlwq_quantize_kernel(const WeightGroup g) {
  __shared__ uint2 tab[HLWQ_SEARCH_ENTRIES];
  const uint32_t* src_tab = (BITS == 5) ? c_search5 : c_search3;
  for (int i = threadIdx.x; i < HLWQ_SEARCH_ENTRIES; i += kThreads)
    tab[i] = make_uint2(src_tab[2 * i], src_tab[2 * i + 1]);
  __syncthreads();

  const int d = group_of(g);
  const uint32_t lb = (blockIdx.x - g.wg_start[d]) * kThreads + threadIdx.x;
  if (lb >= g.nblocks[d]) return;
  const uint32_t nb = g.nb[d];
  const uint32_t row = lb / nb;
  const uint32_t blk = lb - row * nb;
  const int64_t in = g.in[d];
  const int64_t col = static_cast<int64_t>(blk) * kBlock;
  const int n = static_cast<int>((in - col) < kBlock ? (in - col) : kBlock);

  float x[kBlock];
  load_block(g.w[d] + static_cast<int64_t>(row) * in + col, n, x);
  const NormInfo ni = norm_info(sumsq_tree(x));
  fwht(x);
  uint32_t words[4 * BITS];
  encode<BITS, kBlock>(x, ni.r, tab, HLWQ_SEARCH_OFFSET, words);

  u32x4* dst = reinterpret_cast<u32x4*>(g.packed[d] + static_cast<size_t>(lb) * (16 * BITS));
#pragma unroll
  for (int q = 0; q < BITS; ++q) {
    const u32x4 v = {words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]};
    __builtin_nontemporal_store(v, dst + q);
  }
  g.norms[d][lb] = ni.n16;
}

template <int BITS>
__global__ void __launch_bounds__(kThreads) hlwq_dequantize_kernel(const WeightGroup g) {
  __shared__ float cent[1 << BITS];
  const float* src_cent = (BITS == 5) ? c_cent5 : c_cent3;
  if (threadIdx.x < (1 << BITS)) cent[threadIdx.x] = src_cent[threadIdx.x];
  __syncthreads();

  const int d = group_of(g);
  const uint32_t lb = (blockIdx.x - g.wg_start[d]) * kThreads + threadIdx.x;
  if (lb >= g.nblocks[d]) return;
  const uint32_t nb = g.nb[d];
  const uint32_t row = lb / nb;
  const uint32_t blk = lb - row * nb;
  const int64_t in = g.in[d];
  const int64_t col = static_cast<int64_t>(blk) * kBlock;
  const int n = static_cast<int>((in - col) < kBlock ? (in - col) : kBlock);

  const u32x4* src = reinterpret_cast<const u32x4*>(g.packed[d] + static_cast<size_t>(lb) * (16 * BITS));
  uint32_t words[4 * BITS];
#pragma unroll
  for (int q = 0; q < BITS; ++q) {
    const u32x4 v = __builtin_nontemporal_load(src + q);
    words[4 * q] = v.x;
    words[4 * q + 1] = v.y;
    words[4 * q + 2] = v.z;
    words[4 * q + 3] = v.w;
  }
  const float scale = f16_value(g.norms[d][lb]) * 0x1p-7f;

  float v[kBlock];
  decode<BITS, kBlock>(words, cent, v);
  fwht(v);
#pragma unroll
  for (int j = 0; j < kBlock; ++j) v[j] = v[j] * scale;
  store_block(g.w[d] + static_cast<int64_t>(row) * in + col, n, v);
}

// ---------------------------------------------------------------------------
// KV-cache kernels: a 256-wide head vector over two adjacent lanes
// ---------------------------------------------------------------------------

struct KvArgs {
  uint16_t* kv;       // [bh][tokens][256]
  uint8_t* packed;    // [bh][tq][96]
  uint16_t* norms;    // [bh][tq]
  int64_t tokens;
  uint32_t tq;        // quantised tokens per head
  uint32_t nvec;      // bh * tq
};

__global__ void __launch_bounds__(kThreads) hlwq_kv_quantize_kernel(const KvArgs a) {
  __shared__ uint2 tab[HLWQ_KV_SEARCH_ENTRIES];
  for (int i = threadIdx.x; i < HLWQ_KV_SEARCH_ENTRIES; i += kThreads)
    tab[i] = make_uint2(c_kvsearch3[2 * i], c_kvsearch3[2 * i + 1]);
  __syncthreads();

  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t vec = gid >> 1;
  const uint32_t half = gid & 1u;  // 0: entries 0..127, 1: entries 128..255
  if (vec >= a.nvec) return;       // both lanes of a vector leave together
  const uint32_t bh = vec / a.tq;
  const uint32_t t = vec - bh * a.tq;

  float x[kBlock];
  load_block(a.kv + (static_cast<int64_t>(bh) * a.tokens + t) * kKvDim + half * kBlock, kBlock, x);
  // last tree level joins the two halves: lower half first (addition commutes)
  const float s_half = sumsq_tree(x);
  const NormInfo ni = norm_info(s_half + lane_xor1(s_half));
  fwht(x);
  // stride-128 stage across the lane pair: (a, b) -> (a + b, a - b)
  const float sgn = half ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) x[j] = __builtin_fmaf(x[j], sgn, lane_xor1(x[j]));

  uint32_t words[12];
  encode<3, kBlock>(x, ni.r, tab, HLWQ_KV_SEARCH_OFFSET, words);
  u32x4* dst = reinterpret_cast<u32x4*>(a.packed + static_cast<size_t>(vec) * 96 + half * 48);
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const u32x4 v = {words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]};
    __builtin_nontemporal_store(v, dst + q);
  }
  if (half == 0) a.norms[vec] = ni.n16;
}

__global__ void __launch_bounds__(kThreads) hlwq_kv_dequantize_kernel(const KvArgs a) {
  __shared__ float cent[8];
  if (threadIdx.x < 8) cent[threadIdx.x] = c_cent3[threadIdx.x];
  __syncthreads();

  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t vec = gid >> 1;
  const uint32_t half = gid & 1u;
  if (vec >= a.nvec) return;
  const uint32_t bh = vec / a.tq;
  const uint32_t t = vec - bh * a.tq;

  const u32x4* src = reinterpret_cast<const u32x4*>(a.packed + static_cast<size_t>(vec) * 96 + half * 48);
  uint32_t words[12];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const u32x4 v = __builtin_nontemporal_load(src + q);
    words[4 * q] = v.x;
    words[4 * q + 1] = v.y;
    words[4 * q + 2] = v.z;
    words[4 * q + 3] = v.w;
  }
  const float scale = f16_value(a.norms[vec]) * 0x1p-8f;

  float v[kBlock];
  decode<3, kBlock>(words, cent, v);
  fwht(v);
  const float sgn = half ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) v[j] = __builtin_fmaf(v[j], sgn, lane_xor1(v[j]));
#pragma unroll
  for (int j = 0; j < kBlock; ++j) v[j] = v[j] * scale;
  store_block(a.kv + (static_cast<int64_t>(bh) * a.tokens + t) * kKvDim + half * kBlock, kBlock, v);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? HLWQ_OK : HLWQ_ERR_DEVICE;
}

// Validate one weight descriptor; *blocks = rows * nb (0 means nothing to do).
int check_weight_desc(const hlwq_mat_desc& m, int64_t* blocks) {
  *blocks = 0;
  if (m.rows < 0 || m.in < 0) return HLWQ_ERR_SHAPE;
  if (m.rows == 0 || m.in == 0) return HLWQ_OK;
  if (!m.w || !m.packed || !m.norms) return HLWQ_ERR_NULL;
  int64_t elems, bytes;
  if (!mul_ok(m.rows, m.in, &elems) || !mul_ok(elems, 2, &bytes)) return HLWQ_ERR_SHAPE;
  const int64_t nb = ceil_div(m.in, kBlock);
  int64_t nblk;
  if (!mul_ok(m.rows, nb, &nblk) || !mul_ok(nblk, 80, &bytes)) return HLWQ_ERR_SHAPE;
  if (nblk > 0x7fffffff) return HLWQ_ERR_LIMIT;
  if ((reinterpret_cast<uintptr_t>(m.packed) & 15u) || (reinterpret_cast<uintptr_t>(m.norms) & 1u) ||
      (reinterpret_cast<uintptr_t>(m.w) & 1u))
    return HLWQ_ERR_ALIGN;
  *blocks = nblk;
  return HLWQ_OK;
}

template <bool QUANT>
int run_weight_group(const hlwq_mat_desc* mats, int n, int bits, hipStream_t stream) {
  if (n < 0) return HLWQ_ERR_SHAPE;
  if (n > 0 && !mats) return HLWQ_ERR_NULL;
  if (bits != 5 && bits != 3) return HLWQ_ERR_BITS;
  // validate everything before enqueuing anything
  for (int i = 0; i < n; ++i) {
    int64_t b;
    const int st = check_weight_desc(mats[i], &b);
    if (st != HLWQ_OK) return st;
  }
  int i = 0;
  while (i < n) {
    WeightGroup g;
    std::memset(&g, 0, sizeof(g));
    int64_t wg = 0;
    for (; i < n && g.n < kMaxGroup; ++i) {
      int64_t nblk;
      check_weight_desc(mats[i], &nblk);
      if (nblk == 0) continue;
      const int k = g.n++;
      g.wg_start[k] = static_cast<int32_t>(wg);
      g.nblocks[k] = static_cast<uint32_t>(nblk);
      g.nb[k] = static_cast<uint32_t>(ceil_div(mats[i].in, kBlock));
      g.in[k] = mats[i].in;
      g.w[k] = static_cast<uint16_t*>(mats[i].w);
      g.packed[k] = static_cast<uint8_t*>(mats[i].packed);
      g.norms[k] = static_cast<uint16_t*>(mats[i].norms);
      wg += ceil_div(nblk, kThreads);
      if (wg > 0x7fffffff) return HLWQ_ERR_LIMIT;
    }
    if (g.n == 0) continue;
    g.wg_start[g.n] = static_cast<int32_t>(wg);
    const dim3 grid(static_cast<uint32_t>(wg)), block(kThreads);
    if (QUANT) {
      if (bits == 5) hipLaunchKernelGGL(hlwq_quantize_kernel<5>, grid, block, 0, stream, g);
      else hipLaunchKernelGGL(hlwq_quantize_kernel<3>, grid, block, 0, stream, g);
    } else {
      if (bits == 5) hipLaunchKernelGGL(hlwq_dequantize_kernel<5>, grid, block, 0, stream, g);
      else hipLaunchKernelGGL(hlwq_dequantize_kernel<3>, grid, block, 0, stream, g);
    }
    const int st = launch_status();
    if (st != HLWQ_OK) return st;
  }
  return HLWQ_OK;
}

int make_single(const void* w, const void* packed, const void* norms, int64_t n_mats, int64_t out, int64_t in,
                int block, int bits, hlwq_mat_desc* m) {
  if (block != kBlock) return HLWQ_ERR_BLOCK;
  if (bits != 5 && bits != 3) return HLWQ_ERR_BITS;
  if (n_mats < 0 || out < 0 || in < 0) return HLWQ_ERR_SHAPE;
  int64_t rows;
  if (!mul_ok(n_mats, out, &rows)) return HLWQ_ERR_SHAPE;
  m->w = const_cast<void*>(w);
  m->packed = const_cast<void*>(packed);
  m->norms = const_cast<void*>(norms);
  m->rows = rows;
  m->in = in;
  return HLWQ_OK;
}

int run_kv(bool quant, const void* kv, void* packed, void* norms, int64_t batch, int64_t heads, int64_t tokens,
           int head_dim, int bits, int64_t n_residual, hipStream_t stream) {
  if (head_dim != kKvDim) return HLWQ_ERR_BLOCK;
  if (bits != 3) return HLWQ_ERR_BITS;
  if (batch < 0 || heads < 0 || tokens < 0 || n_residual < 0) return HLWQ_ERR_SHAPE;
  const int64_t tq = tokens > n_residual ? tokens - n_residual : 0;
  int64_t bh, nvec, elems, bytes;
  if (!mul_ok(batch, heads, &bh) || !mul_ok(bh, tq, &nvec) || !mul_ok(bh, tokens, &elems) ||
      !mul_ok(elems, 2 * kKvDim, &bytes))
    return HLWQ_ERR_SHAPE;
  if (nvec == 0) return HLWQ_OK;
  if (!kv || !packed || !norms) return HLWQ_ERR_NULL;
  if (nvec > 0x3fffffff || tq > 0x7fffffff) return HLWQ_ERR_LIMIT;
  if ((reinterpret_cast<uintptr_t>(packed) & 15u) || (reinterpret_cast<uintptr_t>(norms) & 1u) ||
      (reinterpret_cast<uintptr_t>(kv) & 1u))
    return HLWQ_ERR_ALIGN;
  KvArgs a;
  a.kv = const_cast<uint16_t*>(static_cast<const uint16_t*>(kv));
  a.packed = static_cast<uint8_t*>(packed);
  a.norms = static_cast<uint16_t*>(norms);
  a.tokens = tokens;
  a.tq = static_cast<uint32_t>(tq);
  a.nvec = static_cast<uint32_t>(nvec);
  const dim3 grid(static_cast<uint32_t>(ceil_div(2 * nvec, kThreads))), block(kThreads);
  if (quant) hipLaunchKernelGGL(hlwq_kv_quantize_kernel, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(hlwq_kv_dequantize_kernel, grid, block, 0, stream, a);
  return launch_status();
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int hlwq_quantize(const void* w_bf16, int64_t n_mats, int64_t out, int64_t in, int block, int bits,
                  void* packed_u8, void* norms_f16, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16, packed_u8, norms_f16, n_mats, out, in, block, bits, &m);
  if (st != HLWQ_OK) return st;
  return run_weight_group<true>(&m, 1, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_dequantize(const void* packed_u8, const void* norms_f16, int64_t n_mats, int64_t out, int64_t in,
                    int block, int bits, void* w_bf16_out, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16_out, packed_u8, norms_f16, n_mats, out, in, block, bits, &m);
  if (st != HLWQ_OK) return st;
  return run_weight_group<false>(&m, 1, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_quantize_grouped(const hlwq_mat_desc* mats, int n, int bits, void* hip_stream) {
  return run_weight_group<true>(mats, n, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_dequantize_grouped(const hlwq_mat_desc* mats, int n, int bits, void* hip_stream) {
  return run_weight_group<false>(mats, n, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_kv_quantize(const void* kv_bf16, int64_t batch, int64_t heads, int64_t tokens, int head_dim, int bits,
                     int64_t n_residual, void* packed_u8, void* norms_f16, void* hip_stream) {
  return run_kv(true, kv_bf16, packed_u8, norms_f16, batch, heads, tokens, head_dim, bits, n_residual,
                static_cast<hipStream_t>(hip_stream));
}

int hlwq_kv_dequantize(const void* packed_u8, const void* norms_f16, int64_t batch, int64_t heads,
                       int64_t tokens, int head_dim, int bits, int64_t n_residual, void* kv_bf16_out,
                       void* hip_stream) {
  return run_kv(false, kv_bf16_out, const_cast<void*>(packed_u8), const_cast<void*>(norms_f16), batch, heads,
                tokens, head_dim, bits, n_residual, static_cast<hipStream_t>(hip_stream));
}

size_t hlwq_packed_bytes(int64_t rows, int64_t in, int block, int bits) {
  if (rows < 0 || in < 0 || block <= 0 || (block % 8) != 0 || bits <= 0 || bits > 8) return 0;
  int64_t nblk, bytes;
  if (!mul_ok(rows, ceil_div(in, block), &nblk) || !mul_ok(nblk, static_cast<int64_t>(block) * bits / 8, &bytes))
    return 0;
  return static_cast<size_t>(bytes);
}

size_t hlwq_norm_count(int64_t rows, int64_t in, int block) {
  if (rows < 0 || in < 0 || block <= 0) return 0;
  int64_t nblk;
  if (!mul_ok(rows, ceil_div(in, block), &nblk)) return 0;
  return static_cast<size_t>(nblk);
}

int hlwq_centroids(int bits, float* centroids, float* thresholds) {
  if (bits != 5 && bits != 3) return HLWQ_ERR_BITS;
  const int K = 1 << bits;
  const float* c = bits == 5 ? h_cent5 : h_cent3;
  const float* t = bits == 5 ? h_thr5 : h_thr3;
  if (centroids) std::memcpy(centroids, c, sizeof(float) * K);
  if (thresholds) std::memcpy(thresholds, t, sizeof(float) * (K - 1));
  return HLWQ_OK;
}

int hlwq_search_table(int kind, uint32_t* words, int capacity, float* offset) {
  const uint32_t* src;
  int entries;
  float off;
  switch (kind) {
    case 0: src = h_search5; entries = HLWQ_SEARCH_ENTRIES; off = HLWQ_SEARCH_OFFSET; break;
    case 1: src = h_search3; entries = HLWQ_SEARCH_ENTRIES; off = HLWQ_SEARCH_OFFSET; break;
    case 2: src = h_kvsearch3; entries = HLWQ_KV_SEARCH_ENTRIES; off = HLWQ_KV_SEARCH_OFFSET; break;
    default: return HLWQ_ERR_BITS;
  }
  if (words) {
    const int m = capacity < entries ? capacity : entries;
    if (m > 0) std::memcpy(words, src, sizeof(uint32_t) * 2 * m);
  }
  if (offset) *offset = off;
  return entries;
}

const char* hlwq_status_string(int status) {
  switch (status) {
    case HLWQ_OK: return "ok";
    case HLWQ_ERR_NULL: return "a required pointer is NULL";
    case HLWQ_ERR_SHAPE: return "negative size or size overflow";
    case HLWQ_ERR_BITS: return "unsupported bits";
    case HLWQ_ERR_BLOCK: return "unsupported block size / head_dim";
    case HLWQ_ERR_DEVICE: return "HIP launch failed";
    case HLWQ_ERR_ALIGN: return "buffer misaligned";
    case HLWQ_ERR_LIMIT: return "too many blocks for one call";
    default: return "unknown status";
  }
}

}  // extern "C"
