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
// 128 weights.  A KV head vector (256 values) is split over four adjacent
// lanes of 64 values: the last two norm levels and the last two butterfly
// stages (strides 64 and 128) cross lanes through DPP quad permutations (the
// decode-step append kernel uses four values per lane instead, and the ring
// append kernel lane pairs).
//
// Code search.  A rotated value y becomes, by one fused multiply-add with a
// denormal addend, a denormal whose bit pattern is the index of its 1/8-wide
// bucket; one LDS byte read there gives the offset of the entry
// {threshold, base} in a second small table, and the code is
// base + (y > threshold).  The tables are built and proven exact against the
// plain count at build time (gen_tables.cpp), so the kernels reproduce
// "number of fp32 thresholds below y" bit for bit with one compare.

// Rounding.  The file is compiled with -ffp-contract=off: every + and * below
// is one IEEE round-to-nearest operation in the order written, sqrtf and the
// division are correctly rounded, and the only fused multiply-adds are the
// explicit __builtin_fmaf calls of the first norm-tree level and the
// cross-lane KV butterflies, a + (+-1) b (the product is exact, so the one
// rounding is that of a +- b), so no rounding differs from the operation order
// documented in include/hlwq.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cstdint>
#include <cstring>
#include <vector>

#include "hlwq.h"
#include "hlwq_tables.inc"

namespace {

constexpr int kBlock = 128;    // weights per HLWQ block
constexpr int kKvDim = 256;    // KV head vector length
constexpr int kThreads = 256;  // work-items per workgroup (4 wave64)
constexpr int kMaxGroup = 16;  // matrices per grouped launch
constexpr int kKvPoolWaves = 16;   // waves of the KV quantizer's work-pool workgroup (one per CU)
constexpr int kKvPoolThreads = 64 * kKvPoolWaves;
constexpr int kPoolWaves = 8;   // waves of a work-pool workgroup (one workgroup per CU)
constexpr int kPoolThreads = 64 * kPoolWaves;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__constant__ float c_cent5[32] = HLWQ_CENTROIDS_5;
__constant__ float c_cent3[8] = HLWQ_CENTROIDS_3;
__constant__ uint32_t c_bucket5[HLWQ_BUCKETS / 4] = HLWQ_BUCKET_5;
__constant__ uint32_t c_bucket3[HLWQ_BUCKETS / 4] = HLWQ_BUCKET_3;
__constant__ uint32_t c_kvbucket3[HLWQ_KV_BUCKETS / 4] = HLWQ_KV_BUCKET_3;
__constant__ uint32_t c_entry5[2 * 32] = HLWQ_ENTRY_5;
__constant__ uint32_t c_entry3[2 * 8] = HLWQ_ENTRY_3;
__constant__ uint32_t c_bucket3m[HLWQ_BUCKETS / 4] = HLWQ_BUCKET_3M;  // TQ3's mirrored search
__constant__ uint32_t c_entry3m[2 * 8] = HLWQ_ENTRY_3M;
__constant__ float c_cent2[4] = HLWQ_CENTROIDS_2;
__constant__ uint32_t c_entry2[2 * 4] = HLWQ_ENTRY_2;
__constant__ uint32_t c_kvbucket2[HLWQ_KV_BUCKETS / 4] = HLWQ_KV_BUCKET_2;

const float h_cent5[32] = HLWQ_CENTROIDS_5;
const float h_thr5[31] = HLWQ_THRESHOLDS_5;
const float h_cent3[8] = HLWQ_CENTROIDS_3;
const float h_thr3[7] = HLWQ_THRESHOLDS_3;
const uint32_t h_bucket5[HLWQ_BUCKETS / 4] = HLWQ_BUCKET_5;
const uint32_t h_bucket3[HLWQ_BUCKETS / 4] = HLWQ_BUCKET_3;
const uint32_t h_kvbucket3[HLWQ_KV_BUCKETS / 4] = HLWQ_KV_BUCKET_3;
const uint32_t h_entry5[2 * 32] = HLWQ_ENTRY_5;
const uint32_t h_entry3[2 * 8] = HLWQ_ENTRY_3;
const float h_cent2[4] = HLWQ_CENTROIDS_2;
const float h_thr2[3] = HLWQ_THRESHOLDS_2;
const uint32_t h_entry2[2 * 4] = HLWQ_ENTRY_2;
const uint32_t h_kvbucket2[HLWQ_KV_BUCKETS / 4] = HLWQ_KV_BUCKET_2;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even).
// Dequantised values are never fp32 denormals (|value| >= 2^-59 when nonzero:
// centroid sums are multiples of 2^-27 and the scale is at least 2^-32), so
// the conversion agrees with bf16_rne bit for bit.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> fp16 bits (round to nearest even, overflow to inf) and back (exact)
__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }
__device__ __forceinline__ float f16_value(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

// value of the lane whose id differs in bit 0 (quad permutation [1,0,3,2])
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Butterfly across a lane pair: the even lane holds a, the odd lane b; both
// call this with sgn = +1 (even) or -1 (odd) and get a + b, resp. a - b.
// partner + sgn * self is that sum with one rounding (sgn * self is exact),
// and the partner operand folds into a DPP-modified add.
__device__ __forceinline__ float cross_pair(float self, float sgn) { return lane_xor1(self) + self * sgn; }

// +1 on even lanes, -1 on odd lanes; laundered through an empty asm so the
// compiler keeps "self * sgn" as a multiply (rewriting it into a select of
// two butterflies would stop the DPP operand from folding into the add)
__device__ __forceinline__ float pair_sign(uint32_t half) {
  float s = half ? -1.0f : 1.0f;
  asm volatile("" : "+v"(s));
  return s;
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

// Store the first n (1..128) values of a block, packed as bf16 pairs, to p.
__device__ __forceinline__ void store_block(uint16_t* __restrict__ p, int n, const uint32_t (&pk)[kBlock / 2]) {
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(p) & 15u) == 0);
  if (vec_ok && (n & 7) == 0) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (8 * c < n) {
        const u32x4 v = {pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
        __builtin_nontemporal_store(v, q + c);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kBlock; ++j)
      if (j < n) p[j] = static_cast<uint16_t>(pk[j / 2] >> (16 * (j & 1)));
  }
}

// Sum of squares by the adjacent-pair tree: level 0 forms each pair
// x[2i]^2 + x[2i+1]^2 with one fused multiply-add (x[2i]^2 exact inside it,
// x[2i+1]^2 rounded), every further level adds neighbouring partial sums.
template <int L>
__device__ __forceinline__ float sumsq_tree(const float (&x)[L]) {
  float s[L / 2];
#pragma unroll
  for (int i = 0; i < L / 2; ++i) s[i] = __builtin_fmaf(x[2 * i], x[2 * i], x[2 * i + 1] * x[2 * i + 1]);
#pragma unroll
  for (int w = L / 4; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) s[i] = s[2 * i] + s[2 * i + 1];
  return s[0];
}

// Unnormalised Walsh-Hadamard butterflies, strides H0, 2 H0, ..., L/2 (natural
// order; H0 = 1 is the whole transform).
template <int L, int H0 = 1>
__device__ __forceinline__ void fwht(float (&v)[L]) {
#pragma unroll
  for (int h = H0; h < L; h <<= 1)
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
  float n, r;
  uint16_t n16;
};
__device__ __forceinline__ NormInfo norm_info(float s) {
  const float n = sqrtf(s);
  NormInfo ni;
  ni.n = n;
  ni.n16 = f16_bits(n);
  ni.r = (n >= FLT_MIN) ? 1.0f / n : 0.0f;
  return ni;
}

// A 128-bit string of TQ3 signs, bit i of word i / 32 for entry i (set: the
// entry is -1).  Uniform across the grid, so it and every mask below live in
// scalar registers.
struct SignBits {
  uint32_t w[4];
};
// the sign bit (0 or 1 << 31) that negates entry i
__device__ __forceinline__ uint32_t sign_bit(const SignBits& s, int i) {
  return (s.w[i >> 5] << (31 - (i & 31))) & 0x80000000u;
}
// The same bits, opaque to the compiler from here on: called once per batch,
// it keeps every mask derived from them inside the batch loop (a few scalar
// operations each) instead of hoisted out of it, where 256 live masks would
// overflow the scalar register file.
__device__ __forceinline__ SignBits per_batch(SignBits s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+s"(s.w[i]));
  return s;
}
// the xor mask that negates bf16 entries 2m (low half) and 2m + 1 (high half)
// of a packed pair
__device__ __forceinline__ uint32_t pair_sign_mask(const SignBits& s, int m) {
  return (sign_bit(s, 2 * m) >> 16) | sign_bit(s, 2 * m + 1);
}

// Code of one rotated value y = z * r.  u = fma(y, 2^-146, bias) is a
// denormal for every reachable y (bias = C * 2^-149), so bits(u) = RN(8 y) + C
// is the index of y's 1/8-wide bucket; the byte there (bucket table at LDS
// byte offset `bucket`) is the offset of the entry {threshold, base} in the
// entry table at LDS offset 0, and the code is base + (y > threshold).  The
// table generator proves this equals the number of fp32 thresholds strictly
// below y for every reachable y.
__device__ __forceinline__ uint32_t code_of(float z, float r, const uint8_t* __restrict__ lds, uint32_t bucket,
                                            float bias) {
  const float y = z * r;
  const uint32_t k = __float_as_uint(__builtin_fmaf(y, HLWQ_SEARCH_SCALE, bias));
  const uint32_t e = lds[bucket + k];
  const uint2 v = *reinterpret_cast<const uint2*>(lds + e);
  return v.y + ((y > __uint_as_float(v.x)) ? 1u : 0u);
}

// Encode L values into L * BITS / 32 words: 8 codes of BITS bits per group,
// little-endian, so code j occupies bits [BITS*j, BITS*j + BITS) of the block's
// bit string.  Words are built top-down by Horner steps acc = (acc << BITS) +
// code; a code that straddles two words is computed once, finishes the upper
// word's bottom bits and starts the lower word.
// With MIRROR (TQ3's D2, 3-bit codes), value j whose bit in the 128-bit
// string s2 is set is searched in the mirrored tables, which follow the plain
// bucket table (bias + HLWQ_BUCKETS), and gives 7 - code(-y); the caller
// turns it into code(-y) with an xor of the packed words.
template <int BITS, int L, bool MIRROR = false>
__device__ __forceinline__ void encode(const float (&z)[L], float r, const uint8_t* __restrict__ lds, uint32_t bucket,
                                       float bias, uint32_t (&w)[L * BITS / 32], const SignBits& s2 = SignBits{}) {
  constexpr int W = L * BITS / 32;
  static_assert(HLWQ_BUCKETS == 2048, "sign_bit >> 20 selects the mirrored bucket table");
  auto code = [&](int j) {
    const float b = MIRROR ? __uint_as_float(__float_as_uint(bias) + (sign_bit(s2, j) >> 20)) : bias;
    return code_of(z[j], r, lds, bucket, b);
  };
  uint32_t carry = 0;  // straddling code shared with the word below
#pragma unroll
  for (int wi = W - 1; wi >= 0; --wi) {
    const int jhi = (32 * wi + 31) / BITS;              // last code touching this word
    const int jlo = (32 * wi + BITS - 1) / BITS;        // first code starting in this word
    const int off = BITS * jlo - 32 * wi;               // its bit position (0 .. BITS-1)
    const bool top_shared = (BITS * jhi + BITS > 32 * (wi + 1)) && (jhi < L);
    uint32_t acc = top_shared ? carry : code(jhi);
#pragma unroll
    for (int j = jhi - 1; j >= jlo; --j) acc = (acc << BITS) + code(j);
    if (off > 0) {
      const uint32_t c = code(jlo - 1);
      acc = (acc << off) + (c >> (BITS - off));
      carry = c;
    }
    w[wi] = acc;
  }
}

// Unpack L codes of BITS bits, look up their centroids and apply the first
// butterfly stage, two values at a time.  Stage 1 pairs exactly the two codes
// of a pair index (codes are LSB-first, so code 2m is the low half of pair m),
// so the pair table (LDS offset 0) holds, for every 2*BITS-bit index i with
// a = i mod 2^BITS and b = i >> BITS, the stage-1 outputs
// {c[a] + c[b], c[a] - c[b]}, computed with the same fp32 operations.  One
// 8-byte read serves two values; its byte offset 8 i comes out of the packed
// words with one shift or funnel shift and one mask.
template <int BITS, int SH, int W>
__device__ __forceinline__ uint32_t pair_offset(const uint32_t (&w)[W], int m) {
  constexpr uint32_t kMask = ((1u << (2 * BITS)) - 1u) << SH;
  const int p = 2 * BITS * m;  // bit position of pair m
  const int lo = p & 31, wi = p >> 5;
  uint32_t off;
  if (lo + 2 * BITS <= 32)
    off = (lo >= SH) ? (w[wi] >> (lo - SH)) : (w[wi] << (SH - lo));
  else
    off = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], lo - SH);
  return off & kMask;
}

template <int BITS, int L>
__device__ __forceinline__ void decode_stage1(const uint32_t (&w)[L * BITS / 32], const uint8_t* __restrict__ pairs,
                                              float (&v)[L]) {
#pragma unroll
  for (int m = 0; m < L / 2; ++m) {
    const float2 c = *reinterpret_cast<const float2*>(pairs + pair_offset<BITS, 3>(w, m));
    v[2 * m] = c.x;
    v[2 * m + 1] = c.y;
  }
}

// The same for codes stored one per byte (the low BITS bits of each byte):
// the pair index of codes 2m and 2m+1 is assembled from two byte fields.
template <int BITS, int L>
__device__ __forceinline__ void decode_bytes_stage1(const uint32_t (&w)[L / 4], const uint8_t* __restrict__ pairs,
                                                    float (&v)[L]) {
#pragma unroll
  for (int m = 0; m < L / 2; ++m) {
    const uint32_t word = w[m >> 1];
    const int sh = 16 * (m & 1);
    const uint32_t lo = __builtin_amdgcn_ubfe(word, sh, BITS);
    const uint32_t hi = __builtin_amdgcn_ubfe(word, sh + 8, BITS);
    const float2 c = *reinterpret_cast<const float2*>(pairs + 8u * (lo | (hi << BITS)));
    v[2 * m] = c.x;
    v[2 * m + 1] = c.y;
  }
}

// Squared norm of the 8-centroid codes a block selects, summed exactly and
// rounded once.  c is symmetric, so c[k]^2 depends only on the magnitude
// class m of code k = (b2 b1 b0): m = 2 (b1 XNOR b2) + (b0 XNOR b2), c[4 + m]
// for b2 = 1 and c[3 - m] = -c[4 + m] for b2 = 0.  Three popcounts over the
// 384-bit code string give A = #(b1 XNOR b2), B = #(b0 XNOR b2) and
// C = #(both); the class counts are then N3 = C, N2 = A - C, N1 = B - C,
// N0 = 128 - A - B + C.  Every RN(c^2) is a multiple of 2^-28 and the total is
// below 2^10, so the fp64 products and sum are exact and the conversion to
// fp32 is the one rounding.  Per word: two funnel shifts bring b1 and b2 of
// every code onto its b0 position; the masks pick the b0 positions of the
// word (period 3 words, as 32 = 2 mod 3).
__device__ __forceinline__ float recon_sumsq3(const uint32_t (&w)[12]) {
  constexpr uint32_t kB0[3] = {0x49249249u, 0x92492492u, 0x24924924u};
  constexpr float cent[8] = HLWQ_CENTROIDS_3;
  constexpr float c4 = cent[4], c5 = cent[5], c6 = cent[6], c7 = cent[7];
  uint32_t a = 0, b = 0, c = 0;
#pragma unroll
  for (int q = 0; q < 12; ++q) {
    const uint32_t next = q + 1 < 12 ? w[q + 1] : 0u;
    const uint32_t t1 = __builtin_amdgcn_alignbit(next, w[q], 1);  // b1 at b0
    const uint32_t t2 = __builtin_amdgcn_alignbit(next, w[q], 2);  // b2 at b0
    const uint32_t m0 = ~(w[q] ^ t2) & kB0[q % 3];
    const uint32_t m1 = ~(t1 ^ t2) & kB0[q % 3];
    b += __builtin_popcount(m0);
    a += __builtin_popcount(m1);
    c += __builtin_popcount(m0 & m1);
  }
  const double e0 = (double)(c4 * c4), e1 = (double)(c5 * c5), e2 = (double)(c6 * c6), e3 = (double)(c7 * c7);
  const double s = (double)(128u - a - b + c) * e0 + (double)(b - c) * e1 + (double)(a - c) * e2 + (double)c * e3;
  return (float)s;
}

// Fill the pair table of a K-centroid codebook (K * K entries of 8 bytes).
template <int BITS, int NT = kThreads>
__device__ __forceinline__ void fill_pairs(float* pairs, const float* __restrict__ cent) {
  constexpr int K = 1 << BITS;
  for (int i = threadIdx.x; i < K * K; i += NT) {
    const float a = cent[i & (K - 1)], b = cent[i >> BITS];
    pairs[2 * i] = a + b;
    pairs[2 * i + 1] = a - b;
  }
}

// ---------------------------------------------------------------------------
// LDS staging
//
// Every wave owns a 16 KB slice of LDS.  Inputs reach it through direct
// global->LDS loads (buffer_load_dwordx4 ... lds): in load instruction i, lane l
// fills slot 64 i + l, so each instruction is one contiguous 1 KB of LDS and,
// with the slot->chunk map below, one contiguous 1 KB of global memory too.
// The map XORs the low 4 bits of a 16-byte chunk index with its 256-byte-row
// index: when every lane then reads chunk c of its own 256-byte block, 16
// consecutive lanes touch 16 different bank groups.  Outputs go the other
// way: lanes write their results into the slice, the wave reads it back in
// chunk order and issues 1 KB-contiguous global stores.  The slice is private
// to the wave and LDS operations of one wave complete in order, so no
// workgroup barrier is needed.
// ---------------------------------------------------------------------------

constexpr int kWaves = kThreads / 64;  // waves per workgroup
constexpr int kStage = 16384;          // LDS bytes per wave

__device__ __forceinline__ uint32_t swz(uint32_t q) { return q ^ ((q >> 4) & 15u); }

// streaming (nontemporal) accesses: cache-policy bit 1
constexpr int kNt = 2;

// wait for this wave's outstanding vector-memory operations, including the
// direct-to-LDS loads; the memory clobber keeps LDS reads below it
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Lanes of a wave hand data to each other through LDS (one lane writes a
// slot, another reads it).  A wave's LDS operations execute in order, but the
// compiler reasons per lane and may, for instance, keep a value a lane loaded
// before another lane's write; this compiler barrier marks each hand-over, so
// no access moves across it and nothing loaded before it is reused after it.
__device__ __forceinline__ void lds_handover() { asm volatile("" ::: "memory"); }

// Per-lane byte offsets of the swizzled slot pattern: in load / store
// instruction i, lane l handles chunk 64 i + (l ^ (4 (i & 3) + (l >> 4))),
// i.e. byte offset 1024 i + o[i & 3] (swz(64 i + l) written out: the row index
// (64 i + l) >> 4 is 4 i + (l >> 4), whose low 4 bits are 4 (i & 3) + (l >> 4)).
struct SwzLane {
  uint32_t o[4];
};

// Make per-lane address bases opaque at the top of a loop iteration, so the
// compiler derives the 16 chunk addresses of a batch inside the loop (one add
// or xor each, or an instruction offset) instead of holding all of them in
// VGPRs across the whole loop.
__device__ __forceinline__ void refresh(SwzLane& sl, uint32_t& a) {
  asm volatile("" : "+v"(sl.o[0]), "+v"(sl.o[1]), "+v"(sl.o[2]), "+v"(sl.o[3]), "+v"(a));
}
__device__ __forceinline__ SwzLane swz_lane(int lane) {
  SwzLane sl;
#pragma unroll
  for (int k = 0; k < 4; ++k) sl.o[k] = 16u * (static_cast<uint32_t>(lane) ^ (4u * k + (static_cast<uint32_t>(lane) >> 4)));
  return sl;
}

// Stage `bytes` (<= 1024 * NI, a multiple of 16) of global memory starting
// at the 16-byte aligned address src: chunk q (16 bytes) lands in slot swz(q)
// if SWZ, else q.  The loads go through a buffer resource over exactly those
// bytes, so chunks past the end read as zeros without a per-lane clamp (the
// whole offset is in the VGPR operand, which is what the range check covers).
// AUX is the cache policy of the loads.
template <int NI, bool SWZ, int AUX>
__device__ __forceinline__ void stage_in(const uint8_t* src, uint32_t bytes, uint8_t* stage, int lane,
                                         const SwzLane& sl) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), static_cast<short>(0),
                                                   static_cast<int>(bytes), 0x00020000);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(stage + 1024 * i), 16,
                                             1024u * i + (SWZ ? sl.o[i & 3] : 16u * lane), 0, 0, AUX);
}

// Write back `bytes` (a multiple of 16) of staged output (chunk q in slot
// swz(q) if SWZ) to dst with 1 KB-contiguous stores; through a buffer
// resource over exactly those bytes, so the stores of chunks past the end are
// dropped without a branch.
template <int NI, bool SWZ>
__device__ __forceinline__ void stage_out(uint8_t* dst, uint32_t bytes, const uint8_t* stage, int lane,
                                          const SwzLane& sl) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(dst, static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
  lds_handover();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + 1024u * i + (SWZ ? sl.o[i & 3] : 16u * lane));
    __builtin_amdgcn_raw_buffer_store_b128(v, r, 1024u * i + 16u * lane, 0, kNt);
  }
  lds_handover();
}

__device__ __forceinline__ int64_t first_lane64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Fast paths for a full batch whose blocks are all whole and contiguous
// (64 x 256 bytes): lane l's block sits at bytes [256 l, 256 l + 256) of the
// batch, so its chunk c lives in slot 16 l + (c ^ (l & 15)) and its LDS
// address is A_l ^ 16c with A_l = stage + 256 l + 16 (l & 15) (the wave's
// stage is 256-byte aligned).  In load / store instruction i, lane l handles
// chunk 64 i + (l ^ (4 (i & 3) + (l >> 4))), i.e. byte offset 1024 i + o[i & 3].
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)p));
}
__device__ __forceinline__ u32x4 lds_read16(uint32_t a) { return *(const lds_u32x4*)static_cast<uintptr_t>(a); }
__device__ __forceinline__ void lds_write16(uint32_t a, u32x4 v) { *(lds_u32x4*)static_cast<uintptr_t>(a) = v; }

// Read one 128-value block whose bytes start at byte offset `off` (a multiple
// of 16) of a swizzled stage; only the first n values are real.  Chunks past
// n are read from `zero` (the LDS address of 16 zero bytes) instead of being
// skipped, so every lane runs the same instructions and no chunk needs a
// branch.  All 16 reads are issued before the first is unpacked (the
// scheduling barrier keeps them together): left to itself the compiler
// interleaves each read's address arithmetic and waits for it, one read in
// flight at a time (measured: the Gemma-4 bank's quantize 1-2% faster).
__device__ __forceinline__ void read_staged_block(const uint8_t* stage, uint32_t off, int n, float (&x)[kBlock],
                                                  uint32_t zero) {
  const uint32_t base = lds_addr(stage);
  const uint32_t q0 = off >> 4;
  u32x4 raw[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) raw[c] = lds_read16(8 * c < n ? base + 16u * swz(q0 + c) : zero);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < 16; ++c) unpack8(raw[c], x, c);
}

// Write the first n values (n a multiple of 8) of a block, already packed as
// bf16 pairs, at byte offset `off` of a swizzled stage.  Chunks past n go to
// `junk` (the LDS address of a 16-byte slot nobody reads).
__device__ __forceinline__ void write_staged_block(uint8_t* stage, uint32_t off, int n, const uint32_t (&pk)[kBlock / 2],
                                                   uint32_t junk) {
  const uint32_t base = lds_addr(stage);
  const uint32_t q0 = off >> 4;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    lds_write16(8 * c < n ? base + 16u * swz(q0 + c) : junk, u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]});
}


// Buffer resource over `bytes` bytes at `base` (raw, unswizzled): the full
// paths address a batch as base + per-lane VGPR offset + scalar offset, so
// their loads and stores need no per-lane 64-bit address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t batch_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// Stage a full batch (16 KB, read once: streaming loads).
__device__ __forceinline__ void stage_in_full(__amdgpu_buffer_rsrc_t src, uint8_t* stage, const SwzLane& sl) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(stage + 1024 * i), 16,
                                             sl.o[i & 3], 1024 * i, 0, kNt);
}

__device__ __forceinline__ void read_block_full(uint32_t a, float (&x)[kBlock]) {
#pragma unroll
  for (int c = 0; c < 16; ++c) unpack8(lds_read16(a ^ (16u * c)), x, c);
}

// The same with TQ3's D1 applied at no extra cost: the low bf16 of a word
// becomes (w << 16) + sign (adding 2^31 to a value whose low 16 bits are zero
// flips bit 31 and nothing else) and the high one (w & 0xffff0000) ^ sign, one
// instruction each, as without the signs.
__device__ __forceinline__ void read_block_full_signed(uint32_t a, float (&x)[kBlock], const SignBits& d1) {
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const u32x4 v = lds_read16(a ^ (16u * c));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = 8 * c + 2 * q;
      x[j] = __uint_as_float((w[q] << 16) + sign_bit(d1, j));
      x[j + 1] = __uint_as_float((w[q] & 0xffff0000u) ^ sign_bit(d1, j + 1));
    }
  }
}

__device__ __forceinline__ void write_block_full(uint32_t a, const uint32_t (&pk)[kBlock / 2]) {
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const u32x4 v = {pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]};
    lds_write16(a ^ (16u * c), v);
  }
}


__device__ __forceinline__ void stage_out_full(__amdgpu_buffer_rsrc_t dst, uint32_t stage, const SwzLane& sl, int lane) {
  lds_handover();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const u32x4 v = lds_read16(stage + 1024u * i + sl.o[i & 3]);
    __builtin_amdgcn_raw_buffer_store_b128(v, dst, 16u * lane, 1024 * i, kNt);
  }
  lds_handover();
}

// ---------------------------------------------------------------------------
// weight kernels (grouped: up to kMaxGroup matrices per launch)
//
// A wave works on batches of 64 consecutive blocks of one matrix, one block
// per lane.  Blocks are numbered row-major, so a batch covers one contiguous
// byte range of W (rows are contiguous; a tail block holds only its real
// columns).  Quantize workgroups loop over batches (persistent grid);
// dequantize workgroups each own a run of consecutive batches (batch_range).
// ---------------------------------------------------------------------------

// TQ3's quantizer state for a launch: the two sign vectors, and D2 once more
// as a mask over a block's 384-bit string of 3-bit codes (0b111 on every code
// whose D2 entry is -1).  Negating a centroid is the same as mirroring its
// code, c[7 - k] = -c[k] exactly (the codebook is symmetric), and 7 - k = k ^ 7,
// so the dequantizer applies D2 with one xor per code word.
struct TqSigns {
  SignBits d1, d2;
  uint32_t flip2[12];
};

// SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): the state advances by the golden-ratio gamma and
// each output is the state through the variant-13 mix (shifts 30, 27, 31).
constexpr uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// TQ3's state for a seed: entry i of D1 is -1 when the top bit of output i is
// set, entry i of D2 likewise with output 128 + i.
constexpr TqSigns tq3_state(uint64_t seed) {
  TqSigns t{};
  uint64_t state = seed;
  for (int i = 0; i < 2 * kBlock; ++i) {
    if (splitmix64_next(state) >> 63) {
      SignBits& d = i < kBlock ? t.d1 : t.d2;
      const int e = i & (kBlock - 1);
      d.w[e >> 5] |= 1u << (e & 31);
    }
  }
  for (int j = 0; j < kBlock; ++j)
    if ((t.d2.w[j >> 5] >> (j & 31)) & 1u)
      for (int b = 3 * j; b < 3 * j + 3; ++b) t.flip2[b >> 5] |= 1u << (b & 31);
  return t;
}

// The format's recorded quantizer state (seed 42, "Qwen3.6-35B-A3B-TQ3-native",
// section "Files"), compiled into its own kernels: every sign is then a
// constant and costs nothing (a negation folds into the instruction that reads
// the value, a table choice into an immediate).
constexpr uint64_t kTq3Seed = 42;
constexpr TqSigns kTq3Seed42 = tq3_state(kTq3Seed);

struct WeightGroup {
  int32_t n;                           // matrices in this launch
  uint32_t total_batches;              // sum of batches over the matrices
  uint32_t chunk;                      // batches per workgroup (a multiple of kWaves), 0: persistent grid
  uint32_t batch_start[kMaxGroup + 1]; // first batch of every matrix (prefix sum)
  uint32_t nblocks[kMaxGroup];         // rows * nb
  uint32_t nb[kMaxGroup];              // blocks per row
  int32_t staged[kMaxGroup];           // 1: W rows start 16-byte aligned (in % 8 == 0, W aligned)
  int32_t whole[kMaxGroup];            // 1: staged and in % 128 == 0 (every block whole)
  int64_t in[kMaxGroup];               // columns
  uint16_t* w[kMaxGroup];
  uint8_t* packed[kMaxGroup];
  void* norms[kMaxGroup];              // fp16 (HLWQ) or fp32 (TQ3)
  TqSigns tq;                          // TQ3 launches only
};

// The batches of one wave: with a persistent grid (chunk == 0) every wave
// strides over the whole range; otherwise workgroup k owns the `chunk`
// consecutive batches from k * chunk on, the grid has one workgroup per chunk,
// and the hardware hands out workgroups as earlier ones finish.
struct BatchRange {
  uint32_t b, step, end;
};
__device__ __forceinline__ BatchRange batch_range(uint32_t total, uint32_t chunk, int wave) {
  BatchRange r;
  if (chunk == 0u) {
    r.b = blockIdx.x * kWaves + wave;
    r.step = gridDim.x * kWaves;
    r.end = total;
  } else {
    r.b = blockIdx.x * chunk + wave;
    r.step = kWaves;
    const uint32_t e = (blockIdx.x + 1u) * chunk;
    r.end = e < total ? e : total;
  }
  return r;
}

// matrix owning batch b (uniform across the wave)
__device__ __forceinline__ int group_of(const WeightGroup& g, uint32_t b) {
  int d = 0;
  for (int i = 1; i < g.n; ++i) d = (b >= g.batch_start[i]) ? i : d;
  return d;
}

struct BatchPos {
  uint32_t g0, nvalid, lb;
  int64_t e;  // element offset of this lane's block in W
  int n;      // real values in this lane's block
};

__device__ __forceinline__ BatchPos batch_pos(const WeightGroup& g, int d, uint32_t b, int lane) {
  BatchPos p;
  p.g0 = (b - g.batch_start[d]) * 64u;
  const uint32_t left = g.nblocks[d] - p.g0;
  p.nvalid = left < 64u ? left : 64u;
  p.lb = p.g0 + (static_cast<uint32_t>(lane) < p.nvalid ? static_cast<uint32_t>(lane) : p.nvalid - 1);
  const uint32_t nb = g.nb[d];
  const uint32_t row = p.lb / nb;
  const uint32_t blk = p.lb - row * nb;
  const int64_t in = g.in[d];
  const int64_t col = static_cast<int64_t>(blk) * kBlock;
  p.e = static_cast<int64_t>(row) * in + col;
  p.n = static_cast<int>((in - col) < kBlock ? (in - col) : kBlock);
  return p;
}

// FIELD: bits per stored code, BITS (packed) or 8 (one code per byte).
// TQ: TQ3 ("Qwen3.6-35B-A3B-TQ3-native", section "What TQ3 actually does"):
// the block is multiplied by D1 before the butterflies and its rotated values
// by D2, and the stored norm is the fp32 shape-gain n / (rho / sqrt(128)), rho
// the norm of the selected centroids.  TQ = 1 takes the signs from the launch
// arguments, TQ = 2 is the compiled-in seed-42 state.
template <int BITS, int FIELD, int TQ = 0>
__global__ void __launch_bounds__(kPoolThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) hlwq_quantize_kernel(const WeightGroup g) {
  static_assert(!TQ || (BITS == 3 && FIELD == 3), "TQ3 stores packed 3-bit codes");
  // one LDS array: the entry table at offset 0 (so its reads need no base
  // add), the bucket table (and TQ3's mirrored one), a zero slot, then the
  // 256-byte aligned per-wave stages
  constexpr int kZero = 256 + (TQ ? 2 : 1) * HLWQ_BUCKETS;  // 16 zero bytes for the reads past a tail block
  constexpr int kTab = kZero + 256;
  __shared__ __attribute__((aligned(256))) uint8_t lds[kTab + kPoolWaves * kStage];
  __shared__ uint32_t next_batch;  // the workgroup's work pool
  uint32_t* tab = reinterpret_cast<uint32_t*>(lds);
  uint8_t* stage_all = lds + kTab;
  if (threadIdx.x < 4) tab[kZero / 4 + threadIdx.x] = 0u;
  const uint32_t* src_bucket = (BITS == 5) ? c_bucket5 : c_bucket3;
  const uint32_t* src_entry = (BITS == 5) ? c_entry5 : c_entry3;
  if (threadIdx.x == 0) next_batch = kPoolWaves;
  for (int i = threadIdx.x; i < HLWQ_BUCKETS / 4; i += kPoolThreads) tab[64 + i] = src_bucket[i];
  if (threadIdx.x < 2 * (1 << BITS)) tab[threadIdx.x] = src_entry[threadIdx.x];
  if constexpr (TQ) {
    // the mirrored entries at byte 64, the mirrored buckets after the plain ones
    for (int i = threadIdx.x; i < HLWQ_BUCKETS / 4; i += kPoolThreads) tab[64 + HLWQ_BUCKETS / 4 + i] = c_bucket3m[i];
    if (threadIdx.x < 16) tab[16 + threadIdx.x] = c_entry3m[threadIdx.x];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = stage_all + wave * kStage;
  SwzLane sl = swz_lane(lane);
  uint32_t lane_a = lds_addr(stage) + 256u * lane + 16u * (lane & 15);
  constexpr uint32_t kOut = 16 * FIELD;  // code bytes per block

  // Work pool: the workgroup (one per CU) owns batches blockIdx.x + gridDim.x m,
  // m = 0, 1, ..., and its waves take m in turn from an LDS counter, each
  // fetching its next m one batch ahead.  Of the two waves sharing a SIMD the
  // older one is issued first and runs ahead, so with a fixed share per wave
  // the younger ones finish last; drawing from a common pool, the waves of a
  // CU finish within about one batch of each other.
  uint32_t m = wave;
  for (uint32_t b = blockIdx.x + gridDim.x * m; b < g.total_batches;) {
    uint32_t m_next = 0;
    if (lane == 0) m_next = __hip_atomic_fetch_add(&next_batch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    refresh(sl, lane_a);
    const int d = group_of(g, b);
    const BatchPos p = batch_pos(g, d, b, lane);

    // TQ3's sign vectors (D1 is applied while the block is read; squares, and
    // so the norm, do not see it)
    SignBits d1{}, d2{};
    if constexpr (TQ == 1) {
      d1 = per_batch(g.tq.d1);
      d2 = per_batch(g.tq.d2);
    } else if constexpr (TQ == 2) {
      d1 = kTq3Seed42.d1;
      d2 = kTq3Seed42.d2;
    }
    float x[kBlock];
    if (g.whole[d] && p.nvalid == 64u) {
      stage_in_full(batch_rsrc(g.w[d] + static_cast<int64_t>(p.g0) * kBlock, 64u * 2u * kBlock), stage, sl);
      wait_vmem();
      if constexpr (TQ != 0) read_block_full_signed(lane_a, x, d1);
      else read_block_full(lane_a, x);
    } else {
      if (g.staged[d]) {
        const int64_t e0 = first_lane64(p.e);
        const uint32_t off = static_cast<uint32_t>(p.e - e0) * 2u;
        const uint32_t end = __builtin_amdgcn_readlane(off + 2u * p.n, p.nvalid - 1);
        stage_in<16, true, kNt>(reinterpret_cast<const uint8_t*>(g.w[d] + e0), end, stage, lane, sl);
        wait_vmem();
        read_staged_block(stage, off, p.n, x, lds_addr(lds + kZero));
      } else {
        load_block(g.w[d] + p.e, p.n, x);
      }
      if constexpr (TQ != 0) {
#pragma unroll
        for (int i = 0; i < kBlock; ++i) x[i] = __uint_as_float(__float_as_uint(x[i]) ^ sign_bit(d1, i));
      }
    }

    const NormInfo ni = norm_info(sumsq_tree(x));
    fwht(x);
    uint32_t words[4 * FIELD];
    encode<FIELD, kBlock, TQ != 0>(x, ni.r, lds, 256u, __uint_as_float(HLWQ_BUCKET_BIAS), words, d2);
    float gain = 0.0f;
    if constexpr (TQ != 0) {
      // mirrored codes -> codes of -y
#pragma unroll
      for (int q = 0; q < 4 * FIELD; ++q) words[q] ^= (TQ == 2) ? kTq3Seed42.flip2[q] : g.tq.flip2[q];
      // RN(1 / sqrt(128)) = RN(sqrt(2)) / 16
      const float t = sqrtf(recon_sumsq3(words)) * 0x1.6a09e6p-4f;
      gain = ni.n / t;
    }

    // the codes of the batch are contiguous: kOut bytes per block
#pragma unroll
    for (int q = 0; q < FIELD; ++q) {
      const u32x4 v = {words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]};
      *reinterpret_cast<u32x4*>(stage + kOut * lane + 16 * q) = v;
    }
    stage_out<FIELD, false>(g.packed[d] + static_cast<size_t>(p.g0) * kOut, p.nvalid * kOut, stage, lane, sl);
    if (static_cast<uint32_t>(lane) < p.nvalid) {
      if constexpr (TQ != 0) static_cast<float*>(g.norms[d])[p.lb] = gain;
      else static_cast<uint16_t*>(g.norms[d])[p.lb] = ni.n16;
    }
    m = __builtin_amdgcn_readfirstlane(m_next);
    b = blockIdx.x + gridDim.x * m;
  }
}

// TQ: TQ3's inverse (1: signs from the launch arguments, 2: the compiled-in
// seed-42 state): D2 mirrors the codes, the butterflies run as for HLWQ, the
// scale is the fp32 shape-gain / 128 and D1 negates the bf16 results.
template <int BITS, int FIELD, int TQ = 0>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) hlwq_dequantize_kernel(const WeightGroup g) {
  static_assert(!TQ || (BITS == 3 && FIELD == 3), "TQ3 stores packed 3-bit codes");
  // one LDS array: the centroid pair table at offset 0, then the per-wave stages
  constexpr int kPairs = 8 << (2 * BITS);
  constexpr int kJunk = kPairs;  // a 16-byte slot for the writes past a tail block
  __shared__ __attribute__((aligned(256))) uint8_t lds[kPairs + 256 + kWaves * kStage];
  uint8_t* stage_all = lds + kPairs + 256;
  fill_pairs<BITS>(reinterpret_cast<float*>(lds), (BITS == 5) ? c_cent5 : c_cent3);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = stage_all + wave * kStage;
  SwzLane sl = swz_lane(lane);
  uint32_t lane_a = lds_addr(stage) + 256u * lane + 16u * (lane & 15);
  constexpr uint32_t kIn = 16 * FIELD;  // code bytes per block

  const BatchRange br = batch_range(g.total_batches, g.chunk, wave);
  for (uint32_t b = br.b; b < br.end; b += br.step) {
    refresh(sl, lane_a);
    const int d = group_of(g, b);
    const BatchPos p = batch_pos(g, d, b, lane);

    stage_in<FIELD, false, 0>(g.packed[d] + static_cast<size_t>(p.g0) * kIn, p.nvalid * kIn, stage, lane, sl);
    float nv;
    if constexpr (TQ != 0) nv = static_cast<const float*>(g.norms[d])[p.lb];
    else nv = f16_value(static_cast<const uint16_t*>(g.norms[d])[p.lb]);
    const float scale = nv * 0x1p-7f;
    wait_vmem();
    // lanes past the end of the batch read (and later write) the last block
    const uint32_t slot = p.lb - p.g0;
    uint32_t words[4 * FIELD];
#pragma unroll
    for (int q = 0; q < FIELD; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + kIn * slot + 16 * q);
      words[4 * q] = v.x;
      words[4 * q + 1] = v.y;
      words[4 * q + 2] = v.z;
      words[4 * q + 3] = v.w;
    }
    SignBits d1{};
    if constexpr (TQ == 1) {
      d1 = per_batch(g.tq.d1);
#pragma unroll
      for (int q = 0; q < 4 * FIELD; ++q) words[q] ^= g.tq.flip2[q];
    } else if constexpr (TQ == 2) {
      d1 = kTq3Seed42.d1;
#pragma unroll
      for (int q = 0; q < 4 * FIELD; ++q) words[q] ^= kTq3Seed42.flip2[q];
    }

    float v[kBlock];
    if constexpr (FIELD == BITS) decode_stage1<BITS, kBlock>(words, lds, v);
    else decode_bytes_stage1<BITS, kBlock>(words, lds, v);
    fwht<kBlock, 2>(v);
    uint32_t pk[kBlock / 2];
#pragma unroll
    for (int j = 0; j < kBlock; j += 2)
      pk[j / 2] = pack_bf16x2(v[j] * scale, v[j + 1] * scale) ^ (TQ != 0 ? pair_sign_mask(d1, j / 2) : 0u);

    if (g.whole[d] && p.nvalid == 64u) {
      write_block_full(lane_a, pk);
      stage_out_full(batch_rsrc(g.w[d] + static_cast<int64_t>(p.g0) * kBlock, 64u * 2u * kBlock), lds_addr(stage), sl,
                     lane);
    } else if (g.staged[d]) {
      const int64_t e0 = first_lane64(p.e);
      const uint32_t off = static_cast<uint32_t>(p.e - e0) * 2u;
      const uint32_t end = __builtin_amdgcn_readlane(off + 2u * p.n, p.nvalid - 1);
      // lanes past the end of the batch repeat the last block: identical bytes
      write_staged_block(stage, off, p.n, pk, lds_addr(lds + kJunk));
      stage_out<16, true>(reinterpret_cast<uint8_t*>(g.w[d] + e0), end, stage, lane, sl);
    } else if (static_cast<uint32_t>(lane) < p.nvalid) {
      store_block(g.w[d] + p.e, p.n, pk);
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantize straight to INT4 with one scale and zero point per 128-column
// group (= one HLWQ block; `in` is a multiple of 128): the bf16 values the
// dequantize kernel would write are formed in registers and re-quantised,
// without the bf16 round trip through HBM.  Per group, in fp32:
// lo = min(0, min w), hi = max(0, max w), scale = (hi - lo) / 15 (1 if 0),
// inv = 1 / scale, zp = clamp(rint(-lo * inv), 0, 15),
// q = clamp(rint(w * inv) + zp, 0, 15), two codes per byte, low nibble first.
// ---------------------------------------------------------------------------

// Up to kMaxGroup matrices per launch, batches of 64 blocks numbered over the
// matrices in order (a prefix sum), as in the grouped weight kernels.
struct Int4Group {
  int32_t n;
  uint32_t total_batches;
  uint32_t batch_start[kMaxGroup + 1];
  uint32_t nblocks[kMaxGroup];
  const uint8_t* packed[kMaxGroup];   // [nblocks][16 * bits]
  const uint16_t* norms[kMaxGroup];   // [nblocks]
  uint8_t* q4[kMaxGroup];             // [nblocks][64]
  float* scales[kMaxGroup];           // [nblocks]
  uint8_t* zeros[kMaxGroup];          // [nblocks]
};

__device__ __forceinline__ int int4_group_of(const Int4Group& g, uint32_t b) {
  int d = 0;
  for (int i = 1; i < g.n; ++i) d = (b >= g.batch_start[i]) ? i : d;
  return d;
}

constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23: x + it rounds x to an integer, ties to even

template <int BITS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) hlwq_dequantize_int4_kernel(const Int4Group a) {
  constexpr int kPairs = 8 << (2 * BITS);
  constexpr uint32_t kIn = 16 * BITS;  // packed bytes per block
  constexpr int kArea = 8192;          // per wave: the batch's codes in, then its nibbles out
  __shared__ __attribute__((aligned(256))) uint8_t pairs[kPairs];
  __shared__ __attribute__((aligned(256))) uint8_t areas[kWaves * kArea];
  fill_pairs<BITS>(reinterpret_cast<float*>(pairs), (BITS == 5) ? c_cent5 : c_cent3);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* area = areas + wave * kArea;
  SwzLane sl = swz_lane(lane);
  uint32_t lane_a = 0;

  for (uint32_t b = blockIdx.x * kWaves + wave; b < a.total_batches; b += gridDim.x * kWaves) {
    refresh(sl, lane_a);
    const int d = int4_group_of(a, b);
    const uint32_t g0 = (b - a.batch_start[d]) * 64u;
    const uint32_t left = a.nblocks[d] - g0;
    const uint32_t nvalid = left < 64u ? left : 64u;
    // lanes past the end of the batch repeat the last block and store nothing
    const uint32_t slot = static_cast<uint32_t>(lane) < nvalid ? static_cast<uint32_t>(lane) : nvalid - 1;
    stage_in<BITS, false, 0>(a.packed[d] + static_cast<size_t>(g0) * kIn, nvalid * kIn, area, lane, sl);
    const float nscale = f16_value(a.norms[d][g0 + slot]) * 0x1p-7f;
    wait_vmem();
    uint32_t words[4 * BITS];
#pragma unroll
    for (int q = 0; q < BITS; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(area + kIn * slot + 16 * q);
      words[4 * q] = v.x;
      words[4 * q + 1] = v.y;
      words[4 * q + 2] = v.z;
      words[4 * q + 3] = v.w;
    }
    lds_handover();  // the area is refilled with output below

    float v[kBlock];
    decode_stage1<BITS, kBlock>(words, pairs, v);
    fwht<kBlock, 2>(v);
    // the group's bounds, taken on the fp32 values before their bf16
    // rounding: rounding to nearest is monotone, so the rounded minimum is
    // the minimum of the rounded values (likewise the maximum)
#pragma unroll
    for (int j = 0; j < kBlock; ++j) v[j] = v[j] * nscale;
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
      lo = fminf(lo, v[j]);
      hi = fmaxf(hi, v[j]);
    }
    {
      const uint32_t lh = pack_bf16x2(lo, hi);
      lo = bf16_lo(lh);
      hi = bf16_hi(lh);
    }
    float scale = (hi - lo) / 15.0f;
    scale = (scale == 0.0f) ? 1.0f : scale;
    const float inv = 1.0f / scale;
    const int32_t zp = static_cast<int32_t>(__builtin_fminf(__builtin_fmaxf(__builtin_rintf(-lo * inv), 0.0f), 15.0f));
    // q = clamp(rint(RN(w * inv)) + zp, 0, 15): t = RN(RN(w * inv) + 1.5 2^23)
    // is the integer rint(RN(w * inv)) + 1.5 2^23, exact in the binade
    // [2^23, 2^24) where consecutive integers have consecutive bit patterns;
    // clamped there to [B, B + 15], B = 1.5 2^23 - zp, its bits are bits(B) + q.
    // The Horner steps acc = acc 16 + bits(t) then give, modulo 2^32, the
    // nibbles plus bits(B) 0x11111111, taken off once per word.
    const float qlo = kRoundMagic - static_cast<float>(zp), qhi = qlo + 15.0f;
    const uint32_t excess = __float_as_uint(qlo) * 0x11111111u;
    uint32_t nib[16];
#pragma unroll
    for (int mw = 0; mw < 16; ++mw) {
      uint32_t w2[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w2[k] = pack_bf16x2(v[8 * mw + 2 * k], v[8 * mw + 2 * k + 1]);
      uint32_t acc = 0;
#pragma unroll
      for (int k = 7; k >= 0; --k) {
        const float w = (k & 1) ? bf16_hi(w2[k >> 1]) : bf16_lo(w2[k >> 1]);
        const float t = __builtin_amdgcn_fmed3f(w * inv + kRoundMagic, qlo, qhi);
        acc = (acc << 4) + __float_as_uint(t);
      }
      nib[mw] = acc - excess;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 val = {nib[4 * q], nib[4 * q + 1], nib[4 * q + 2], nib[4 * q + 3]};
      *reinterpret_cast<u32x4*>(area + 64 * lane + 16 * q) = val;
    }
    stage_out<4, false>(a.q4[d] + static_cast<size_t>(g0) * 64, nvalid * 64u, area, lane, sl);
    if (static_cast<uint32_t>(lane) < nvalid) {
      a.scales[d][g0 + lane] = scale;
      a.zeros[d][g0 + lane] = static_cast<uint8_t>(zp);
    }
  }
}

// ---------------------------------------------------------------------------
// KV-cache kernels: a 256-wide head vector over four adjacent lanes (64
// values each); a wave works on batches of 16 consecutive tokens of one head
// (8 KB of bf16).  With ~110 VGPRs and 8 KB of stage per wave, four waves
// share a SIMD: a KV launch is a few rounds of batches, and the extra waves
// hide the start and the end of the launch better than two waves with twice
// the batch (measured 13% faster quantize, 2% faster dequantize).
//
// Stage layout: lane l's quarter vector (128 B) is row l of the stage, its
// 16-byte chunk c at byte 128 l + 16 (c ^ (l % 8)), so the eight lanes an LDS
// cycle serves hit eight different bank groups.  Load instruction k, lane i
// fetches the chunk that lands in slot 64 k + i: row 8 k + i / 8, chunk
// (i % 8) ^ (i / 8 % 8), i.e. global byte 1024 k + kv_lane_offset(i); every
// instruction is still one contiguous KB of HBM.  Stores use the same map.
// ---------------------------------------------------------------------------

// Division of a wave-uniform 32-bit numerator by a launch-invariant divisor
// d >= 1 on the scalar unit (Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, section 4): with l = ceil(log2 d)
// and m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> s1)) >> s2
// for t = mulhi(m, n), s1 = min(l, 1), s2 = max(l - 1, 0).
struct UDiv {
  uint32_t m, s1, s2;
};
UDiv make_udiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t{1} << l) < d) ++l;
  UDiv v;
  v.m = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
  v.s1 = l < 1 ? l : 1;
  v.s2 = l > 1 ? l - 1 : 0;
  return v;
}
__device__ __forceinline__ uint32_t udiv(uint32_t n, const UDiv& v) {
  const uint32_t t = __umulhi(v.m, n);
  return (t + ((n - t) >> v.s1)) >> v.s2;
}

struct KvArgs {
  uint16_t* kv;       // [bh][tokens][256]
  uint8_t* packed;    // [bh][out_stride][32 * bits]
  uint16_t* norms;    // [bh][out_stride]
  int64_t tokens;     // kv rows per head
  int64_t out_stride; // packed / norms rows per head
  int64_t out_offset; // row of token 0 in packed / norms
  uint32_t tq;        // quantised tokens per head
  uint32_t nbt;       // batches per head, ceil(tq / 16)
  UDiv nbt_div;       // division by nbt
  uint32_t total_batches;
  uint32_t chunk;      // batches per workgroup, 0 for a persistent grid (batch_range)
};

constexpr int kKvTokens = 16;    // tokens per batch
constexpr int kKvStage = 8192;   // LDS bytes per wave

__device__ __forceinline__ uint32_t kv_lane_offset(uint32_t i) { return 128u * (i >> 3) + 16u * ((i & 7u) ^ ((i >> 3) & 7u)); }

// value of the lane whose id differs in bit 1 (quad permutation [2,3,0,1])
__device__ __forceinline__ float lane_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}


// One butterfly stage across lanes folded into one instruction per value:
// x = fma(partner's x, c, x) with c = +1 or -1 per lane, v_fmac_f32 with a DPP
// quad permutation on the partner operand.  The lower lane of a pair gets
// a + b and the upper one b - a = -(a - b): the true value times a sign the
// caller tracks (negation is exact, and so is c * partner).  The compiler does
// not fold a DPP operand into a fused multiply-add, hence the inline assembly;
// a DPP read of a VGPR needs two wait states after the VALU write of it, which
// the leading s_nop 1 provides for the whole group (every instruction of a
// group reads a value written before the group).
#define HLWQ_FMAC_DPP(i, perm) "v_fmac_f32_dpp %" #i ", %" #i ", %16 quad_perm:" perm " row_mask:0xf bank_mask:0xf\n\t"
#define HLWQ_FMAC_DPP16(perm)                                                                                          \
  "s_nop 1\n\t" HLWQ_FMAC_DPP(0, perm) HLWQ_FMAC_DPP(1, perm) HLWQ_FMAC_DPP(2, perm) HLWQ_FMAC_DPP(3, perm)            \
      HLWQ_FMAC_DPP(4, perm) HLWQ_FMAC_DPP(5, perm) HLWQ_FMAC_DPP(6, perm) HLWQ_FMAC_DPP(7, perm)                      \
          HLWQ_FMAC_DPP(8, perm) HLWQ_FMAC_DPP(9, perm) HLWQ_FMAC_DPP(10, perm) HLWQ_FMAC_DPP(11, perm)                \
              HLWQ_FMAC_DPP(12, perm) HLWQ_FMAC_DPP(13, perm) HLWQ_FMAC_DPP(14, perm) HLWQ_FMAC_DPP(15, perm)

template <int XOR>
__device__ __forceinline__ void cross_stage(float (&x)[64], float c) {
#pragma unroll
  for (int j = 0; j < 64; j += 16) {
    if constexpr (XOR == 1)
      asm volatile(HLWQ_FMAC_DPP16("[1,0,3,2]")
                   : "+v"(x[j]), "+v"(x[j + 1]), "+v"(x[j + 2]), "+v"(x[j + 3]), "+v"(x[j + 4]), "+v"(x[j + 5]),
                     "+v"(x[j + 6]), "+v"(x[j + 7]), "+v"(x[j + 8]), "+v"(x[j + 9]), "+v"(x[j + 10]), "+v"(x[j + 11]),
                     "+v"(x[j + 12]), "+v"(x[j + 13]), "+v"(x[j + 14]), "+v"(x[j + 15])
                   : "v"(c));
    else
      asm volatile(HLWQ_FMAC_DPP16("[2,3,0,1]")
                   : "+v"(x[j]), "+v"(x[j + 1]), "+v"(x[j + 2]), "+v"(x[j + 3]), "+v"(x[j + 4]), "+v"(x[j + 5]),
                     "+v"(x[j + 6]), "+v"(x[j + 7]), "+v"(x[j + 8]), "+v"(x[j + 9]), "+v"(x[j + 10]), "+v"(x[j + 11]),
                     "+v"(x[j + 12]), "+v"(x[j + 13]), "+v"(x[j + 14]), "+v"(x[j + 15])
                   : "v"(c));
  }
}

struct KvBatch {
  uint32_t bh, t0, nvalid;
};
__device__ __forceinline__ KvBatch kv_batch(const KvArgs& a, uint32_t b) {
  KvBatch p;
  p.bh = udiv(b, a.nbt_div);
  p.t0 = (b - p.bh * a.nbt) * kKvTokens;
  const uint32_t left = a.tq - p.t0;
  p.nvalid = left < kKvTokens ? left : kKvTokens;
  return p;
}

template <int BITS, int NT = kThreads>
__device__ __forceinline__ void fill_kv_search(uint32_t* tab) {
  const uint32_t* bucket = (BITS == 3) ? c_kvbucket3 : c_kvbucket2;
  const uint32_t* entry = (BITS == 3) ? c_entry3 : c_entry2;
  for (int i = threadIdx.x; i < HLWQ_KV_BUCKETS / 4; i += NT) tab[64 + i] = bucket[i];
  if (threadIdx.x < 2 * (1 << BITS)) tab[threadIdx.x] = entry[threadIdx.x];
}

template <int BITS>
__global__ void __launch_bounds__(kKvPoolThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) hlwq_kv_quantize_kernel(const KvArgs a) {
  // entry table at offset 0, bucket table, per-wave stages
  constexpr int kTab = 256 + HLWQ_KV_BUCKETS;
  constexpr uint32_t kVec = 32 * BITS;  // packed bytes per vector
  __shared__ __attribute__((aligned(256))) uint8_t lds[kTab + kKvPoolWaves * kKvStage];
  __shared__ uint32_t next_batch;
  if (threadIdx.x == 0) next_batch = kKvPoolWaves;
  uint32_t* tab = reinterpret_cast<uint32_t*>(lds);
  fill_kv_search<BITS, kKvPoolThreads>(tab);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = lds + kTab + wave * kKvStage;
  const uint32_t ul = static_cast<uint32_t>(lane);
  uint32_t vsrc = kv_lane_offset(ul);
  uint32_t row_a = lds_addr(stage) + 128u * ul;
  const uint32_t q = ul & 3u;  // quarter of the vector
  const uint32_t v = ul >> 2;  // token of the batch
  const float sgn1 = pair_sign(q & 1u), sgn2 = pair_sign(q & 2u);

  // work pool, as in the weight quantizer: one 16-wave workgroup per CU takes
  // batches blockIdx.x + gridDim.x m in turn from an LDS counter
  uint32_t m = wave;
  for (uint32_t b = blockIdx.x + gridDim.x * m; b < a.total_batches;) {
    uint32_t m_next = 0;
    if (lane == 0) m_next = __hip_atomic_fetch_add(&next_batch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    asm volatile("" : "+v"(vsrc), "+v"(row_a));  // keep the address bases in one VGPR each
    const KvBatch p = kv_batch(a, b);
    const uint16_t* src = a.kv + (static_cast<int64_t>(p.bh) * a.tokens + p.t0) * kKvDim;
    // a buffer resource over the batch's tokens: the chunks of a short
    // batch's missing tokens lie past its end and read as zeros (their lanes
    // compute on them and store nothing); the whole offset is in the VGPR
    // operand, which is what the range check covers
    const auto rs = batch_rsrc(src, p.nvalid * 2u * kKvDim);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + 1024 * k), 16,
                                               1024u * k + vsrc, 0, 0, kNt);
    wait_vmem();
    float x[64];
#pragma unroll
    for (int c = 0; c < 8; ++c) unpack8(lds_read16(row_a + 16u * (static_cast<uint32_t>(c) ^ (ul & 7u))), x, c);

    // norm tree: levels 0..5 in the lane, 6 and 7 across the quarters (addition commutes)
    const float s1 = sumsq_tree(x);
    const float s2 = s1 + lane_xor1(s1);
    const NormInfo ni = norm_info(s2 + lane_xor2(s2));
    // butterflies at strides 1..32 in the lane, 64 and 128 across the quarters
    fwht(x);
    // strides 64 and 128: lane q then holds its values times sgn1 * sgn2
    // (+, -, -, + for q = 0..3), which the reciprocal norm takes back exactly
    cross_stage<1>(x, sgn1);
    cross_stage<2>(x, sgn2);
    uint32_t words[2 * BITS];
    encode<BITS, 64>(x, ni.r * (sgn1 * sgn2), lds, 256u, __uint_as_float(HLWQ_KV_BUCKET_BIAS), words);
    // the batch's codes are contiguous: lane l's 8 BITS bytes at 8 BITS l
    lds_handover();
    if constexpr (BITS == 3) {
      uint2* o = reinterpret_cast<uint2*>(stage + 24u * ul);
      o[0] = uint2{words[0], words[1]};
      o[1] = uint2{words[2], words[3]};
      o[2] = uint2{words[4], words[5]};
    } else {
      *reinterpret_cast<u32x4*>(stage + 16u * ul) = u32x4{words[0], words[1], words[2], words[3]};
    }
    const size_t vec0 = static_cast<size_t>(p.bh) * a.out_stride + a.out_offset + p.t0;
    const SwzLane linear{};
    stage_out<2, false>(a.packed + vec0 * kVec, p.nvalid * kVec, stage, lane, linear);
    if (q == 0u && v < p.nvalid) a.norms[vec0 + v] = ni.n16;
    m = __builtin_amdgcn_readfirstlane(m_next);
    b = blockIdx.x + gridDim.x * m;
  }
}

template <int BITS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) hlwq_kv_dequantize_kernel(const KvArgs a) {
  // centroid pair table at offset 0 (512 bytes at most), then the per-wave stages
  constexpr uint32_t kVec = 32 * BITS;  // packed bytes per vector
  __shared__ __attribute__((aligned(256))) uint8_t lds[512 + kWaves * kKvStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* stage = lds + 512 + wave * kKvStage;
  const uint32_t ul = static_cast<uint32_t>(lane);
  uint32_t vsrc = kv_lane_offset(ul);
  uint32_t stage_a = lds_addr(stage);
  const uint32_t q = ul & 3u;
  const uint32_t v = ul >> 2;
  const float sgn1 = pair_sign(q & 1u), sgn2 = pair_sign(q & 2u);
  const SwzLane linear{};

  // Codes and norm of batch b: the codes go to the stage, the norm to `n16`.
  // A workgroup is short-lived (one batch per wave at the usual chunk), so the
  // first batch's are requested before the pair table is built and the table
  // fill runs while they are in flight.  (The longer-lived weight dequantizer
  // and the KV quantizer measured slower with the same change.)
  KvBatch p{};
  size_t vec0 = 0;
  uint32_t vv = 0;
  uint16_t n16 = 0;
  auto request = [&](uint32_t bb) {
    asm volatile("" : "+v"(vsrc), "+v"(stage_a));
    p = kv_batch(a, bb);
    vv = v < p.nvalid ? v : p.nvalid - 1u;  // lanes past the end repeat the last token
    vec0 = static_cast<size_t>(p.bh) * a.out_stride + a.out_offset + p.t0;
    stage_in<2, false, 0>(a.packed + vec0 * kVec, p.nvalid * kVec, stage, lane, linear);
    n16 = a.norms[vec0 + vv];
  };
  const BatchRange br = batch_range(a.total_batches, a.chunk, wave);
  if (br.b < br.end) request(br.b);
  fill_pairs<BITS>(reinterpret_cast<float*>(lds), (BITS == 3) ? c_cent3 : c_cent2);
  __syncthreads();

  for (uint32_t b = br.b; b < br.end; b += br.step) {
    if (b != br.b) request(b);
    const float scale = f16_value(n16) * 0x1p-8f;
    wait_vmem();
    uint32_t words[2 * BITS];
    const uint32_t lo = kVec * vv + 8u * BITS * q;
    if constexpr (BITS == 3) {
      const uint2* w = reinterpret_cast<const uint2*>(stage + lo);
      const uint2 w0 = w[0], w1 = w[1], w2 = w[2];
      words[0] = w0.x;
      words[1] = w0.y;
      words[2] = w1.x;
      words[3] = w1.y;
      words[4] = w2.x;
      words[5] = w2.y;
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(stage + lo);
      words[0] = w.x;
      words[1] = w.y;
      words[2] = w.z;
      words[3] = w.w;
    }
    lds_handover();  // the stage is rewritten with this batch's output below

    float x[64];
    decode_stage1<BITS, 64>(words, lds, x);
    fwht<64, 2>(x);
#pragma unroll
    for (int j = 0; j < 64; ++j) x[j] = lane_xor1(x[j]) + x[j] * sgn1;
    // stride-128 stage, then scale and round to bf16
    uint32_t pk[32];
#pragma unroll
    for (int j = 0; j < 64; j += 2)
      pk[j / 2] = pack_bf16x2((lane_xor2(x[j]) + x[j] * sgn2) * scale, (lane_xor2(x[j + 1]) + x[j + 1] * sgn2) * scale);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      lds_write16(stage_a + 128u * ul + 16u * (static_cast<uint32_t>(c) ^ (ul & 7u)),
                  u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]});
    lds_handover();
    // stores through a buffer resource over the batch's tokens: those of
    // missing tokens lie past its end and are dropped
    const auto rd = batch_rsrc(a.kv + (static_cast<int64_t>(p.bh) * a.tokens + p.t0) * kKvDim, p.nvalid * 2u * kKvDim);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      __builtin_amdgcn_raw_buffer_store_b128(lds_read16(stage_a + 1024u * k + 16u * ul), rd, 1024u * k + vsrc, 0, kNt);
    lds_handover();
  }
}

// ---------------------------------------------------------------------------
// Streaming KV append: during generation every new token enters the bf16
// window of the newest n_residual tokens (a ring: token t in slot
// t mod n_residual), and the token it pushes out is encoded into the packed
// cache.  The new tokens that arrive and leave within one call are encoded
// straight from the new tokens by the KV quantize kernel (launch_kv with the
// cache's row stride and the call's first row).  The leaving tokens that are
// still in the ring are encoded by one wave per head; a copy kernel launched
// after it on the same stream then writes the new tokens that stay into their
// ring slots, so no slot is overwritten before it is read.
// ---------------------------------------------------------------------------

struct KvAppendArgs {
  const uint16_t* src;  // new tokens [bh][n_new][256]
  uint16_t* ring;       // window [bh][n_res][256]
  uint8_t* packed;      // [bh][capacity][32 * bits]
  uint16_t* norms;      // [bh][capacity]
  int64_t tokens, n_new, n_res, capacity;
  uint32_t bh;           // batch * heads
};

// Encode tokens o0 .. o0 + count - 1 (count <= 32) of head bhi: lane pair
// v = lane / 2 takes token o0 + v (lanes past count repeat the last token and
// store nothing), each lane one half of its 256 values.
template <int BITS>
__device__ __forceinline__ void append_encode(const KvAppendArgs& a, const uint8_t* __restrict__ lds, uint32_t bhi,
                                              int64_t o0, uint32_t count, int lane) {
  constexpr uint32_t kVec = 32 * BITS;
  const uint32_t v = static_cast<uint32_t>(lane) >> 1;
  const uint32_t half = lane & 1;
  const int64_t o = o0 + (v < count ? v : count - 1);
  const uint16_t* p = a.ring + (static_cast<int64_t>(bhi) * a.n_res + o % a.n_res) * kKvDim;
  float x[kBlock];
  load_block(p + half * kBlock, kBlock, x);
  const float s_half = sumsq_tree(x);
  const NormInfo ni = norm_info(s_half + lane_xor1(s_half));
  fwht(x);
  const float sgn = pair_sign(half);
#pragma unroll
  for (int j = 0; j < kBlock; ++j) x[j] = cross_pair(x[j], sgn);
  uint32_t words[4 * BITS];
  encode<BITS, kBlock>(x, ni.r, lds, 256u, __uint_as_float(HLWQ_KV_BUCKET_BIAS), words);
  if (v < count) {
    const int64_t vec = static_cast<int64_t>(bhi) * a.capacity + o;
    u32x4* dst = reinterpret_cast<u32x4*>(a.packed + vec * kVec + half * (kVec / 2));
#pragma unroll
    for (int q = 0; q < BITS; ++q) dst[q] = u32x4{words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]};
    if (half == 0) a.norms[vec] = ni.n16;
  }
}

template <int BITS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) hlwq_kv_append_kernel(const KvAppendArgs a) {
  __shared__ __attribute__((aligned(256))) uint8_t lds[256 + HLWQ_KV_BUCKETS];
  fill_kv_search<BITS>(reinterpret_cast<uint32_t*>(lds));
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const uint32_t bhi = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (bhi >= a.bh) return;
  const int64_t leave_end = a.tokens + a.n_new - a.n_res;              // tokens below this index are encoded afterwards
  const int64_t o_begin = a.tokens > a.n_res ? a.tokens - a.n_res : 0;  // oldest token in the ring
  const int64_t o_end = leave_end < a.tokens ? leave_end : a.tokens;     // leaving tokens still in the ring
  for (int64_t o0 = o_begin; o0 < o_end; o0 += 32) {
    const int64_t n = o_end - o0;
    append_encode<BITS>(a, lds, bhi, o0, static_cast<uint32_t>(n < 32 ? n : 32), lane);
  }
}

// The new tokens that stay in the window, t0 + i for i < ntok (ntok <= n_res),
// into their ring slots (slot0 + i) mod n_res, one 16-byte chunk per
// work-item.  Launched after the ring kernel on the same stream, so every ring
// read of the call has returned before a slot is rewritten.
__global__ void __launch_bounds__(kThreads) hlwq_kv_ring_fill_kernel(const KvAppendArgs a, int64_t t0, int64_t ntok,
                                                                     int64_t slot0) {
  constexpr int64_t kChunks = kKvDim / 8;  // 16-byte chunks per token
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_head = ntok * kChunks;
  if (c >= static_cast<int64_t>(a.bh) * per_head) return;
  const int64_t h = c / per_head;
  const int64_t r = c - h * per_head;
  const int64_t i = r / kChunks, k = r % kChunks;
  const int64_t slot = slot0 + i < a.n_res ? slot0 + i : slot0 + i - a.n_res;
  const u32x4 v = reinterpret_cast<const u32x4*>(a.src + (h * a.n_new + (t0 - a.tokens) + i) * kKvDim)[k];
  reinterpret_cast<u32x4*>(a.ring + (h * a.n_res + slot) * kKvDim)[k] = v;
}

// Streaming KV append, latency path for a few new tokens per head (a decode
// step).  The batch kernel above spends a lane pair on every encoded vector,
// so one token per head would leave 62 of 64 lanes idle and run the whole
// transform serially.  Here one wave encodes one vector at a time with four
// values per lane (lane l holds values 4l .. 4l+3): the norm tree and the
// butterflies finish across lanes (xor shuffles; fp32 addition is
// commutative, so each step is exactly the canonical pairwise sum), and the
// code is the plain count of thresholds below y, which needs no LDS table and
// so no table fill before the first load.  The new tokens that stay in the
// window are loaded at the start and written to the ring last, after every
// ring read of the call has returned.  One wave per head.
constexpr int kSmallAppend = 8;  // new tokens per head handled by the latency path

// Value of lane l ^ d (d a compile-time power of two after unrolling): a DPP
// quad permutation for d = 1 and 2, a swizzle (xor mode, within each half
// wave) for d = 4, 8 and 16, and a bpermute only for d = 32.  The first two
// stay in the VALU and the swizzle needs no address operand; with them the
// decode-step kernel runs 5% faster than with bpermutes throughout.
__device__ __forceinline__ uint32_t shfl_xor(uint32_t v, int d) {
  const int i = static_cast<int>(v);
  if (d == 1) return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));
  if (d == 2) return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));
  // swizzle offset, bit mode: and-mask 0x1F, or-mask 0, xor-mask d
  if (d == 4) return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(i, 0x1F | (4 << 10)));
  if (d == 8) return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(i, 0x1F | (8 << 10)));
  if (d == 16) return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(i, 0x1F | (16 << 10)));
  return static_cast<uint32_t>(__shfl_xor(i, d, 64));
}
__device__ __forceinline__ float shfl_xor(float v, int d) { return __uint_as_float(shfl_xor(__float_as_uint(v), d)); }

template <int BITS>
__device__ __forceinline__ void append_encode_wave(const KvAppendArgs& a, uint32_t bhi, int64_t o, uint2 w, int lane) {
  constexpr int K = 1 << BITS;
  constexpr float thr3[7] = HLWQ_THRESHOLDS_3;
  constexpr float thr2[3] = HLWQ_THRESHOLDS_2;
  float x[4] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  // norm: level 0 (two fused pairs) and level 1 in the lane, levels 2..7 across lanes
  float s = __builtin_fmaf(x[0], x[0], x[1] * x[1]) + __builtin_fmaf(x[2], x[2], x[3] * x[3]);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) s = s + shfl_xor(s, d);
  const NormInfo ni = norm_info(s);
  // butterflies at strides 1 and 2 in the lane, 4 .. 128 across lanes
  {
    const float a0 = x[0] + x[1], a1 = x[0] - x[1], a2 = x[2] + x[3], a3 = x[2] - x[3];
    x[0] = a0 + a2;
    x[2] = a0 - a2;
    x[1] = a1 + a3;
    x[3] = a1 - a3;
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float q = shfl_xor(x[j], d);
      x[j] = upper ? q - x[j] : x[j] + q;
    }
  }
  // codes: the number of thresholds strictly below y
  uint32_t f = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float y = x[j] * ni.r;
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < K - 1; ++k) c += (y > (BITS == 3 ? thr3[k] : thr2[k])) ? 1u : 0u;
    f |= c << (BITS * j);
  }
  constexpr uint32_t kVec = 32 * BITS;
  const int64_t vec = static_cast<int64_t>(bhi) * a.capacity + o;
  uint8_t* dst = a.packed + vec * kVec;
  if constexpr (BITS == 2) {
    dst[lane] = static_cast<uint8_t>(f);  // 4 codes of 2 bits: one byte per lane
  } else {
    // 8 lanes hold 32 codes = 96 bits = 3 words: place the lane's 12 bits at
    // bit 12 i of its group's string and or the group together
    const int i = lane & 7;
    const int bit = 12 * i;
    const uint64_t v = static_cast<uint64_t>(f) << (bit & 31);
    uint32_t wd[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
      wd[k] = ((bit >> 5) == k ? static_cast<uint32_t>(v) : 0u) | ((bit >> 5) + 1 == k ? static_cast<uint32_t>(v >> 32) : 0u);
#pragma unroll
    for (int d = 1; d < 8; d <<= 1)
#pragma unroll
      for (int k = 0; k < 3; ++k) wd[k] |= shfl_xor(wd[k], d);
    if (i == 0) {
      uint32_t* out = reinterpret_cast<uint32_t*>(dst + 12 * (lane >> 3));
      out[0] = wd[0];
      out[1] = wd[1];
      out[2] = wd[2];
    }
  }
  if (lane == 0) a.norms[vec] = ni.n16;
}

template <int BITS>
__global__ void __launch_bounds__(64) hlwq_kv_append_small_kernel(const KvAppendArgs a) {
  const int lane = threadIdx.x;
  const uint32_t bhi = blockIdx.x;
  const int64_t total = a.tokens + a.n_new;
  const int64_t leave_end = total - a.n_res;
  const int64_t leave_begin = a.tokens > a.n_res ? a.tokens - a.n_res : 0;
  const uint2* src = reinterpret_cast<const uint2*>(a.src + static_cast<int64_t>(bhi) * a.n_new * kKvDim);
  // the new tokens that stay in the window: t in [max(tokens, total - n_res), total)
  const int64_t t0 = leave_end > a.tokens ? leave_end : a.tokens;
  const int nstay = static_cast<int>(total - t0);
  uint2 stay[kSmallAppend];
#pragma unroll
  for (int k = 0; k < kSmallAppend; ++k)
    if (k < nstay) stay[k] = src[(t0 + k - a.tokens) * (kKvDim / 4) + lane];
  for (int64_t o = leave_begin; o < leave_end; ++o) {
    const uint2* p = o < a.tokens
                         ? reinterpret_cast<const uint2*>(a.ring + (static_cast<int64_t>(bhi) * a.n_res + o % a.n_res) * kKvDim)
                         : src + (o - a.tokens) * (kKvDim / 4);
    append_encode_wave<BITS>(a, bhi, o, p[lane], lane);
  }
  // every ring read above has returned before any slot is rewritten
  wait_vmem();
  uint2* ring = reinterpret_cast<uint2*>(a.ring + static_cast<int64_t>(bhi) * a.n_res * kKvDim);
#pragma unroll
  for (int k = 0; k < kSmallAppend; ++k)
    if (k < nstay) ring[((t0 + k) % a.n_res) * (kKvDim / 4) + lane] = stay[k];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One buffer of a call: the bytes [lo, hi) of `count` items of `unit` bytes
// at p, and whether the call writes it (a size past the address space counts
// as reaching its end).
struct Span {
  uintptr_t lo, hi;
  bool written;
};
void add_span(std::vector<Span>& v, const void* p, int64_t count, int64_t unit, bool written) {
  int64_t bytes;
  if (!p || count <= 0) return;
  if (!mul_ok(count, unit, &bytes)) bytes = INT64_MAX;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  uintptr_t hi;
  if (__builtin_add_overflow(lo, static_cast<uintptr_t>(bytes), &hi)) hi = UINTPTR_MAX;
  v.push_back(Span{lo, hi, written});
}

// HLWQ_ERR_OVERLAP if a buffer the call writes shares a byte with any other
// buffer of the call; buffers it only reads may overlap each other.  Sorted by
// start, a span overlaps an earlier one exactly when it starts before that
// one's end, so one pass with the running ends of all spans and of the
// written ones decides.
int check_disjoint(std::vector<Span>& v) {
  std::sort(v.begin(), v.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  uintptr_t end_any = 0, end_written = 0;
  for (const Span& x : v) {
    if (x.lo < end_written || (x.written && x.lo < end_any)) return HLWQ_ERR_OVERLAP;
    end_any = std::max(end_any, x.hi);
    if (x.written) end_written = std::max(end_written, x.hi);
  }
  return HLWQ_OK;
}

template <typename T>
struct same_type {
  using type = T;
};

// Launch a kernel and return the status of this launch itself (the runtime's
// "last error" may hold an error some earlier, unrelated call left pending;
// it is neither reported as ours nor cleared).  The arguments take the
// kernel's own parameter types.
template <typename... P>
int launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, typename same_type<P>::type... args) {
  void* params[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, 0, stream) == hipSuccess
             ? HLWQ_OK
             : HLWQ_ERR_DEVICE;
}

// Validate one weight descriptor; *blocks = rows * nb (0 means nothing to do).
// norm_bytes: 2 (fp16 norms) or 4 (TQ3's fp32 norms).
int check_weight_desc(const hlwq_mat_desc& m, int64_t* blocks, int norm_bytes = 2) {
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
  if ((reinterpret_cast<uintptr_t>(m.packed) & 15u) ||
      (reinterpret_cast<uintptr_t>(m.norms) & static_cast<uintptr_t>(norm_bytes - 1)) ||
      (reinterpret_cast<uintptr_t>(m.w) & 1u))
    return HLWQ_ERR_ALIGN;
  *blocks = nblk;
  return HLWQ_OK;
}

constexpr uint32_t kDequantChunk = 2 * kWaves;  // batches per dequantize workgroup
// Workgroups per launch: a dispatch's size in work-items is a 32-bit field.
constexpr int64_t kMaxDispatch = 0xffffffffll / kThreads;

// Resident workgroups per launch: per_cu per CU (the weight quantizer's
// 8-wave workgroup uses ~131 KB of LDS, so one fits; the INT4 kernel's 4-wave
// workgroups ~41 KB, two; the KV quantizer's ~37 KB with ~110 VGPRs, four),
// at most one per `waves` batches; the workgroups loop over batches.
uint32_t persistent_grid(uint32_t batches, int per_cu = 2, int waves = kWaves) {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int n = dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
  }
  const uint64_t want = (static_cast<uint64_t>(batches) + waves - 1) / waves;
  const uint64_t cap = static_cast<uint64_t>(n) * per_cu;
  return static_cast<uint32_t>(want < cap ? want : cap);
}

// The 8 sign words of hlwq_tq3_signs: D1 in words 0-3, D2 in words 4-7.
void tq3_sign_words(uint64_t seed, uint32_t words[8]) {
  const TqSigns t = tq3_state(seed);
  for (int i = 0; i < 4; ++i) {
    words[i] = t.d1.w[i];
    words[4 + i] = t.d2.w[i];
  }
}

// field: bits per stored code (bits for packed codes, 8 for one code per byte);
// tq: TQ3's quantizer state (bits 3, packed codes, fp32 norms), or NULL for HLWQ.
template <bool QUANT>
int run_weight_group(const hlwq_mat_desc* mats, int n, int bits, int field, hipStream_t stream,
                     const TqSigns* tq = nullptr) {
  if (n < 0) return HLWQ_ERR_SHAPE;
  if (n > 0 && !mats) return HLWQ_ERR_NULL;
  if (bits != 5 && bits != 3) return HLWQ_ERR_BITS;
  if (tq && (bits != 3 || field != 3)) return HLWQ_ERR_BITS;
  const int norm_bytes = tq ? 4 : 2;
  // validate everything before enqueuing anything
  std::vector<Span> spans;
  for (int i = 0; i < n; ++i) {
    int64_t b;
    const int st = check_weight_desc(mats[i], &b, norm_bytes);
    if (st != HLWQ_OK) return st;
    if (b == 0) continue;
    add_span(spans, mats[i].w, mats[i].rows * mats[i].in, 2, !QUANT);
    add_span(spans, mats[i].packed, b, 16 * field, QUANT);
    add_span(spans, mats[i].norms, b, norm_bytes, QUANT);
  }
  if (check_disjoint(spans) != HLWQ_OK) return HLWQ_ERR_OVERLAP;
  int i = 0;
  while (i < n) {
    WeightGroup g;
    std::memset(&g, 0, sizeof(g));
    if (tq) g.tq = *tq;
    int64_t batches = 0;
    for (; i < n && g.n < kMaxGroup; ++i) {
      int64_t nblk;
      check_weight_desc(mats[i], &nblk, norm_bytes);
      if (nblk == 0) continue;
      // a matrix has at most 2^25 batches, so a launch always takes its first one
      if (batches + ceil_div(nblk, 64) > kDequantChunk * kMaxDispatch) break;
      const int k = g.n++;
      g.batch_start[k] = static_cast<uint32_t>(batches);
      g.nblocks[k] = static_cast<uint32_t>(nblk);
      g.nb[k] = static_cast<uint32_t>(ceil_div(mats[i].in, kBlock));
      g.in[k] = mats[i].in;
      g.w[k] = static_cast<uint16_t*>(mats[i].w);
      g.packed[k] = static_cast<uint8_t*>(mats[i].packed);
      g.norms[k] = mats[i].norms;
      g.staged[k] = (mats[i].in % 8 == 0) && ((reinterpret_cast<uintptr_t>(mats[i].w) & 15u) == 0);
      g.whole[k] = g.staged[k] && (mats[i].in % kBlock == 0);
      batches += ceil_div(nblk, 64);
    }
    if (g.n == 0) continue;
    g.batch_start[g.n] = static_cast<uint32_t>(batches);
    g.total_batches = static_cast<uint32_t>(batches);
    // quantize: one 8-wave workgroup per CU drawing batches from its work
    // pool (5-7% faster on the MoE banks than a fixed share per wave);
    // dequantize: workgroups of two batches per wave, handed out by the
    // hardware as earlier ones finish (6-7% faster than a persistent grid, and
    // 3% faster than the work pool)
    g.chunk = QUANT ? 0u : kDequantChunk;
    const dim3 grid(QUANT ? persistent_grid(g.total_batches, 1, kPoolWaves)
                          : (g.total_batches + kDequantChunk - 1) / kDequantChunk),
        block(QUANT ? kPoolThreads : kThreads);
    const bool bytes = field == 8;
    int st;
    if (tq) {
      // the recorded seed runs the kernels with the signs compiled in
      const bool seed42 = std::memcmp(tq, &kTq3Seed42, sizeof(TqSigns)) == 0;
      if (QUANT)
        st = launch(seed42 ? hlwq_quantize_kernel<3, 3, 2> : hlwq_quantize_kernel<3, 3, 1>, grid, block, stream, g);
      else
        st = launch(seed42 ? hlwq_dequantize_kernel<3, 3, 2> : hlwq_dequantize_kernel<3, 3, 1>, grid, block, stream, g);
    } else if (QUANT) {
      if (bits == 5) st = launch(bytes ? hlwq_quantize_kernel<5, 8> : hlwq_quantize_kernel<5, 5>, grid, block, stream, g);
      else st = launch(bytes ? hlwq_quantize_kernel<3, 8> : hlwq_quantize_kernel<3, 3>, grid, block, stream, g);
    } else {
      if (bits == 5) st = launch(bytes ? hlwq_dequantize_kernel<5, 8> : hlwq_dequantize_kernel<5, 5>, grid, block, stream, g);
      else st = launch(bytes ? hlwq_dequantize_kernel<3, 8> : hlwq_dequantize_kernel<3, 3>, grid, block, stream, g);
    }
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

// Launch the KV quantize or dequantize kernel over bh heads of `a` (a.tq
// tokens each, a.tokens kv rows and a.out_stride packed rows per head), whole
// heads per launch, at most kMaxDispatch workgroups' worth of batches each.
int launch_kv(bool quant, int bits, KvArgs a, int64_t bh, hipStream_t stream) {
  a.nbt = static_cast<uint32_t>(ceil_div(a.tq, kKvTokens));
  if (a.nbt == 0 || bh == 0) return HLWQ_OK;
  a.nbt_div = make_udiv(a.nbt);
  // quantize: one 16-wave workgroup per CU drawing from its work pool (5%
  // faster than a fixed share per wave on a 2 x 4-head cache of 32768
  // tokens); dequantize: one batch per wave, workgroups handed out by the
  // hardware (12-15% faster than a persistent grid)
  a.chunk = quant ? 0u : static_cast<uint32_t>(kWaves);
  const int64_t max_batches = static_cast<int64_t>(kWaves) * kMaxDispatch;
  if (a.nbt > max_batches) return HLWQ_ERR_LIMIT;
  const int64_t heads_per_launch = max_batches / a.nbt;
  const int64_t vec_bytes = 32 * bits;
  for (int64_t h0 = 0; h0 < bh; h0 += heads_per_launch) {
    const int64_t nh = bh - h0 < heads_per_launch ? bh - h0 : heads_per_launch;
    KvArgs l = a;
    l.kv += h0 * a.tokens * kKvDim;
    l.packed += h0 * a.out_stride * vec_bytes;
    l.norms += h0 * a.out_stride;
    l.total_batches = static_cast<uint32_t>(nh * a.nbt);
    const dim3 grid(quant ? persistent_grid(l.total_batches, 1, kKvPoolWaves) : (l.total_batches + l.chunk - 1) / l.chunk),
        block(quant ? kKvPoolThreads : kThreads);
    const int st = quant ? launch(bits == 3 ? hlwq_kv_quantize_kernel<3> : hlwq_kv_quantize_kernel<2>, grid, block,
                                  stream, l)
                         : launch(bits == 3 ? hlwq_kv_dequantize_kernel<3> : hlwq_kv_dequantize_kernel<2>, grid, block,
                                  stream, l);
    if (st != HLWQ_OK) return st;
  }
  return HLWQ_OK;
}

int run_kv(bool quant, const void* kv, void* packed, void* norms, int64_t batch, int64_t heads, int64_t tokens,
           int head_dim, int bits, int64_t n_residual, hipStream_t stream) {
  if (head_dim != kKvDim) return HLWQ_ERR_BLOCK;
  if (bits != 3 && bits != 2) return HLWQ_ERR_BITS;
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
      (reinterpret_cast<uintptr_t>(kv) & 15u))
    return HLWQ_ERR_ALIGN;
  std::vector<Span> spans;
  add_span(spans, kv, bytes, 1, !quant);
  add_span(spans, packed, nvec, 32 * bits, quant);
  add_span(spans, norms, nvec, 2, quant);
  if (check_disjoint(spans) != HLWQ_OK) return HLWQ_ERR_OVERLAP;
  KvArgs a;
  a.kv = const_cast<uint16_t*>(static_cast<const uint16_t*>(kv));
  a.packed = static_cast<uint8_t*>(packed);
  a.norms = static_cast<uint16_t*>(norms);
  a.tokens = tokens;
  a.out_stride = tq;
  a.out_offset = 0;
  a.tq = static_cast<uint32_t>(tq);
  return launch_kv(quant, bits, a, bh, stream);
}

// Validate one INT4 descriptor; *blocks = rows * in / 128 (0: nothing to do).
int check_int4_desc(const hlwq_int4_desc& m, int64_t* blocks) {
  *blocks = 0;
  if (m.rows < 0 || m.in < 0 || m.in % kBlock) return HLWQ_ERR_SHAPE;
  int64_t nblk, bytes;
  if (!mul_ok(m.rows, m.in / kBlock, &nblk) || !mul_ok(nblk, 80, &bytes)) return HLWQ_ERR_SHAPE;
  if (nblk == 0) return HLWQ_OK;
  if (!m.packed || !m.norms || !m.q4 || !m.scales || !m.zeros) return HLWQ_ERR_NULL;
  if (nblk > 0x7fffffff - 64) return HLWQ_ERR_LIMIT;
  if ((reinterpret_cast<uintptr_t>(m.packed) & 15u) || (reinterpret_cast<uintptr_t>(m.norms) & 1u) ||
      (reinterpret_cast<uintptr_t>(m.q4) & 15u) || (reinterpret_cast<uintptr_t>(m.scales) & 3u))
    return HLWQ_ERR_ALIGN;
  *blocks = nblk;
  return HLWQ_OK;
}

int run_dequantize_int4(const hlwq_int4_desc* mats, int n, int bits, hipStream_t stream) {
  if (n < 0) return HLWQ_ERR_SHAPE;
  if (n > 0 && !mats) return HLWQ_ERR_NULL;
  if (bits != 5 && bits != 3) return HLWQ_ERR_BITS;
  std::vector<Span> spans;
  for (int i = 0; i < n; ++i) {  // validate everything before enqueuing anything
    int64_t b;
    const int st = check_int4_desc(mats[i], &b);
    if (st != HLWQ_OK) return st;
    if (b == 0) continue;
    add_span(spans, mats[i].packed, b, 16 * bits, false);
    add_span(spans, mats[i].norms, b, 2, false);
    add_span(spans, mats[i].q4, b, kBlock / 2, true);
    add_span(spans, mats[i].scales, b, 4, true);
    add_span(spans, mats[i].zeros, b, 1, true);
  }
  if (check_disjoint(spans) != HLWQ_OK) return HLWQ_ERR_OVERLAP;
  int i = 0;
  while (i < n) {
    Int4Group g;
    std::memset(&g, 0, sizeof(g));
    int64_t batches = 0;
    for (; i < n && g.n < kMaxGroup; ++i) {
      int64_t nblk;
      check_int4_desc(mats[i], &nblk);
      if (nblk == 0) continue;
      // a matrix has fewer than 2^25 batches, so a launch always takes its first one
      if (batches + ceil_div(nblk, 64) > 0xffffffffll) break;
      const int k = g.n++;
      g.batch_start[k] = static_cast<uint32_t>(batches);
      g.nblocks[k] = static_cast<uint32_t>(nblk);
      g.packed[k] = static_cast<const uint8_t*>(mats[i].packed);
      g.norms[k] = static_cast<const uint16_t*>(mats[i].norms);
      g.q4[k] = static_cast<uint8_t*>(mats[i].q4);
      g.scales[k] = static_cast<float*>(mats[i].scales);
      g.zeros[k] = static_cast<uint8_t*>(mats[i].zeros);
      batches += ceil_div(nblk, 64);
    }
    if (g.n == 0) continue;
    g.batch_start[g.n] = static_cast<uint32_t>(batches);
    g.total_batches = static_cast<uint32_t>(batches);
    const dim3 grid(persistent_grid(g.total_batches)), block_dim(kThreads);
    const int st = launch(bits == 5 ? hlwq_dequantize_int4_kernel<5> : hlwq_dequantize_int4_kernel<3>, grid,
                          block_dim, stream, g);
    if (st != HLWQ_OK) return st;
  }
  return HLWQ_OK;
}

int run_kv_append(const void* src, int64_t batch, int64_t heads, int64_t n_new, int64_t tokens, void* ring,
                  int64_t n_residual, void* packed, void* norms, int64_t capacity, int head_dim, int bits,
                  hipStream_t stream) {
  if (head_dim != kKvDim) return HLWQ_ERR_BLOCK;
  if (bits != 3 && bits != 2) return HLWQ_ERR_BITS;
  if (batch < 0 || heads < 0 || n_new < 0 || tokens < 0 || n_residual < 0 || capacity < 0) return HLWQ_ERR_SHAPE;
  int64_t bh, total;
  if (!mul_ok(batch, heads, &bh) || __builtin_add_overflow(tokens, n_new, &total)) return HLWQ_ERR_SHAPE;
  if (bh == 0 || n_new == 0) return HLWQ_OK;
  const int64_t leave_end = total - n_residual;                          // encoded tokens afterwards
  const int64_t leave_begin = tokens > n_residual ? tokens - n_residual : 0;  // encoded tokens before
  const bool encodes = leave_end > leave_begin;
  if (!src || (n_residual > 0 && !ring) || (encodes && (!packed || !norms))) return HLWQ_ERR_NULL;
  if (encodes && capacity < leave_end) return HLWQ_ERR_SHAPE;
  int64_t elems, bytes, vecs;
  if (!mul_ok(bh, n_new, &elems) || !mul_ok(elems, 2 * kKvDim, &bytes) || !mul_ok(bh, capacity, &vecs) ||
      !mul_ok(bh, n_residual, &elems))
    return HLWQ_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(ring) & 15u) ||
      (reinterpret_cast<uintptr_t>(packed) & 15u) || (reinterpret_cast<uintptr_t>(norms) & 1u))
    return HLWQ_ERR_ALIGN;
  // new tokens that arrive and leave within this call: rows tokens .. tokens + in_leaving - 1
  const int64_t in_leaving = n_new > n_residual ? n_new - n_residual : 0;
  if (bh > 0x3fffffff || in_leaving > 0x7fffffff) return HLWQ_ERR_LIMIT;
  // checked last, after the launch limits of either path below
  const auto overlap = [&]() {
    std::vector<Span> spans;
    add_span(spans, src, bytes, 1, false);
    if (n_residual > 0) add_span(spans, ring, elems, 2 * kKvDim, true);
    if (encodes) {
      add_span(spans, packed, vecs, 32 * bits, true);
      add_span(spans, norms, vecs, 2, true);
    }
    return check_disjoint(spans) != HLWQ_OK;
  };
  KvAppendArgs a;
  a.src = static_cast<const uint16_t*>(src);
  a.ring = static_cast<uint16_t*>(ring);
  a.packed = static_cast<uint8_t*>(packed);
  a.norms = static_cast<uint16_t*>(norms);
  a.tokens = tokens;
  a.n_new = n_new;
  a.n_res = n_residual;
  a.capacity = capacity;
  a.bh = static_cast<uint32_t>(bh);
  if (n_new <= kSmallAppend) {
    // latency path: one wave per head
    if (bh > kMaxDispatch * kThreads / 64) return HLWQ_ERR_LIMIT;
    if (overlap()) return HLWQ_ERR_OVERLAP;
    return launch(bits == 3 ? hlwq_kv_append_small_kernel<3> : hlwq_kv_append_small_kernel<2>,
                  dim3(static_cast<uint32_t>(bh)), dim3(64), stream, a);
  }
  // everything is checked before the first launch
  const int64_t staying = n_new < n_residual ? n_new : n_residual;  // new tokens that stay in the window
  const int64_t fill_groups = ceil_div(bh * staying * (kKvDim / 8), kThreads);
  if (ceil_div(bh, kWaves) > kMaxDispatch || fill_groups > kMaxDispatch ||
      ceil_div(in_leaving, kKvTokens) > static_cast<int64_t>(kWaves) * kMaxDispatch)
    return HLWQ_ERR_LIMIT;
  if (overlap()) return HLWQ_ERR_OVERLAP;
  if (in_leaving > 0) {
    // the streaming path's bulk (a prefill, say): the KV quantize kernel,
    // reading the new tokens and writing cache rows tokens .. leave_end - 1
    KvArgs k;
    k.kv = const_cast<uint16_t*>(a.src);
    k.packed = a.packed;
    k.norms = a.norms;
    k.tokens = n_new;
    k.out_stride = capacity;
    k.out_offset = tokens;
    k.tq = static_cast<uint32_t>(in_leaving);
    const int st = launch_kv(true, bits, k, bh, stream);
    if (st != HLWQ_OK) return st;
  }
  if (n_residual == 0) return HLWQ_OK;
  if (leave_begin < (leave_end < tokens ? leave_end : tokens)) {
    // ring tokens leave: one wave per head encodes them
    const dim3 grid(static_cast<uint32_t>(ceil_div(bh, kWaves))), block(kThreads);
    const int st = launch(bits == 3 ? hlwq_kv_append_kernel<3> : hlwq_kv_append_kernel<2>, grid, block, stream, a);
    if (st != HLWQ_OK) return st;
  }
  // then the new tokens that stay are written into the ring
  const int64_t t0 = leave_end > tokens ? leave_end : tokens;
  const int64_t ntok = total - t0;
  return launch(hlwq_kv_ring_fill_kernel, dim3(static_cast<uint32_t>(fill_groups)), dim3(kThreads), stream, a, t0, ntok,
                t0 % n_residual);
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
  return run_weight_group<true>(&m, 1, bits, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_dequantize(const void* packed_u8, const void* norms_f16, int64_t n_mats, int64_t out, int64_t in,
                    int block, int bits, void* w_bf16_out, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16_out, packed_u8, norms_f16, n_mats, out, in, block, bits, &m);
  if (st != HLWQ_OK) return st;
  return run_weight_group<false>(&m, 1, bits, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_quantize_grouped(const hlwq_mat_desc* mats, int n, int bits, void* hip_stream) {
  return run_weight_group<true>(mats, n, bits, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_dequantize_grouped(const hlwq_mat_desc* mats, int n, int bits, void* hip_stream) {
  return run_weight_group<false>(mats, n, bits, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_quantize_codes8(const void* w_bf16, int64_t n_mats, int64_t out, int64_t in, int block, int bits,
                         void* codes_u8, void* norms_f16, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16, codes_u8, norms_f16, n_mats, out, in, block, bits, &m);
  if (st != HLWQ_OK) return st;
  return run_weight_group<true>(&m, 1, bits, 8, static_cast<hipStream_t>(hip_stream));
}

int hlwq_dequantize_codes8(const void* codes_u8, const void* norms_f16, int64_t n_mats, int64_t out, int64_t in,
                           int block, int bits, void* w_bf16_out, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16_out, codes_u8, norms_f16, n_mats, out, in, block, bits, &m);
  if (st != HLWQ_OK) return st;
  return run_weight_group<false>(&m, 1, bits, 8, static_cast<hipStream_t>(hip_stream));
}

int hlwq_tq3_signs(uint64_t seed, uint32_t* sign_words) {
  if (!sign_words) return HLWQ_ERR_NULL;
  tq3_sign_words(seed, sign_words);
  return HLWQ_OK;
}

int hlwq_tq3_quantize(const void* w_bf16, int64_t n_mats, int64_t out, int64_t in, int group, uint64_t seed,
                      void* packed_u8, void* norms_f32, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16, packed_u8, norms_f32, n_mats, out, in, group, 3, &m);
  if (st != HLWQ_OK) return st;
  const TqSigns tq = tq3_state(seed);
  return run_weight_group<true>(&m, 1, 3, 3, static_cast<hipStream_t>(hip_stream), &tq);
}

int hlwq_tq3_dequantize(const void* packed_u8, const void* norms_f32, int64_t n_mats, int64_t out, int64_t in,
                        int group, uint64_t seed, void* w_bf16_out, void* hip_stream) {
  hlwq_mat_desc m;
  const int st = make_single(w_bf16_out, packed_u8, norms_f32, n_mats, out, in, group, 3, &m);
  if (st != HLWQ_OK) return st;
  const TqSigns tq = tq3_state(seed);
  return run_weight_group<false>(&m, 1, 3, 3, static_cast<hipStream_t>(hip_stream), &tq);
}

int hlwq_tq3_quantize_grouped(const hlwq_mat_desc* mats, int n, uint64_t seed, void* hip_stream) {
  const TqSigns tq = tq3_state(seed);
  return run_weight_group<true>(mats, n, 3, 3, static_cast<hipStream_t>(hip_stream), &tq);
}

int hlwq_tq3_dequantize_grouped(const hlwq_mat_desc* mats, int n, uint64_t seed, void* hip_stream) {
  const TqSigns tq = tq3_state(seed);
  return run_weight_group<false>(mats, n, 3, 3, static_cast<hipStream_t>(hip_stream), &tq);
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

int hlwq_dequantize_int4(const void* packed_u8, const void* norms_f16, int64_t n_mats, int64_t out, int64_t in,
                         int block, int bits, void* q4_u8, void* scales_f32, void* zeros_u8, void* hip_stream) {
  if (block != kBlock) return HLWQ_ERR_BLOCK;
  if (bits != 5 && bits != 3) return HLWQ_ERR_BITS;
  if (n_mats < 0 || out < 0) return HLWQ_ERR_SHAPE;
  hlwq_int4_desc m;
  if (!mul_ok(n_mats, out, &m.rows)) return HLWQ_ERR_SHAPE;
  m.packed = packed_u8;
  m.norms = norms_f16;
  m.q4 = q4_u8;
  m.scales = scales_f32;
  m.zeros = zeros_u8;
  m.in = in;
  return run_dequantize_int4(&m, 1, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_dequantize_int4_grouped(const hlwq_int4_desc* mats, int n, int bits, void* hip_stream) {
  return run_dequantize_int4(mats, n, bits, static_cast<hipStream_t>(hip_stream));
}

int hlwq_kv_append(const void* new_kv_bf16, int64_t batch, int64_t heads, int64_t n_new, int64_t tokens,
                   void* window_bf16, int64_t n_residual, void* packed_u8, void* norms_f16, int64_t capacity,
                   int head_dim, int bits, void* hip_stream) {
  return run_kv_append(new_kv_bf16, batch, heads, n_new, tokens, window_bf16, n_residual, packed_u8, norms_f16,
                       capacity, head_dim, bits, static_cast<hipStream_t>(hip_stream));
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
  if (bits != 5 && bits != 3 && bits != 2) return HLWQ_ERR_BITS;
  const int K = 1 << bits;
  const float* c = bits == 5 ? h_cent5 : bits == 3 ? h_cent3 : h_cent2;
  const float* t = bits == 5 ? h_thr5 : bits == 3 ? h_thr3 : h_thr2;
  if (centroids) std::memcpy(centroids, c, sizeof(float) * K);
  if (thresholds) std::memcpy(thresholds, t, sizeof(float) * (K - 1));
  return HLWQ_OK;
}

int hlwq_search_table(int kind, uint8_t* buckets, int capacity, uint32_t* entries, float* scale,
                      uint32_t* bias_bits) {
  const uint32_t* bucket;
  const uint32_t* entry;
  int n, K;
  uint32_t bias;
  switch (kind) {
    case 0: bucket = h_bucket5; entry = h_entry5; n = HLWQ_BUCKETS; K = 32; bias = HLWQ_BUCKET_BIAS; break;
    case 1: bucket = h_bucket3; entry = h_entry3; n = HLWQ_BUCKETS; K = 8; bias = HLWQ_BUCKET_BIAS; break;
    case 2: bucket = h_kvbucket3; entry = h_entry3; n = HLWQ_KV_BUCKETS; K = 8; bias = HLWQ_KV_BUCKET_BIAS; break;
    case 3: bucket = h_kvbucket2; entry = h_entry2; n = HLWQ_KV_BUCKETS; K = 4; bias = HLWQ_KV_BUCKET_BIAS; break;
    default: return HLWQ_ERR_BITS;
  }
  if (buckets) {
    const int m = capacity < n ? capacity : n;
    if (m > 0) std::memcpy(buckets, bucket, static_cast<size_t>(m));
  }
  if (entries) std::memcpy(entries, entry, sizeof(uint32_t) * 2 * K);
  if (scale) *scale = HLWQ_SEARCH_SCALE;
  if (bias_bits) *bias_bits = bias;
  return n;
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
    case HLWQ_ERR_OVERLAP: return "a buffer the call writes overlaps another of its buffers";
    default: return "unknown status";
  }
}

}  // extern "C"
