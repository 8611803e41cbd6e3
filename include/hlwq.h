/*
 * hlwq.h — C ABI of libhlwq, the MI355X (gfx950) HLWQ quantize / dequantize
 * library (Hadamard-Lloyd Weight Quantization).
 *
 * The method (model card "Qwen3.6-35B-A3B — HLWQ Q5", section "Method",
 * steps [1]-[5]): view a weight matrix W (out x in) as (out, n_blocks, 128)
 * with the last block zero-padded; L2-normalise every block and keep its norm
 * as fp16 ("Gemma-4-26B-A4B-it-HLWQ-Q5", "Technical Details"); rotate each
 * block by the orthonormal 128x128 Walsh-Hadamard matrix scaled by sqrt(128);
 * replace every value by the index of the nearest of 2^bits Lloyd-Max
 * centroids for N(0, 1); pack 8 codes into `bits` bytes.  Dequantisation is
 * the inverse, written as bf16 ("Qwopus3.6-27B-v2 · HLWQ Q5", "Pipeline":
 * dequantize per Linear to BF16).  The KV-cache path ("Qwopus3.6-27B-v2 ·
 * HLWQ Q5", "Methodology notes", KV bullet) does the same per 256-wide head
 * vector with H256 and 8 centroids, and leaves the newest tokens unquantised.
 *
 * Arithmetic.  Every kernel follows one fixed IEEE-fp32 operation order, so
 * results are bit-identical run to run and device to device:
 *   norm   : squares summed by an adjacent-pair tree whose first level forms
 *            each pair as one fused multiply-add, RN(x0^2 + RN(x1^2)); then a
 *            correctly rounded sqrt, fp16 by round-to-nearest-even;
 *   rotate : unnormalised +-1 butterflies (a, b) -> (a + b, a - b) at strides
 *            1, 2, 4, ... (natural / Sylvester order), then y = z * (1 / n),
 *            1 / n correctly rounded, and 0 for blocks whose norm is below the
 *            smallest normal fp32 value (so a zero block gives y = 0);
 *   code   : number of fp32 decision thresholds strictly below y, i.e. the
 *            nearest fp32 centroid with ties to the lower index;
 *   inverse: the same butterflies on the centroids, times n16 / L (L = 128 or
 *            256, exact in fp32), rounded to bf16 nearest-even.
 *
 * Layouts (all row-major, contiguous, little-endian):
 *   W        bf16 [n_mats][out][in]
 *   packed   u8   [n_mats][out][nb][16 * bits], nb = ceil(in / 128); within a
 *                 block, group g of 8 codes (positions 8g .. 8g+7) is the
 *                 little-endian integer sum_i code_i << (bits * i) stored in
 *                 bytes [g * bits, g * bits + bits)
 *   norms    fp16 [n_mats][out][nb]
 *   KV       bf16 [batch][heads][tokens][256]; packed u8 [batch][heads][tq][32 * bits]
 *            and norms fp16 [batch][heads][tq] with tq = max(tokens - n_residual, 0)
 *
 * Ownership and execution: the caller allocates every buffer, in device
 * memory of the current HIP device.  The library keeps no state beyond
 * constant tables compiled into the code object and each device's compute-unit
 * count (read once, kept in an atomic), and allocates no device memory.
 * Every call validates its arguments on the host first; on success it enqueues the
 * work on `hip_stream` (a hipStream_t; NULL means the default stream) and
 * returns without synchronising.  Calls are reentrant; calls on different
 * streams may run concurrently.
 *
 * Errors: every int-returning call returns HLWQ_OK (0) or a negative
 * HLWQ_ERR_* status.  On an argument error nothing is enqueued and output
 * buffers are left untouched; HLWQ_ERR_DEVICE (a launch the runtime refused)
 * can come after earlier launches of the same call, whose outputs are then
 * partly written.  Zero-sized work (n_mats, out, in, batch, heads or the quantised
 * token count equal to 0) is valid, does nothing and accepts NULL pointers.
 * Inputs must be finite; a block whose squared norm overflows fp32 (an entry
 * above ~1.8e19 in magnitude) yields an infinite norm and unspecified codes.
 *
 * Overlap: a buffer a call writes may share no byte with any other buffer of
 * the same call (every buffer taken at its whole extent, e.g. the full
 * [B, H, T, 256] KV tensor even where only rows t < T - n_residual are
 * written); such a call returns HLWQ_ERR_OVERLAP.  Buffers a call only reads
 * may overlap each other.  Calls in flight on different streams are not
 * checked against each other.
 *
 * Alignment: `packed` and KV-cache buffers must be 16-byte aligned, `norms`
 * and weight buffers 2-byte aligned.  Weight matrices whose rows do not all
 * start 16-byte aligned (in % 8 != 0, or an unaligned W) are handled, on a
 * slower element-wise path.
 */
#ifndef HLWQ_H
#define HLWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HLWQ_OK = 0,
  HLWQ_ERR_NULL = -1,    /* a required pointer is NULL */
  HLWQ_ERR_SHAPE = -2,   /* negative size, a size whose byte count overflows int64, or too small a capacity */
  HLWQ_ERR_BITS = -3,    /* bits not supported for this call */
  HLWQ_ERR_BLOCK = -4,   /* block != 128 (weights) or head_dim != 256 (KV) */
  HLWQ_ERR_DEVICE = -5,  /* the HIP launch reported an error */
  HLWQ_ERR_ALIGN = -6,   /* a buffer violates the alignment stated above */
  HLWQ_ERR_LIMIT = -7,   /* more than 2^31 - 1 blocks / vectors in one matrix or cache, or an append
                            whose launch would exceed 2^32 - 1 work-items (about 6.7e7 heads) */
  HLWQ_ERR_OVERLAP = -8  /* a buffer the call writes overlaps another buffer of the call */
};

/* One matrix of a grouped call.  For hlwq_quantize_grouped `w` is read and
 * `packed` / `norms` are written; for hlwq_dequantize_grouped `packed` /
 * `norms` are read and `w` is written.  `rows` = n_mats * out of that matrix
 * (an expert bank [E][out][in] is one descriptor with rows = E * out). */
typedef struct hlwq_mat_desc {
  void* w;        /* bf16 [rows][in] */
  void* packed;   /* u8   [rows][nb][16 * bits] */
  void* norms;    /* fp16 [rows][nb] */
  int64_t rows;
  int64_t in;
} hlwq_mat_desc;

/* Quantize W [n_mats][out][in] (bf16) with HLWQ, block = 128, bits = 5 (32
 * centroids, Q5) or 3 (8 centroids, Q3): steps [1]-[5] of "Qwen3.6-35B-A3B —
 * HLWQ Q5", section "Method".  Writes packed [n_mats][out][nb][16*bits] and
 * fp16 norms [n_mats][out][nb].  The zero-padded tail block of every row is
 * encoded in full (all 128 codes are stored). */
int hlwq_quantize(const void* w_bf16, int64_t n_mats, int64_t out, int64_t in,
                  int block, int bits, void* packed_u8, void* norms_f16,
                  void* hip_stream);

/* Inverse of hlwq_quantize: unpack, centroid lookup, inverse rotation, scale
 * by the fp16 norm, round to bf16; writes only the `in` real columns of every
 * row of W_out [n_mats][out][in]. */
int hlwq_dequantize(const void* packed_u8, const void* norms_f16, int64_t n_mats,
                    int64_t out, int64_t in, int block, int bits,
                    void* w_bf16_out, void* hip_stream);

/* The same quantisation with the codes stored one per byte instead of packed
 * ("Gemma-4-26B-A4B-it-HLWQ-Q5", "Technical Details": int8 codes and fp16
 * norms): codes_u8 [n_mats][out][nb][128], code j of a block in byte j (the
 * zero-padded tail of a row's last block included).  bits 5 or 3. */
int hlwq_quantize_codes8(const void* w_bf16, int64_t n_mats, int64_t out, int64_t in, int block, int bits,
                         void* codes_u8, void* norms_f16, void* hip_stream);

/* Inverse of hlwq_quantize_codes8.  Only the low `bits` bits of each code byte
 * are read. */
int hlwq_dequantize_codes8(const void* codes_u8, const void* norms_f16, int64_t n_mats, int64_t out, int64_t in,
                           int block, int bits, void* w_bf16_out, void* hip_stream);

/* TQ3, the scalar case of HIGGS ("Qwen3.6-35B-A3B-TQ3-native", section "What
 * TQ3 actually does"; stored tensors and quantizer state in section "Files").
 * Per group of 128 consecutive values of a row (the last group zero-padded):
 *   rotate  : y = D2 H D1 x * (1 / n), n the group's norm, H the unnormalised
 *             Walsh-Hadamard butterflies, D1 and D2 diagonal +-1 sign vectors
 *             drawn from `seed` (see hlwq_tq3_signs);
 *   code    : nearest of the 8 Lloyd-Max centroids for N(0, 1), as hlwq Q3;
 *   norm    : the shape-gain n / (rho / sqrt(128)), rho the norm of the
 *             selected centroids, stored as fp32;
 *   inverse : bf16 of D1 H D2 c[codes] * (norm / 128).
 * Fixed fp32 operation order, shared with the HLWQ kernels where the steps
 * coincide: the norm tree, 1 / n and the butterflies as above, y's sign flip
 * after the rounding of z * (1 / n); rho^2 is the exact sum of the 128
 * RN(c^2) of the selected centroids, rounded once to fp32 (each RN(c^2) is a
 * multiple of 2^-28 and the sum is below 2^10, so the sum itself is exact),
 * rho and n / t correctly rounded,
 * t = RN(rho * RN(1 / sqrt(128))); the inverse multiplies by RN(norm * 2^-7)
 * and flips D1's signs after rounding.  Layouts: packed u8
 * [n_mats][out][ng][48] in the 3-bit packing above (ng = ceil(in / 128)),
 * norms fp32 [n_mats][out][ng] (4-byte aligned).  `group` must be 128.  The
 * page records the seed (42) but not its generator, so codes are bit-identical
 * to this library's oracle, not to checkpoints made by other tools. */

/* The two sign vectors for `seed`: SplitMix64 (Steele, Lea & Flood, OOPSLA
 * 2014) output i, i = 0 .. 255, has its top bit set when entry i of D1
 * (i < 128) or entry i - 128 of D2 is -1.  Writes 8 words to the host array
 * sign_words: bit i % 32 of word i / 32 for entry i of D1 (words 0-3) and of
 * D2 (words 4-7).  Host only; returns HLWQ_OK or HLWQ_ERR_NULL. */
int hlwq_tq3_signs(uint64_t seed, uint32_t* sign_words);

/* TQ3-quantize W [n_mats][out][in] (bf16): packed u8 [n_mats][out][ng][48] and
 * fp32 shape-gain norms [n_mats][out][ng]. */
int hlwq_tq3_quantize(const void* w_bf16, int64_t n_mats, int64_t out, int64_t in, int group, uint64_t seed,
                      void* packed_u8, void* norms_f32, void* hip_stream);

/* Inverse of hlwq_tq3_quantize; writes only the `in` real columns of each row. */
int hlwq_tq3_dequantize(const void* packed_u8, const void* norms_f32, int64_t n_mats, int64_t out, int64_t in,
                        int group, uint64_t seed, void* w_bf16_out, void* hip_stream);

/* Grouped forms, as hlwq_quantize_grouped / hlwq_dequantize_grouped: the
 * descriptors' `norms` point to fp32 norms. */
int hlwq_tq3_quantize_grouped(const hlwq_mat_desc* mats, int n, uint64_t seed, void* hip_stream);
int hlwq_tq3_dequantize_grouped(const hlwq_mat_desc* mats, int n, uint64_t seed, void* hip_stream);

/* Quantize several matrices (e.g. the gate_up and down banks of a MoE layer,
 * every expert of which is quantised independently: "Gemma-4-26B-A4B-it-HLWQ-Q5",
 * "Technical Details") in one launch.  `mats` is a host array of n
 * descriptors, read before the call returns; more than 16 descriptors, or
 * more blocks than one launch addresses (about 8.6e9), are split over several
 * launches.  bits = 5 or 3, block 128. */
int hlwq_quantize_grouped(const hlwq_mat_desc* mats, int n, int bits, void* hip_stream);

/* Inverse of hlwq_quantize_grouped over the same descriptors. */
int hlwq_dequantize_grouped(const hlwq_mat_desc* mats, int n, int bits, void* hip_stream);

/* Dequantize HLWQ codes straight to INT4 with one scale and zero point per
 * group of 128 consecutive columns of a row, the step that follows in the
 * pages' pipeline ("Qwopus3.6-27B-v2 · HLWQ Q5", "Pipeline": dequantize per
 * Linear to BF16, then 4-bit weight-only quantisation with group size 128 of
 * the 128-aligned Linears; "Qwen3.5-9B — HLWQ INT4", "Why HLWQ INT4 is
 * Better").  The group is the HLWQ block; `in` must be a multiple of 128.  The
 * bf16 values hlwq_dequantize would write are re-quantised in registers:
 * per group, in fp32, lo = min(0, min w), hi = max(0, max w),
 * scale = (hi - lo) / 15 (1 if that is 0), inv = 1 / scale,
 * zp = clamp(rint(-lo * inv), 0, 15), q = clamp(rint(w * inv) + zp, 0, 15)
 * (rint: nearest, ties to even); a weight dequantises to (q - zp) * scale.
 * Outputs: q4_u8 [n_mats][out][in / 2] (element 2i in the low nibble of byte
 * i), scales_f32 [n_mats][out][in / 128], zeros_u8 [n_mats][out][in / 128].
 * bits 5 or 3, block 128.  packed and q4 16-byte aligned, norms 2-byte and
 * scales 4-byte aligned. */
int hlwq_dequantize_int4(const void* packed_u8, const void* norms_f16, int64_t n_mats, int64_t out, int64_t in,
                         int block, int bits, void* q4_u8, void* scales_f32, void* zeros_u8, void* hip_stream);

/* One matrix of hlwq_dequantize_int4_grouped: `packed` / `norms` are read,
 * `q4` / `scales` / `zeros` written, with the layouts and alignment of
 * hlwq_dequantize_int4; `rows` = n_mats * out, `in` a multiple of 128. */
typedef struct hlwq_int4_desc {
  const void* packed;  /* u8   [rows][in / 128][16 * bits] */
  const void* norms;   /* fp16 [rows][in / 128] */
  void* q4;            /* u8   [rows][in / 2] */
  void* scales;        /* fp32 [rows][in / 128] */
  void* zeros;         /* u8   [rows][in / 128] */
  int64_t rows;
  int64_t in;
} hlwq_int4_desc;

/* hlwq_dequantize_int4 over several matrices (the Linears of a layer, say) in
 * one launch, as hlwq_dequantize_grouped does for bf16: `mats` is a host array
 * of n descriptors, read before the call returns; more than 16 descriptors are
 * split over several launches.  bits 5 or 3; every descriptor is validated
 * before anything is enqueued. */
int hlwq_dequantize_int4_grouped(const hlwq_int4_desc* mats, int n, int bits, void* hip_stream);

/* Quantize a KV cache [batch][heads][tokens][head_dim] (bf16) per head
 * vector: H256 rotation, 8 Lloyd-Max centroids, 3-bit codes ("Qwopus3.6-27B-v2
 * · HLWQ Q5", "Methodology notes", KV bullet), or with bits = 2 the 4-centroid
 * variant ("Qwen3.6-35B-A3B — HLWQ Q5", "Speed Benchmarks": Q3 and Q2 KV).
 * head_dim must be 256 and bits 3 or 2.  Tokens t < tokens - n_residual are
 * encoded into packed [batch][heads][tq][32 * bits] and norms
 * [batch][heads][tq]; the newest n_residual tokens (the unquantised residual
 * window, 128 on that card) are not read. */
int hlwq_kv_quantize(const void* kv_bf16, int64_t batch, int64_t heads, int64_t tokens,
                     int head_dim, int bits, int64_t n_residual,
                     void* packed_u8, void* norms_f16, void* hip_stream);

/* Inverse of hlwq_kv_quantize: writes tokens t < tokens - n_residual of
 * kv_out [batch][heads][tokens][head_dim]; the residual rows of kv_out are
 * not touched (the caller keeps its bf16 residual tokens there). */
int hlwq_kv_dequantize(const void* packed_u8, const void* norms_f16, int64_t batch,
                       int64_t heads, int64_t tokens, int head_dim, int bits,
                       int64_t n_residual, void* kv_bf16_out, void* hip_stream);

/* Append n_new tokens new_kv [batch][heads][n_new][head_dim] (bf16) to a
 * streaming KV cache that holds `tokens` tokens, as a generation loop does
 * ("Qwopus3.6-27B-v2 · HLWQ Q5", "Methodology notes", KV bullet: recent
 * tokens stay unquantised in a residual buffer; "Qwen3.6-35B-A3B — HLWQ Q5",
 * "Speed Benchmarks": Q3 / Q2 KV in a manual generation loop).  The cache:
 *   window  bf16 [batch][heads][n_residual][head_dim], a ring: token t sits in
 *           slot t mod n_residual while it is one of the newest n_residual;
 *   packed  u8   [batch][heads][capacity][32 * bits] and
 *   norms   fp16 [batch][heads][capacity]: token t's codes and norm at index t
 *           once it has left the window.
 * Afterwards tokens [0, tokens + n_new - n_residual) are encoded (exactly as
 * hlwq_kv_quantize encodes them) and the newest min(tokens + n_new,
 * n_residual) tokens are in the window; the call writes only the codes of the
 * tokens that leave the window during it and the ring slots of the new tokens
 * that stay.  head_dim 256, bits 3 or 2.  capacity must be at least
 * tokens + n_new - n_residual whenever a token leaves the window; window may
 * be NULL when n_residual = 0.  new_kv, window and packed must be 16-byte
 * aligned.  n_new = 0 or batch * heads = 0 does nothing. */
int hlwq_kv_append(const void* new_kv_bf16, int64_t batch, int64_t heads, int64_t n_new, int64_t tokens,
                   void* window_bf16, int64_t n_residual, void* packed_u8, void* norms_f16, int64_t capacity,
                   int head_dim, int bits, void* hip_stream);

/* Bytes of packed codes for `rows` rows of `in` columns: rows * nb * block * bits / 8.
 * Returns 0 for invalid arguments. */
size_t hlwq_packed_bytes(int64_t rows, int64_t in, int block, int bits);

/* Number of fp16 norms for `rows` rows of `in` columns: rows * nb.  0 if invalid. */
size_t hlwq_norm_count(int64_t rows, int64_t in, int block);

/* Copy the fp32 codebook the kernels use: 2^bits centroids (ascending) and
 * 2^bits - 1 decision thresholds.  bits = 5, 3 or 2.  Host-only, no GPU needed. */
int hlwq_centroids(int bits, float* centroids, float* thresholds);

/* Copy the two tables the kernels use to find a code with one compare.  For
 * a rotated value y the kernels form u = fma(y, scale, bias) in fp32, with
 * scale = 2^-146 and bias the denormal whose bit pattern is `bias_bits`; for
 * every value a finite input can produce, u is a denormal, so its bit pattern
 * k = RN(8 y) + bias_bits indexes the bucket table.  Byte k of that table is 8
 * times the number of thresholds below the 1/8-wide bucket k; at that byte
 * offset the entry table holds {fp32 bits of threshold b (+inf for the last),
 * b}, and the code is b + (y > threshold b).  kind 0: Q5 weights, 1: Q3
 * weights, 2: Q3 KV, 3: Q2 KV.  Copies at most `capacity` bucket bytes into `buckets`
 * and the 2 * 2^bits entry words into `entries` (either may be NULL), stores
 * scale and bias_bits, and returns the bucket count, or a negative status.
 * Host-only; exposed so the tables can be verified. */
int hlwq_search_table(int kind, uint8_t* buckets, int capacity, uint32_t* entries, float* scale,
                      uint32_t* bias_bits);

/* Static, human-readable text for a status code. */
const char* hlwq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* HLWQ_H */
