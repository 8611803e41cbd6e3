/* Plain C client of libhlwq: compiles against include/hlwq.h with a C
 * compiler and exercises the host-only entry points and the argument checks
 * of the device entry points (no kernel is launched).  Exit status 0 on
 * success; prints the first failed check otherwise. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "hlwq.h"

#define CHECK(cond)                                          \
  do {                                                       \
    if (!(cond)) {                                           \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                              \
    }                                                        \
  } while (0)

int main(void) {
  float c[32], t[31];
  uint32_t signs[8];
  char buf[16];
  hlwq_mat_desc d;
  /* sizes: 80 B of codes and one norm per 128-block of a Q5 row */
  CHECK(hlwq_packed_bytes(4, 256, 128, 5) == 4u * 2u * 80u);
  CHECK(hlwq_packed_bytes(1, 129, 128, 3) == 2u * 48u);
  CHECK(hlwq_norm_count(3, 704, 128) == 18u);
  /* codebooks: ascending, symmetric, thresholds between neighbours */
  CHECK(hlwq_centroids(5, c, t) == HLWQ_OK);
  CHECK(c[0] < c[1] && c[31] == -c[0] && t[15] == 0.0f && c[15] < t[15] && t[15] < c[16]);
  CHECK(hlwq_centroids(4, c, t) == HLWQ_ERR_BITS);
  /* TQ3 signs: deterministic, and different for another seed */
  CHECK(hlwq_tq3_signs(42, signs) == HLWQ_OK);
  memcpy(buf, signs, sizeof(buf));
  CHECK(hlwq_tq3_signs(42, signs) == HLWQ_OK && memcmp(buf, signs, sizeof(buf)) == 0);
  CHECK(hlwq_tq3_signs(43, signs) == HLWQ_OK && memcmp(buf, signs, sizeof(buf)) != 0);
  CHECK(hlwq_tq3_signs(42, NULL) == HLWQ_ERR_NULL);
  /* device entry points reject bad arguments before touching a device */
  CHECK(hlwq_quantize(NULL, 1, 4, 128, 128, 5, buf, buf, NULL) == HLWQ_ERR_NULL);
  CHECK(hlwq_quantize(buf, 1, 4, 128, 64, 5, buf, buf, NULL) == HLWQ_ERR_BLOCK);
  CHECK(hlwq_dequantize(buf, buf, 1, -4, 128, 128, 5, buf, NULL) == HLWQ_ERR_SHAPE);
  CHECK(hlwq_kv_quantize(buf, 1, 4, 300, 128, 3, 128, buf, buf, NULL) == HLWQ_ERR_BLOCK);
  CHECK(hlwq_quantize(NULL, 0, 4, 128, 128, 5, NULL, NULL, NULL) == HLWQ_OK); /* empty work */
  d.w = NULL;
  d.packed = NULL;
  d.norms = NULL;
  d.rows = 4;
  d.in = 128;
  CHECK(hlwq_quantize_grouped(&d, 1, 5, NULL) == HLWQ_ERR_NULL);
  CHECK(hlwq_tq3_quantize_grouped(&d, 1, 42, NULL) == HLWQ_ERR_NULL);
  CHECK(strlen(hlwq_status_string(HLWQ_ERR_ALIGN)) > 0);
  CHECK(strcmp(hlwq_status_string(-99), "unknown status") == 0);

  /* sizes whose byte counts overflow int64 are refused, not wrapped */
  CHECK(hlwq_packed_bytes(INT64_MAX, 1 << 20, 128, 5) == 0u);
  CHECK(hlwq_packed_bytes(4, 256, 100, 5) == 0u && hlwq_packed_bytes(4, 256, 128, 9) == 0u);
  CHECK(hlwq_norm_count(-1, 128, 128) == 0u && hlwq_norm_count(INT64_MAX, 1 << 30, 128) == 0u);
  CHECK(hlwq_quantize(buf, INT64_MAX, 2, 128, 128, 5, buf, buf, NULL) == HLWQ_ERR_SHAPE);
  CHECK(hlwq_quantize(buf, 1, -1, 128, 128, 5, buf, buf, NULL) == HLWQ_ERR_SHAPE);
  d.w = buf;
  d.packed = buf;
  d.norms = buf;
  d.rows = (int64_t)1 << 40;
  d.in = (int64_t)1 << 40;
  CHECK(hlwq_quantize_grouped(&d, 1, 5, NULL) == HLWQ_ERR_SHAPE);
  d.rows = (int64_t)1 << 32; /* 2^32 blocks: more than one matrix may hold */
  d.in = 128;
  CHECK(hlwq_quantize_grouped(&d, 1, 5, NULL) == HLWQ_ERR_LIMIT);
  CHECK(hlwq_dequantize_grouped(&d, 1, 3, NULL) == HLWQ_ERR_LIMIT);
  CHECK(hlwq_quantize_grouped(&d, -1, 5, NULL) == HLWQ_ERR_SHAPE);
  CHECK(hlwq_quantize_grouped(NULL, 1, 5, NULL) == HLWQ_ERR_NULL);
  CHECK(hlwq_quantize_grouped(&d, 1, 4, NULL) == HLWQ_ERR_BITS);
  /* misaligned code buffer */
  d.rows = 4;
  d.packed = buf + 1;
  CHECK(hlwq_quantize_grouped(&d, 1, 5, NULL) == HLWQ_ERR_ALIGN);
  CHECK(hlwq_quantize_codes8(buf, 1, 4, 128, 128, 5, buf + 1, buf, NULL) == HLWQ_ERR_ALIGN);
  CHECK(hlwq_dequantize_codes8(buf, buf, 1, 4, 128, 128, 2, buf, NULL) == HLWQ_ERR_BITS);
  /* TQ3: group 128 only, fp32 norms 4-byte aligned */
  CHECK(hlwq_tq3_quantize(buf, 1, 4, 128, 64, 42, buf, buf, NULL) == HLWQ_ERR_BLOCK);
  CHECK(hlwq_tq3_dequantize(buf, buf + 2, 1, 4, 128, 128, 42, buf, NULL) == HLWQ_ERR_ALIGN);
  /* dequantize to INT4: whole 128-column groups only */
  CHECK(hlwq_dequantize_int4(buf, buf, 1, 4, 200, 128, 5, buf, buf, buf, NULL) == HLWQ_ERR_SHAPE);
  CHECK(hlwq_dequantize_int4(NULL, buf, 1, 4, 256, 128, 5, buf, buf, buf, NULL) == HLWQ_ERR_NULL);
  CHECK(hlwq_dequantize_int4(buf, buf, 1, 4, 256, 128, 6, buf, buf, buf, NULL) == HLWQ_ERR_BITS);
  {
    hlwq_int4_desc q;
    q.packed = buf;
    q.norms = buf;
    q.q4 = buf;
    q.scales = buf;
    q.zeros = buf;
    q.rows = 4;
    q.in = 200;
    CHECK(hlwq_dequantize_int4_grouped(&q, 1, 5, NULL) == HLWQ_ERR_SHAPE);  /* in not a multiple of 128 */
    q.in = 256;
    q.q4 = NULL;
    CHECK(hlwq_dequantize_int4_grouped(&q, 1, 5, NULL) == HLWQ_ERR_NULL);
    q.q4 = buf;
    q.scales = buf + 2;
    CHECK(hlwq_dequantize_int4_grouped(&q, 1, 5, NULL) == HLWQ_ERR_ALIGN);
    q.rows = (int64_t)1 << 40;
    q.in = (int64_t)1 << 40;
    CHECK(hlwq_dequantize_int4_grouped(&q, 1, 3, NULL) == HLWQ_ERR_SHAPE);
    CHECK(hlwq_dequantize_int4_grouped(&q, 1, 4, NULL) == HLWQ_ERR_BITS);
    CHECK(hlwq_dequantize_int4_grouped(NULL, 1, 5, NULL) == HLWQ_ERR_NULL);
    q.rows = 0;
    CHECK(hlwq_dequantize_int4_grouped(&q, 1, 5, NULL) == HLWQ_OK);        /* nothing to do */
  }
  /* KV cache */
  CHECK(hlwq_kv_quantize(buf, 1, 4, 300, 256, 5, 128, buf, buf, NULL) == HLWQ_ERR_BITS);
  CHECK(hlwq_kv_quantize(buf, 1, 4, -3, 256, 3, 128, buf, buf, NULL) == HLWQ_ERR_SHAPE);
  CHECK(hlwq_kv_quantize(buf, 1, 4, 300, 256, 3, 128, buf + 8, buf, NULL) == HLWQ_ERR_ALIGN);
  CHECK(hlwq_kv_quantize(buf, 1, 4, 100, 256, 3, 128, NULL, NULL, NULL) == HLWQ_OK); /* all tokens stay bf16 */
  CHECK(hlwq_kv_dequantize(buf, buf, INT64_MAX, 4, 300, 256, 3, 128, buf, NULL) == HLWQ_ERR_SHAPE);
  CHECK(hlwq_kv_append(buf, 1, 4, 1, 200, buf, 128, buf, buf, 300, 128, 3, NULL) == HLWQ_ERR_BLOCK);
  CHECK(hlwq_kv_append(buf, 1, 4, 0, 200, buf, 128, buf, buf, 300, 256, 3, NULL) == HLWQ_OK); /* nothing new */
  CHECK(hlwq_kv_append(buf, 1, 4, 1, 200, buf, 128, buf, buf, 50, 256, 3, NULL) == HLWQ_ERR_SHAPE); /* capacity */
  CHECK(hlwq_kv_append(NULL, 1, 4, 1, 200, buf, 128, buf, buf, 300, 256, 3, NULL) == HLWQ_ERR_NULL);
  /* a call writing over one of its own buffers is refused (16-byte aligned
     addresses inside a host array; nothing is dereferenced) */
  {
    char raw[256];
    char* a16 = raw + ((16u - ((uintptr_t)raw & 15u)) & 15u);
    CHECK(hlwq_quantize(a16, 1, 1, 8, 128, 5, a16, a16 + 128, NULL) == HLWQ_ERR_OVERLAP);
    CHECK(hlwq_dequantize(a16, a16 + 128, 1, 1, 8, 128, 5, a16 + 64, NULL) == HLWQ_ERR_OVERLAP);
    CHECK(strlen(hlwq_status_string(HLWQ_ERR_OVERLAP)) > 0);
  }
  /* search tables: a partial copy of the bucket bytes, every entry, the constants */
  {
    uint8_t bytes[16];
    uint32_t entries[64];
    float scale = 0.0f;
    uint32_t bias = 0;
    CHECK(hlwq_search_table(0, bytes, (int)sizeof(bytes), entries, &scale, &bias) > 16);
    CHECK(scale > 0.0f && bias > 0u && entries[1] == 0u && entries[63] == 31u);
    CHECK(hlwq_search_table(7, bytes, (int)sizeof(bytes), entries, &scale, &bias) == HLWQ_ERR_BITS);
  }
  printf("c abi ok\n");
  return 0;
}
