/* Plain C client of libhlwq: compiles against include/hlwq.h with a C
 * compiler and exercises the host-only entry points and the argument checks
 * of the device entry points (no kernel is launched).  Exit status 0 on
 * success; prints the first failed check otherwise. */
#include <stdio.h>
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
  printf("c abi ok\n");
  return 0;
}
