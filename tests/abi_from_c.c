/* The library used from plain C through include/ab_attn.h: version, status
 * strings, workspace sizes and argument validation (nothing here reaches a
 * device; every call below fails its checks on the host). Exit status 0 when
 * every check holds, else the number of the first failed check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ab_attn.h"

#define CHECK(n, cond)                                          \
  do {                                                          \
    if (!(cond)) {                                              \
      fprintf(stderr, "check %d failed: %s\n", n, #cond);       \
      return n;                                                 \
    }                                                           \
  } while (0)

int main(void) {
  ab_desc d = {1, 12, 32760, 128, AB_BF16, 128, 32, 8, 4, 0.0f};
  void* fake = (void*)(uintptr_t)256;

  CHECK(1, ab_abi_version() == AB_ABI_VERSION);
  CHECK(2, strlen(ab_status_str(AB_OK)) > 0 && strlen(ab_status_str(AB_ERR_DTYPE)) > 0);
  CHECK(3, ab_score_workspace_size(&d) > 0);
  CHECK(4, ab_fp8_workspace_size(&d) == (size_t)12 * (1024 + 1) * 4);

  ab_desc bad = d;
  bad.d = 96;
  CHECK(5, ab_score_workspace_size(&bad) == 0);
  CHECK(6, strlen(ab_last_error()) > 0);
  CHECK(7, ab_score(&bad, fake, fake, fake, fake, 1u << 30, NULL) == AB_ERR_SHAPE);

  CHECK(8, ab_score(NULL, fake, fake, fake, fake, 1u << 30, NULL) == AB_ERR_NULL);
  CHECK(9, ab_sample(&d, fake, 0.0, 0, fake, fake, fake, NULL, NULL) == AB_ERR_DENSITY);
  CHECK(10, ab_attn_fwd(&d, fake, fake, NULL, fake, fake, fake, fake, NULL, NULL) == AB_ERR_NULL);
  CHECK(11, ab_intra_lists(&d, 7, 0, fake, fake, fake, NULL, NULL) == AB_ERR_PARAM);
  CHECK(12, ab_attn_fwd_ordered(&d, fake, fake, fake, fake, fake, fake, NULL, fake, NULL, NULL) == AB_ERR_NULL);

  ab_desc f32 = d;
  f32.dtype = AB_F32;
  CHECK(13, ab_attn_fwd_fp8(&f32, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, NULL, NULL) ==
                AB_ERR_DTYPE);
  printf("abi_from_c: all checks passed (ABI version %d)\n", ab_abi_version());
  return 0;
}
