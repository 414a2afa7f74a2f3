/*
 * A plain C99 caller of libsa2: the header compiles as C, the library links,
 * and calls that fail validation return their status and message without
 * touching a device (so this runs on a host without a GPU).  Exit status 0
 * when every check holds; the failing check's line otherwise.
 */
#include <stdio.h>
#include <string.h>

#include "sa2.h"

#define CHECK(c)                                            \
  do {                                                      \
    if (!(c)) {                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                             \
    }                                                       \
  } while (0)

int main(void) {
  CHECK(strncmp(sa2_version(), "sa2 ", 4) == 0);
  CHECK(sa2_mask_workspace_bytes(1, 12, 32760, 128, 128, 64) > 0);
  CHECK(sa2_mask_workspace_bytes(0, 12, 32760, 128, 128, 64) == 0);
  CHECK(sa2_bwd_workspace_bytes(1, 12, 32760, 128) > sa2_bwd_workspace_bytes(1, 12, 32760, 64));
  CHECK(sa2_fwd_workspace_bytes(1, 12, 32760, 128) > 0);
  CHECK(sa2_fwd_workspace_bytes(1, 12, 32760, 64) == 0);

  sa2_mask m;
  memset(&m, 0, sizeof m);
  m.B = 1; m.H = 1; m.N = 256; m.bq = 64; m.bk = 64; m.Tq = 4; m.Tk = 4;
  /* null q: rejected before any launch */
  sa2_status st = sa2_build_mask(NULL, NULL, SA2_BF16, 1, 1, 256, 64, 64, 64, 0.1, 0.5, &m,
                                 NULL, 0, NULL);
  CHECK(st == SA2_EINVAL);
  CHECK(strncmp(sa2_last_error(), "sa2_build_mask", 14) == 0);
  /* d = 96 is not implemented by the attention kernels */
  char dummy[64];
  void* p = (void*)(((uintptr_t)dummy + 15) & ~(uintptr_t)15);
  st = sa2_attn_fwd(p, p, p, SA2_BF16, 1, 1, 256, 96, &m, p, (float*)p, NULL, 0, NULL);
  CHECK(st == SA2_EUNSUPPORTED);
  st = sa2_attn_bwd(p, p, p, p, (const float*)p, p, SA2_BF16, 1, 1, 256, 64, &m, p, p, p, p, 16,
                    NULL);
  CHECK(st == SA2_EINVAL);
  printf("c abi ok: %s\n", sa2_version());
  return 0;
}
