/*
 * A plain C99 caller of libsa2: the header compiles as C, the library links,
 * and calls that fail validation return their status and message without
 * touching a device (so this runs on a host without a GPU).  Every pointer
 * below is a fake address that validation refuses before any use.  The same
 * program runs against a build whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Exit status 0 when every check holds; the
 * failing check's line otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sa2.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

/* status `want` and a last-error message containing `text` */
#define EXPECT(call, want, text)                                                        \
  do {                                                                                  \
    sa2_status st_ = (call);                                                            \
    if (st_ != (want) || strstr(sa2_last_error(), (text)) == NULL) {                    \
      fprintf(stderr, "check failed at line %d: status %d, message \"%s\"\n", __LINE__, \
              (int)st_, sa2_last_error());                                              \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)

#define FAKE ((void*)((uintptr_t)1 << 20))
#define FAKE_AT(off) ((void*)(((uintptr_t)1 << 20) + (off)))

static sa2_mask make_mask(int B, int H, int N, int bq, int bk) {
  sa2_mask m;
  memset(&m, 0, sizeof m);
  m.B = B; m.H = H; m.N = N; m.bq = bq; m.bk = bk;
  m.Tq = (N + bq - 1) / bq; m.Tk = (N + bk - 1) / bk;
  m.bitmap = (uint8_t*)FAKE;
  m.row_cnt = m.row_idx = m.col_cnt = m.col_idx = m.row_plan = m.col_plan = (int32_t*)FAKE;
  return m;
}

int main(void) {
  CHECK(strncmp(sa2_version(), "sa2 ", 4) == 0);

  /* size queries */
  CHECK(sa2_mask_workspace_bytes(1, 12, 32760, 128, 128, 64) > 0);
  CHECK(sa2_mask_workspace_bytes(0, 12, 32760, 128, 128, 64) == 0);
  CHECK(sa2_mask_plan_bytes(1, 12, 32760, 128, 64, 0) > 0);
  CHECK(sa2_mask_plan_bytes(1, 12, 32760, 128, 64, 1) > 0);
  CHECK(sa2_mask_plan_bytes(1, 12, 32760, 128, 64, 2) == 0);
  CHECK(sa2_bwd_workspace_bytes(1, 12, 32760, 128) > sa2_bwd_workspace_bytes(1, 12, 32760, 64));
  CHECK(sa2_bwd_atomic_workspace_bytes(1, 12, 32760, 128) >
        sa2_bwd_workspace_bytes(1, 12, 32760, 128));
  CHECK(sa2_fwd_workspace_bytes(1, 12, 32760, 128) > 0);
  CHECK(sa2_fwd_workspace_bytes(1, 12, 32760, 64) == 0);
  CHECK(sa2_distill_workspace_bytes(1, 2, 64, 64) >= 8);
  CHECK(sa2_distill_workspace_bytes(0, 2, 64, 64) == 0);

  /* mask builder: every argument check, each message naming the call */
  {
    sa2_mask m = make_mask(1, 1, 256, 64, 64);
    const size_t big = (size_t)1 << 30;
    EXPECT(sa2_build_mask(NULL, FAKE, SA2_BF16, 1, 1, 256, 64, 64, 64, 0.1, 0.5, &m, FAKE, big,
                          NULL), SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 0, 64, 64, 64, 0.1, 0.5, &m, FAKE, big,
                          NULL), SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, 7, 1, 1, 256, 64, 64, 64, 0.1, 0.5, &m, FAKE, big, NULL),
           SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 256, 60, 64, 64, 0.1, 0.5, &m, FAKE, big,
                          NULL), SA2_EUNSUPPORTED, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 256, 64, 64, 64, 0.0, 0.0, &m, FAKE, big,
                          NULL), SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 256, 64, 64, 64, (double)NAN, 0.5, &m, FAKE,
                          big, NULL), SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE_AT(4), FAKE, SA2_BF16, 1, 1, 256, 64, 64, 64, 0.1, 0.5, &m, FAKE,
                          big, NULL), SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 256, 64, 64, 64, 0.1, 0.5, &m, FAKE_AT(64),
                          big, NULL), SA2_EINVAL, "sa2_build_mask");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 300, 64, 64, 64, 0.1, 0.5, &m, FAKE, big,
                          NULL), SA2_EINVAL, "sa2_build_mask");   /* mask geometry differs */
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 1, 256, 64, 64, 64, 0.1, 0.5, &m, FAKE, 16,
                          NULL), SA2_EINVAL, "sa2_build_mask");
    /* more (batch, head) pairs than a grid dimension holds */
    sa2_mask wide = make_mask(1, 70000, 256, 64, 64);
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, 1, 70000, 256, 64, 64, 64, 0.1, 0.5, &wide, FAKE,
                          (size_t)1 << 40, NULL), SA2_EUNSUPPORTED, "sa2_build_mask");
  }

  /* attention: unsupported shapes, missing buffers, short workspaces */
  {
    sa2_mask m = make_mask(1, 1, 256, 64, 64);
    sa2_mask m32 = make_mask(1, 1, 256, 64, 32);
    sa2_mask m128 = make_mask(1, 1, 256, 128, 64);
    EXPECT(sa2_attn_fwd(FAKE, FAKE, FAKE, SA2_BF16, 1, 1, 256, 96, &m, FAKE, (float*)FAKE, NULL, 0,
                        NULL), SA2_EUNSUPPORTED, "d must be");
    EXPECT(sa2_attn_fwd(FAKE, FAKE, FAKE, SA2_BF16, 1, 1, 256, 64, &m32, FAKE, (float*)FAKE, NULL,
                        0, NULL), SA2_EUNSUPPORTED, "key blocks");
    EXPECT(sa2_attn_fwd(FAKE, FAKE, NULL, SA2_BF16, 1, 1, 256, 64, &m, FAKE, (float*)FAKE, NULL, 0,
                        NULL), SA2_EINVAL, "sa2_attn_fwd");
    const size_t fneed = sa2_fwd_workspace_bytes(1, 1, 256, 128);
    EXPECT(sa2_attn_fwd(FAKE, FAKE, FAKE, SA2_BF16, 1, 1, 256, 128, &m128, FAKE, (float*)FAKE,
                        NULL, 0, NULL), SA2_EINVAL, "workspace");
    EXPECT(sa2_attn_fwd(FAKE, FAKE, FAKE, SA2_BF16, 1, 1, 256, 128, &m128, FAKE, (float*)FAKE,
                        FAKE, fneed - 1, NULL), SA2_EINVAL, "workspace");
    EXPECT(sa2_attn_bwd(FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, SA2_BF16, 1, 1, 256, 64,
                        &m, FAKE, FAKE, FAKE, FAKE, 16, NULL), SA2_EINVAL, "workspace");
    /* the atomic-dQ backward: bf16 with d = 128 only, and its larger workspace */
    EXPECT(sa2_attn_bwd_atomic_dq(FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, SA2_BF16, 1, 1,
                                  256, 64, &m, FAKE, FAKE, FAKE, FAKE, (size_t)1 << 30, NULL),
           SA2_EUNSUPPORTED, "bf16 with d = 128");
    EXPECT(sa2_attn_bwd_atomic_dq(FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, SA2_BF16, 1, 1,
                                  256, 128, &m128, FAKE, FAKE, FAKE, FAKE,
                                  sa2_bwd_workspace_bytes(1, 1, 256, 128), NULL),
           SA2_EINVAL, "workspace");
  }

  /* bf16, d = 128: a mask without its plans (or with a misaligned one) */
  {
    const int B = 1, H = 1, N = 256;
    sa2_mask no_rows = make_mask(B, H, N, 128, 64);
    sa2_mask no_cols = make_mask(B, H, N, 128, 64);
    sa2_mask odd = make_mask(B, H, N, 128, 64);
    no_rows.row_plan = NULL;
    no_cols.col_plan = NULL;
    odd.row_plan = (int32_t*)FAKE_AT(4);
    const size_t wsb = sa2_bwd_workspace_bytes(B, H, N, 128);
    const size_t fwb = sa2_fwd_workspace_bytes(B, H, N, 128);
    const sa2_mask* bad[2] = {&no_rows, &odd};
    int i;
    for (i = 0; i < 2; ++i) {
      EXPECT(sa2_attn_fwd(FAKE, FAKE, FAKE, SA2_BF16, B, H, N, 128, bad[i], FAKE, (float*)FAKE,
                          FAKE, fwb, NULL), SA2_EINVAL, "row plan");
      EXPECT(sa2_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, SA2_BF16, B, H, N,
                             128, bad[i], FAKE, FAKE, wsb, NULL), SA2_EINVAL, "row plan");
    }
    EXPECT(sa2_attn_bwd_dkdv(FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, SA2_BF16, B, H, N, 128,
                             &no_cols, FAKE, FAKE, FAKE, wsb, NULL), SA2_EINVAL, "column plan");
    EXPECT(sa2_build_mask(FAKE, FAKE, SA2_BF16, B, H, N, 128, 128, 64, 0.1, 0.5, &no_cols, FAKE,
                          (size_t)1 << 30, NULL), SA2_EINVAL, "null");
    EXPECT(sa2_mask_plans(&no_rows, NULL), SA2_EINVAL, "sa2_mask_plans");
  }

  /* the allocation-free mask builder: a geometry beyond its static scratch */
  {
    const int B = 1, H = 40, N = 75600, d = 128;
    sa2_mask m = make_mask(B, H, N, 128, 64);
    CHECK(sa2_mask_workspace_bytes(B, H, N, d, 128, 64) > SA2_MASK_NOALLOC_MAX_BYTES);
    EXPECT(sa2_build_mask_noalloc(FAKE, FAKE, SA2_BF16, B, H, N, d, 128, 64, 0.03, 0.1, &m, NULL),
           SA2_EUNSUPPORTED, "static scratch");
    EXPECT(sa2_build_mask_noalloc(FAKE, FAKE, SA2_BF16, B, H, N, d, 128, 64, 0.0, 0.0, &m, NULL),
           SA2_EINVAL, "sa2_build_mask_noalloc");
  }

  /* the distillation loss */
  {
    double* loss = (double*)FAKE;
    const size_t big = (size_t)1 << 20;
    EXPECT(sa2_distill_loss_grad(NULL, FAKE, SA2_BF16, 1, 2, 64, 64, FAKE, loss, FAKE, big, NULL),
           SA2_EINVAL, "sa2_distill");
    EXPECT(sa2_distill_loss_grad(FAKE, FAKE, 5, 1, 2, 64, 64, FAKE, loss, FAKE, big, NULL),
           SA2_EINVAL, "sa2_distill");
    EXPECT(sa2_distill_loss_grad(FAKE, FAKE, SA2_BF16, 1, 2, 64, 12, FAKE, loss, FAKE, big, NULL),
           SA2_EUNSUPPORTED, "sa2_distill");
    EXPECT(sa2_distill_loss_grad(FAKE, FAKE, SA2_BF16, 1, 2, 0, 64, FAKE, loss, FAKE, big, NULL),
           SA2_EINVAL, "sa2_distill");
    EXPECT(sa2_distill_loss_grad(FAKE, FAKE, SA2_BF16, 1, 2, 64, 64, FAKE_AT(8), loss, FAKE, big,
                                 NULL), SA2_EINVAL, "sa2_distill");
    EXPECT(sa2_distill_loss_grad(FAKE, FAKE, SA2_BF16, 1, 2, 64, 64, FAKE, loss, FAKE_AT(16), big,
                                 NULL), SA2_EINVAL, "sa2_distill");
    EXPECT(sa2_distill_loss_grad(FAKE, FAKE, SA2_BF16, 1, 2, 64, 64, FAKE, loss, FAKE, 8, NULL),
           SA2_EINVAL, "sa2_distill");
  }

  printf("c abi ok: %s\n", sa2_version());
  return 0;
}
