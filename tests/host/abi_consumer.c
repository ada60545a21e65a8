/* A plain C99 caller of libsolattn: the header must compile as C, and the host-side
 * entry points (argument checks, workspace sizing and layout, the errors that every
 * call returns before launching anything) must behave as include/solattn.h states.
 * Nothing here touches a device: no call below reaches a launch.  Exit status 0 and
 * one "ok" line per check on success. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "solattn.h"

static int failures = 0;

static void check(int cond, const char* what) {
  printf("%s %s\n", cond ? "ok" : "FAIL", what);
  if (!cond) ++failures;
}

int main(void) {
  /* sol_attn_validate: the tensor contract and the threshold (host only) */
  check(sol_attn_validate(1, 1024, 2, 128, 1.0f, -1, 0, SOL_THRESH_DIAG) == SOL_OK, "validate: good shape");
  check(sol_attn_validate(1, 1024, 2, 64, 1.0f, -1, 0, SOL_THRESH_DIAG) == SOL_ERR_HEAD_DIM, "validate: head_dim 64");
  check(sol_attn_validate(0, 1024, 2, 128, 1.0f, -1, 0, SOL_THRESH_DIAG) == SOL_ERR_SHAPE, "validate: batch 0");
  check(sol_attn_validate(1, 1024, 2, 128, (float)NAN, -1, 0, SOL_THRESH_DIAG) == SOL_ERR_TAU, "validate: NaN tau");
  check(sol_attn_validate(1, 1024, 2, 128, (float)INFINITY, -1, 0, SOL_THRESH_DIAG) == SOL_ERR_TAU,
        "validate: infinite tau");
  check(sol_attn_validate(1, 1024, 2, 128, 1.0f, 1000, 100, SOL_THRESH_DIAG) == SOL_ERR_SINK,
        "validate: sink past the end");
  check(sol_attn_validate(1, 1024, 2, 128, 1.0f, 0, 1024, SOL_THRESH_EXACT) == SOL_OK,
        "validate: whole-sequence sink, exact threshold");
  check(sol_attn_validate(1, 1024, 2, 128, 1.0f, -1, 0, 7) == SOL_ERR_ARG, "validate: unknown threshold type");

  /* workspace size and layout agree; Sol-Attn2 layouts exist; bad shapes give 0 / an error */
  {
    sol_ws_layout L;
    const size_t bytes = sol_attn_workspace_bytes(SOL_VARIANT_SOL1, 1, 32768, 32, 128);
    memset(&L, 0, sizeof L);
    check(sol_attn_workspace_layout(SOL_VARIANT_SOL1, 1, 32768, 32, 128, &L) == SOL_OK, "layout: Sol-Attn");
    check(bytes > 0 && (int64_t)bytes == L.total_bytes, "layout: total matches workspace_bytes");
    check(L.nb == 512 && L.nbp == 512 && L.kv_splits == 1, "layout: 512 blocks, one key split at 32768 tokens");
    check(L.qbar >= 0 && L.kh >= 0 && L.vh >= 0 && L.order >= 0 && L.q8 == -1, "layout: Sol-Attn arrays only");
    check(sol_attn_workspace_layout(SOL_VARIANT_SOL2_PV8, 1, 32768, 32, 128, &L) == SOL_OK && L.v8t >= 0 &&
              L.q8 >= 0,
          "layout: Sol-Attn2 FP8 PV");
    check(sol_attn_workspace_bytes(SOL_VARIANT_SOL1, 1, 1024, 2, 96) == 0, "workspace_bytes: head_dim 96 gives 0");
    check(sol_attn_workspace_layout(9, 1, 1024, 2, 128, &L) != SOL_OK, "layout: unknown variant");
    check(sol_attn_kv_splits(1, 32768, 32, 0) == 1 && sol_attn_kv_splits(1, 131584, 32, 0) == 4,
          "kv_splits: automatic rule (1 at 32768 tokens, 4 at 512 + 131072)");
  }

  /* full calls return their argument errors before any launch; the pointers are never read */
  {
    void* const fake = (void*)(uintptr_t)0x100000;   /* 16-byte aligned, never dereferenced */
    check(sol_attn(NULL, fake, fake, fake, 1, 1024, 2, 128, 1.0f, -1, 0, SOL_THRESH_DIAG, fake, 1u << 30, NULL) ==
              SOL_ERR_NULL,
          "sol_attn: NULL q");
    check(sol_attn(fake, fake, fake, fake, 1, 1024, 2, 128, 1.0f, -1, 0, SOL_THRESH_DIAG, fake, 64, NULL) ==
              SOL_ERR_WORKSPACE,
          "sol_attn: workspace too small");
    check(sol_attn2(fake, fake, fake, fake, 1, 1024, 2, 128, (float)NAN, -1, 0, SOL_THRESH_DIAG, fake, 1u << 30,
                    NULL) == SOL_ERR_TAU,
          "sol_attn2: NaN tau");
    check(sol_attn_noalloc(fake, fake, fake, fake, 1, 32768, 32, 128, 1.0f, -1, 0, SOL_THRESH_DIAG, NULL) ==
              SOL_ERR_SCRATCH,
          "sol_attn_noalloc: shape beyond the static scratch");
  }
  check(sol_status_string(SOL_ERR_TAU) != NULL && sol_status_string(SOL_ERR_TAU)[0] != '\0' &&
            sol_status_string(12345) != NULL,
        "status strings");
  printf("%d failures\n", failures);
  return failures != 0;
}
