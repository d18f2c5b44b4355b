/* Host-side checks of the C ABI (include/mamba_mi355x.h) for a build of the
 * library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py).  Every call here is rejected or answered on the
 * host before the HIP runtime is touched; no GPU is needed.  The fake device
 * pointers are never dereferenced. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mamba_mi355x.h"

static int fails = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      ++fails;                                                          \
    }                                                                   \
  } while (0)

int main(void) {
  void* F = (void*)(uintptr_t)0x10000; /* aligned, never dereferenced */
  void* M = (void*)(uintptr_t)0x10004; /* misaligned */
  CHECK(mamba_version() == 200);
  for (int st = 0; st < 12; ++st) CHECK(mamba_status_string(st) != NULL && strlen(mamba_status_string(st)) > 0);
  /* workspace sizes: pure host functions */
  CHECK(mamba_scan_fwd_workspace_size(4, 4096, 5120, 16, MAMBA_IO_BF16) == 0);
  CHECK(mamba_scan_fwd_workspace_size(1, 1 << 20, 256, 16, MAMBA_IO_F32) > 0);
  CHECK(mamba_scan_fwd_workspace_size(1, 16, 64, 3, MAMBA_IO_F32) == 0);
  CHECK(mamba_scan_fwd_workspace_size(-1, 16, 64, 16, MAMBA_IO_F32) == 0);
  CHECK(mamba_scan_bwd_workspace_size(4, 4096, 5120, 16, MAMBA_IO_BF16) > 0);
  CHECK(mamba_scan_fwd_complex_workspace_size(2, 3000, 128, 16, MAMBA_IO_F32) > 0);
  CHECK(mamba_selection_fwd_workspace_size(2, 100, 256, 16, 8, MAMBA_IO_F32) < ((size_t)1 << 40));
  CHECK(mamba_ssm_fwd_workspace_size(2, 100, 256, 16, 8, MAMBA_IO_F32) < ((size_t)1 << 40));
  CHECK(mamba_block_fwd_workspace_size(2, 100, 128, 256, 16, 8, MAMBA_IO_F32) < ((size_t)1 << 40));
  /* options */
  const int64_t keep = mamba_get_option(MAMBA_OPT_ENGINE);
  CHECK(mamba_set_option(MAMBA_OPT_ENGINE, 2) == MAMBA_OK && mamba_get_option(MAMBA_OPT_ENGINE) == 2);
  CHECK(mamba_scan_fwd_workspace_size(4, 4096, 5120, 16, MAMBA_IO_BF16) > 0);
  CHECK(mamba_set_option(MAMBA_OPT_ENGINE, 9) == MAMBA_ERR_OPTION);
  CHECK(mamba_set_option(MAMBA_OPT_ENGINE, keep) == MAMBA_OK);
  CHECK(mamba_set_option(99, 0) == MAMBA_ERR_OPTION && mamba_get_option(99) == -1);
  CHECK(mamba_set_option(MAMBA_OPT_SPIN_LIMIT, (int64_t)1 << 33) == MAMBA_ERR_OPTION);
  CHECK(mamba_set_option(MAMBA_OPT_AGG_SKIP, 2) == MAMBA_ERR_OPTION);
  /* forward scan validation */
  CHECK(mamba_scan_fwd(1, 8, 64, 16, 7, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_DTYPE);
  CHECK(mamba_scan_fwd(1, 8, 64, 3, 0, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_UNSUPPORTED);
  CHECK(mamba_scan_fwd(-1, 8, 64, 16, 0, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_DIM);
  CHECK(mamba_scan_fwd(1, 8, 64, 16, 0, NULL, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_NULL);
  CHECK(mamba_scan_fwd(1, 8, 64, 16, 0, M, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_ALIGN);
  CHECK(mamba_scan_fwd(1, 1 << 20, 256, 16, 0, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_WORKSPACE);
  CHECK(mamba_scan_fwd(0, 8, 64, 16, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL, NULL, 0,
                       NULL) == MAMBA_OK);
  /* the no-allocation scan refuses workspaces beyond its array */
  CHECK(mamba_set_option(MAMBA_OPT_ENGINE, 2) == MAMBA_OK);
  CHECK(mamba_scan_fwd_noalloc(64, 1, 16384, 16, 0, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL) ==
        MAMBA_ERR_WORKSPACE);
  CHECK(mamba_set_option(MAMBA_OPT_ENGINE, keep) == MAMBA_OK);
  CHECK(mamba_scan_fwd_noalloc(1, 8, 64, 3, 0, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL) ==
        MAMBA_ERR_UNSUPPORTED);
  /* decode and complex entry points */
  CHECK(mamba_state_update(2, 64, 16, 0, NULL, F, F, NULL, F, F, F, NULL, NULL, 1, F, NULL) == MAMBA_ERR_NULL);
  CHECK(mamba_state_update(2, 64, 5, 0, F, F, F, NULL, F, F, F, NULL, NULL, 1, F, NULL) == MAMBA_ERR_UNSUPPORTED);
  CHECK(mamba_state_update_complex(2, 64, 16, 0, F, M, F, NULL, F, F, F, NULL, NULL, 1, F, NULL) == MAMBA_ERR_ALIGN);
  CHECK(mamba_scan_fwd_complex(1, 8, 64, 16, 3, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, F, NULL, NULL, 0, NULL) ==
        MAMBA_ERR_DTYPE);
  /* backward, selection and block validation */
  CHECK(mamba_scan_bwd(1, 8, 64, 16, 0, F, F, NULL, F, F, F, NULL, NULL, 1, NULL, NULL, NULL, F, F, F, F, F, NULL,
                       NULL, NULL, NULL, NULL, 0, NULL) == MAMBA_ERR_NULL);
  CHECK(mamba_selection_fwd(1, 8, 64, 16, 0, 0, F, F, F, F, F, F, NULL, 0, NULL) != MAMBA_OK);
  CHECK(mamba_calibrate_copy(F, F, 17, 16, NULL) == MAMBA_ERR_ALIGN);
  CHECK(mamba_calibrate_copy(NULL, F, 16, 16, NULL) == MAMBA_ERR_NULL);
  CHECK(mamba_calibrate_copy(F, F, 16, -4, NULL) == MAMBA_ERR_DIM);
  CHECK(mamba_calibrate_copy(F, F, 0, 1, NULL) == MAMBA_OK);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("abi driver: all checks passed\n");
  return 0;
}
