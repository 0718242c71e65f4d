/* A plain C99 caller of the library, built and run by tests/test_abi.py:
 * it includes the public header as C, links against the shared library and
 * exercises the calls that need no GPU (version, status strings, workspace
 * queries, argument validation).  Prints one line per check; exits 0 when
 * every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lightning_attn.h"

static int failures = 0;

static void check(int ok, const char *what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  check(lightning_attn_version() > 0, "version is positive");
  check(strcmp(lightning_attn_status_string(LA_OK), "") != 0, "status string of LA_OK");
  check(lightning_attn_status_string(LA_ERR_INVALID_ARG) != lightning_attn_status_string(LA_OK),
        "distinct status strings");

  /* Workspace queries: a multi-segment plan needs a workspace, a plan of one
   * segment per sequence needs none. */
  const size_t ws = lightning_attn_fwd_workspace_size(1, 64, 32768, 128, 128, LA_BF16, 0);
  check(ws > 0, "headline prefill needs a workspace");
  check(lightning_attn_fwd_workspace_size(1, 64, 32768, 128, 128, LA_BF16,
                                          LA_SEGMENT_PER_SEQUENCE) == 0,
        "one segment per sequence needs no workspace");

  /* Argument validation returns before anything is launched. */
  const void *p = (const void *)(uintptr_t)0x1000; /* never dereferenced */
  check(lightning_attn_fwd(NULL, p, p, (const float *)p, 1, 1, 16, 128, 128, LA_BF16, NULL,
                           (void *)p, NULL, 0, NULL, 0, NULL) == LA_ERR_INVALID_ARG,
        "null q is rejected");
  check(lightning_attn_fwd(p, p, p, (const float *)p, 1, 1, 16, 96, 128, LA_BF16, NULL,
                           (void *)p, NULL, 0, NULL, 0, NULL) == LA_ERR_UNSUPPORTED,
        "d = 96 is unsupported");
  check(lightning_attn_fwd(p, p, p, (const float *)p, 1, 1, 16, 128, 48, LA_BF16, NULL,
                           (void *)p, NULL, 0, NULL, 0, NULL) == LA_ERR_UNSUPPORTED,
        "block 48 is unsupported");
  check(lightning_attn_decode(p, p, p, (const float *)p, (float *)p, (void *)p, 1, 1, 128,
                              (la_dtype)7, NULL) != LA_OK,
        "an unknown dtype is rejected");
  printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
