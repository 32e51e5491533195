/* Uses libwfattn.so from plain C99 through include/wf_attn.h: size queries, status strings and the
 * host-side argument checks (every call below is rejected before anything is enqueued, so no GPU is
 * needed).  Prints "ok" and exits 0 when every expectation holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "wf_attn.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "expectation failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  char buf[64];
  void* const fake = (void*)(size_t)0x10000; /* aligned, never dereferenced */
  EXPECT(wf_abi_version() == 4);
  EXPECT(strcmp(wf_status_string(WF_OK), "WF_OK") == 0);
  EXPECT(strcmp(wf_status_string(WF_ERR_WORKSPACE), "WF_ERR_WORKSPACE") == 0);
  EXPECT(wf_vsa_num_cubes(21, 30, 52) == 624);
  EXPECT(wf_vsa_num_cubes(0, 1, 1) == 0);
  EXPECT(wf_attn_dense_workspace_bytes(2, 40, 32760, 128) == (size_t)2 * 40 * 128 * 32768 * 2);
  EXPECT(wf_vsa_workspace_bytes(1, 40, 21, 30, 52, 128) > 0);
  EXPECT(wf_sta_workspace_bytes(1, 40, 36, 48, 48, 128, 5, 5, 5) > 0);
  EXPECT(wf_sta_workspace_bytes(1, 40, 36, 48, 48, 128, 11, 5, 5) == 0);
  EXPECT(wf_attn_dense(NULL, fake, fake, (float*)fake, NULL, 1, 1, 64, 128, 0.1f, fake, 1u << 30, NULL) ==
         WF_ERR_INVALID_ARG);
  EXPECT(strlen(wf_last_error_detail()) > 0);
  EXPECT(wf_attn_dense(fake, fake, fake, (float*)fake, NULL, 1, 1, 64, 96, 0.1f, fake, 1u << 30, NULL) ==
         WF_ERR_UNSUPPORTED);
  EXPECT(wf_attn_dense_ex(fake, fake, fake, (float*)fake, NULL, 1, 1, 64, 128, 0.1f, 9, fake, 1u << 30, NULL) ==
         WF_ERR_INVALID_ARG);
  EXPECT(wf_attn_dense(fake, fake, fake, (float*)fake, NULL, 1, 1, 64, 128, NAN, fake, 1u << 30, NULL) ==
         WF_ERR_INVALID_ARG);
  EXPECT(wf_vsa_coarse_topk(fake, fake, fake, 1, 2, 5, 6, 7, 128, 0.1f, 9, (int32_t*)fake, NULL, fake, 1u << 30,
                            NULL) == WF_ERR_INVALID_ARG);
  EXPECT(wf_vsa_fine(fake, 16, (const int32_t*)fake, 1, 2, 5, 6, 7, 128, 0.1f, 2, (float*)fake, NULL, NULL) ==
         WF_ERR_WORKSPACE);
  EXPECT(wf_vsa(fake, fake, fake, 1, 2, 5, 6, 7, 128, 0.1f, 3, (int32_t*)fake, NULL, NULL, NULL, NULL, fake,
                1u << 30, NULL) == WF_ERR_INVALID_ARG);
  EXPECT(wf_rope_qk(fake, fake, fake, fake, 1, 2, 5, 6, 7, 128, 1e4, 16, NULL) == WF_ERR_INVALID_ARG);
  EXPECT(wf_sta(fake, fake, fake, 1, 2, 5, 6, 7, 128, 0.1f, 1, 1, 1, (float*)fake, NULL, NULL, fake, 1u << 30,
                NULL) == WF_ERR_UNSUPPORTED);
  EXPECT(wf_sta(fake, fake, fake, 1, 2, 18, 48, 80, 128, 0.1f, 4, 1, 1, (float*)fake, NULL, NULL, fake, 1u << 30,
                NULL) == WF_ERR_INVALID_ARG);
  {
    int64_t n = 0;
    double ms = 0.0;
    EXPECT(wf_profile_query("wf_dense_fwd", &n, &ms) == WF_ERR_INVALID_ARG);
  }
  snprintf(buf, sizeof buf, "%s", failures ? "failed" : "ok");
  puts(buf);
  return failures ? 1 : 0;
}
