/* Host-side sanitizer driver for the C ABI's argument checking (test
 * infrastructure only).  Built against an AddressSanitizer /
 * UndefinedBehaviorSanitizer build of api.cpp, it calls every entry point
 * with a null handle or with invalid arguments and checks the status codes
 * and error messages; every such call must return before any HIP call, so
 * it runs without a GPU.  Host buffers stand in for device pointers: the
 * checks compare addresses and never dereference them.  Exit status 0 when
 * every call returned what it should. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssm_scan.h"

static int fails = 0;
static void expect(ssm_status got, ssm_status want, const char *needle, const char *what) {
  const char *msg = ssm_last_error_message();
  if (got != want || (needle && (!msg || !strstr(msg, needle)))) {
    fprintf(stderr, "%s: status %d (want %d), message '%s' (want '%s')\n", what, (int)got,
            (int)want, msg ? msg : "(null)", needle ? needle : "");
    ++fails;
  }
}

int main(void) {
  enum { NBUF = 24 };
  char *buf[NBUF];
  for (int i = 0; i < NBUF; ++i) buf[i] = aligned_alloc(256, 1 << 20);
  void **P = (void **)buf;
  const ssm_status OK = SSM_OK, BAD = SSM_ERR_INVALID_ARG, UNS = SSM_ERR_UNSUPPORTED;
  (void)OK;

  for (int s = 0; s <= 4; ++s)
    if (!ssm_status_string((ssm_status)s)) {
      fprintf(stderr, "status_string(%d) is NULL\n", s);
      ++fails;
    }
  expect(ssm_scan_destroy(NULL), SSM_OK, NULL, "destroy(NULL)");
  expect(ssm_scan_create(NULL, 0), BAD, NULL, "create(NULL)");

  /* forward */
  expect(ssm_selective_scan_fwd(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, P[5],
                                NULL, 2, 8, 16, 32, SSM_F32, NULL), BAD, "handle", "fwd handle");
  expect(ssm_selective_scan_fwd(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, P[5],
                                NULL, 0, 8, 16, 32, SSM_F32, NULL), BAD, "batch", "fwd batch 0");
  expect(ssm_selective_scan_fwd(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, P[5],
                                NULL, 2, 8, 65, 32, SSM_F32, NULL), UNS, "dstate", "fwd dstate");
  expect(ssm_selective_scan_fwd(NULL, NULL, P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, P[5],
                                NULL, 2, 8, 16, 32, SSM_F32, NULL), BAD, "u", "fwd u NULL");
  expect(ssm_selective_scan_fwd(NULL, P[0] , P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1,
                                buf[0] + 64, NULL, 2, 8, 16, 32, SSM_BF16, NULL), BAD, "overlap",
         "fwd y overlaps u");
  expect(ssm_selective_scan_fwd(NULL, buf[0] + 4, P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1,
                                P[5], NULL, 2, 8, 16, 32, SSM_F32, NULL), BAD, "aligned",
         "fwd misaligned");
  expect(ssm_selective_scan_fwd(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, P[5],
                                NULL, 2, 8, 16, 32, (ssm_dtype)7, NULL), BAD, "dtype", "fwd dtype");
  expect(ssm_selective_scan_fwd_with_state(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL,
                                           1, (const float *)P[6], P[5], (float *)P[7], 2, 8, 16,
                                           32, SSM_F32, NULL), BAD, "handle", "fwd state");
  expect(ssm_selective_scan_fwd_grouped(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1,
                                        NULL, P[5], NULL, 2, 8, 16, 32, 3, SSM_F32, NULL), BAD,
         "ngroups", "fwd grouped ngroups");
  {
    size_t n = 7;
    expect(ssm_selective_scan_fwd_workspace_size(NULL, 2, 8, 16, 32, 1, &n), BAD, "handle",
           "fwd ws size");
    expect(ssm_selective_scan_fwd_workspace_size(NULL, 2, 8, 16, 32, 1, NULL), BAD, NULL,
           "fwd ws size NULL");
  }
  expect(ssm_selective_scan_fwd_ws(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, NULL,
                                   P[5], NULL, 2, 8, 16, 32, 1, P[8], 1 << 20, SSM_F32, NULL), BAD,
         "handle", "fwd ws");
  expect(ssm_selective_scan_fwd_noalloc(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1,
                                        NULL, P[5], NULL, 2, 8, 16, 32, 1, SSM_F32, NULL), BAD,
         "handle", "fwd noalloc");

  /* backward */
  {
    size_t n = 7;
    expect(ssm_selective_scan_bwd_workspace_size(NULL, 2, 8, 16, 32, &n), BAD, "handle",
           "bwd ws size");
    expect(ssm_selective_scan_bwd_grouped_workspace_size(NULL, 2, 8, 16, 32, 3, &n), BAD,
           "ngroups", "bwd ws size ngroups");
    expect(ssm_selective_scan_bwd_grouped_workspace_size(NULL, 2, 8, 16, 32, 8, &n), BAD,
           "handle", "bwd ws size per channel");
  }
  expect(ssm_selective_scan_bwd(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1, NULL,
                                P[5], NULL, P[6], P[7], (float *)P[8], (float *)P[9],
                                (float *)P[10], NULL, NULL, NULL, NULL, P[11], 1 << 20, 2, 8, 16,
                                32, SSM_F32, NULL), BAD, "handle", "bwd");
  expect(ssm_selective_scan_bwd(NULL, P[0], P[1], P[2], P[3], P[4], NULL, P[12], NULL, 1, NULL,
                                P[5], NULL, P[6], P[7], (float *)P[8], (float *)P[9],
                                (float *)P[10], NULL, NULL, NULL, NULL, P[11], 1 << 20, 2, 8, 16,
                                32, SSM_F32, NULL), BAD, "dz", "bwd z without dz");
  expect(ssm_selective_scan_bwd_grouped(NULL, P[0], P[1], P[2], P[3], P[4], NULL, NULL, NULL, 1,
                                        NULL, P[5], NULL, P[6], P[7], (float *)P[8],
                                        (float *)P[9], (float *)P[10], NULL, NULL, NULL, NULL,
                                        P[11], 1 << 20, 2, 8, 16, 32, 8, SSM_BF16, NULL), BAD,
         "handle", "bwd per channel");

  /* decode steps */
  expect(ssm_selective_state_update(NULL, (float *)P[0], P[1], P[2], (float *)P[3], P[4], P[5],
                                    NULL, NULL, NULL, 1, P[6], 2, 8, 16, SSM_F32, NULL), BAD,
         "handle", "step");
  expect(ssm_selective_state_update_grouped(NULL, (float *)P[0], P[1], P[2], (float *)P[3], P[4],
                                            P[5], NULL, NULL, NULL, 1, P[6], 2, 8, 16, 3,
                                            SSM_F32, NULL), BAD, "ngroups", "step grouped");
  expect(ssm_selective_state_update(NULL, (float *)P[0], P[1], P[2], (float *)P[3], P[4], P[5],
                                    NULL, NULL, NULL, 1, P[0], 2, 8, 16, SSM_F32, NULL), BAD,
         "overlap", "step y is state");
  expect(ssd_state_update(NULL, (float *)P[0], P[1], P[2], (float *)P[3], P[4], P[5], NULL, NULL,
                          1, P[6], 2, 4, 16, 32, 3, SSM_BF16, NULL), BAD, "ngroups",
         "ssd step ngroups");
  expect(ssd_state_update(NULL, (float *)P[0], P[1], P[2], (float *)P[3], P[4], P[5], NULL, NULL,
                          1, P[6], 2, 4, 16, 257, 1, SSM_BF16, NULL), UNS, "dstate",
         "ssd step dstate");

  /* SSD chunked scan */
  {
    size_t n = 7;
    expect(ssd_chunk_scan_workspace_size(NULL, 2, 512, 4, 64, 128, 1, 256, &n), BAD, "handle",
           "ssd ws size");
    expect(ssd_chunk_scan_workspace_size(NULL, 2, 512, 4, 64, 128, 1, 100, &n), UNS, NULL,
           "ssd ws chunk");
    expect(ssd_chunk_scan_workspace_size(NULL, 2, 512, 4, 129, 128, 1, 256, &n), UNS, NULL,
           "ssd ws headdim");
  }
  expect(ssd_chunk_scan_fwd(NULL, P[0], P[1], (float *)P[2], P[3], P[4], NULL, NULL, 1, P[5],
                            NULL, P[6], 1 << 20, 2, 512, 4, 64, 128, 1, 256, SSM_BF16, NULL), BAD,
         "handle", "ssd");
  expect(ssd_chunk_scan_fwd(NULL, P[0], P[1], (float *)P[2], P[3], P[4], NULL, NULL, 1, P[5],
                            NULL, P[6], 1 << 20, 2, 512, 4, 64, 128, 1, 256, SSM_F32, NULL), UNS,
         NULL, "ssd f32");
  expect(ssd_chunk_scan_fwd_with_state(NULL, P[0], P[1], (float *)P[2], P[3], P[4], NULL, NULL,
                                       1, (const float *)P[7], P[5], NULL, P[6], 1 << 20, 2, 512,
                                       4, 64, 128, 1, 256, SSM_BF16, NULL), BAD, "handle",
         "ssd state");

  for (int i = 0; i < NBUF; ++i) free(buf[i]);
  if (fails) {
    fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  printf("abi driver: all calls as expected\n");
  return 0;
}
