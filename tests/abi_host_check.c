/*
 * Host-side checks of the C ABI (include/streamkl.h), built against a copy of
 * the host layer compiled with AddressSanitizer and UndefinedBehaviorSanitizer
 * (see attention_kl_divergence_amd/build.py, build_host_check) and run on a
 * machine without a GPU.  Every call here either fails validation before any
 * device call or only plans and sizes; a sanitizer report or a wrong status
 * ends the program with a non-zero code.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/streamkl.h"

static int failures = 0;

#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static streamkl_shape shape(int64_t B, int64_t H, int64_t n_q, int64_t n_k, int d1, int d2, int dtype) {
  streamkl_shape s;
  memset(&s, 0, sizeof s);
  s.B = B; s.H = H; s.n_q = n_q; s.n_k = n_k; s.d1 = d1; s.d2 = d2; s.dtype = dtype;
  return s;
}

int main(void) {
  void* p = (void*)(uintptr_t)256;   /* aligned, never dereferenced: validation fails first */
  void* odd = (void*)(uintptr_t)258;
  float* fp = (float*)p;
  streamkl_shape good = shape(1, 2, 64, 64, 128, 128, STREAMKL_BF16);

  /* invalid shapes, for every entry point */
  streamkl_shape bad[6];
  bad[0] = shape(0, 2, 64, 64, 128, 128, STREAMKL_BF16);
  bad[1] = shape(1, 2, 0, 64, 128, 128, STREAMKL_BF16);
  bad[2] = shape(1, 2, 64, 64, 96, 128, STREAMKL_BF16);
  bad[3] = shape(1, 2, 64, 64, 128, 128, 9);
  bad[4] = shape(1, 2, (int64_t)1 << 25, 64, 128, 128, STREAMKL_BF16);
  bad[5] = shape((int64_t)1 << 21, 1, 64, 64, 128, 128, STREAMKL_BF16);
  for (int i = 0; i < 6; ++i) {
    EXPECT(streamkl_fwd(p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, &bad[i], NULL, NULL) != STREAMKL_OK);
    EXPECT(streamkl_fwd_loss(p, p, p, p, 0, 0.f, 0.f, NULL, fp, fp, fp, fp, &bad[i], NULL, NULL) != STREAMKL_OK);
    EXPECT(streamkl_fwd_loss_noalloc(p, p, p, p, 0, 0.f, 0.f, NULL, fp, fp, fp, fp, &bad[i], NULL, NULL) !=
           STREAMKL_OK);
    EXPECT(streamkl_bwd(1, p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, fp, fp, fp, &bad[i], NULL, NULL) != STREAMKL_OK);
    EXPECT(streamkl_bwd_joint(p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, fp, fp, fp, fp, fp, &bad[i], NULL, NULL) !=
           STREAMKL_OK);
    EXPECT(streamkl_fwd_workspace_bytes(&bad[i], 0, NULL) == STREAMKL_INVALID_BYTES);
    EXPECT(streamkl_fwd_loss_workspace_bytes(&bad[i], 0, NULL) == STREAMKL_INVALID_BYTES);
    EXPECT(streamkl_bwd_workspace_bytes(&bad[i], 0, 1, NULL) == STREAMKL_INVALID_BYTES);
    EXPECT(streamkl_fwd_plan(&bad[i], 0, NULL) == 0);
    EXPECT(streamkl_bwd_plan(&bad[i], 0, 1, NULL) == 0);
  }
  EXPECT(streamkl_fwd(p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, NULL, NULL, NULL) == STREAMKL_ERR_INVALID);

  /* null and misaligned pointers, non-finite scales, bad settings and modes */
  EXPECT(streamkl_fwd(NULL, p, p, p, 0, 0.f, 0.f, fp, fp, fp, &good, NULL, NULL) == STREAMKL_ERR_INVALID);
  EXPECT(streamkl_fwd(odd, p, p, p, 0, 0.f, 0.f, fp, fp, fp, &good, NULL, NULL) == STREAMKL_ERR_INVALID);
  EXPECT(streamkl_fwd(p, p, p, p, 0, NAN, 0.f, fp, fp, fp, &good, NULL, NULL) == STREAMKL_ERR_INVALID);
  EXPECT(streamkl_fwd(p, p, p, p, 0, 0.f, INFINITY, fp, fp, fp, &good, NULL, NULL) == STREAMKL_ERR_INVALID);
  EXPECT(streamkl_fwd_loss(p, p, p, p, 0, 0.f, 0.f, (float*)odd, fp, fp, fp, fp, &good, NULL, NULL) ==
         STREAMKL_ERR_INVALID);
  EXPECT(streamkl_bwd(3, p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, fp, fp, fp, &good, NULL, NULL) ==
         STREAMKL_ERR_INVALID);
  EXPECT(streamkl_bwd(2, p, p, p, p, 0, 0.f, 0.f, NULL, fp, fp, fp, fp, fp, &good, NULL, NULL) ==
         STREAMKL_ERR_INVALID);
  EXPECT(streamkl_bwd(1, p, p, p, p, 0, -NAN, 0.f, fp, fp, fp, fp, fp, fp, &good, NULL, NULL) ==
         STREAMKL_ERR_INVALID);
  streamkl_launch bad_mode = {0, 9, NULL, 0};
  EXPECT(streamkl_bwd(1, p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, fp, fp, fp, &good, &bad_mode, NULL) ==
         STREAMKL_ERR_INVALID);
  EXPECT(streamkl_bwd_workspace_bytes(&good, 0, 1, &bad_mode) == STREAMKL_INVALID_BYTES);
  EXPECT(streamkl_bwd_workspace_bytes(&good, 0, 0, NULL) == STREAMKL_INVALID_BYTES);
  EXPECT(streamkl_bwd_workspace_bytes(&good, 1, 2, NULL) == 0);
  EXPECT(streamkl_kl_loss(NULL, NULL, 10, fp, NULL) == STREAMKL_ERR_INVALID);
  EXPECT(streamkl_kl_loss(fp, NULL, 0, fp, NULL) == STREAMKL_ERR_INVALID);

  /* grouped key heads and ragged lengths */
  streamkl_shape g = shape(1, 32, 64, 64, 128, 128, STREAMKL_BF16);
  g.kv_heads1 = 3;
  EXPECT(streamkl_fwd(p, p, p, p, 0, 0.f, 0.f, fp, fp, fp, &g, NULL, NULL) == STREAMKL_ERR_INVALID);
  int64_t ql[3] = {600, 0, 97}, kl[3] = {600, 5, 97}, qbad[3] = {600, 10, 97}, kzero[3] = {600, 0, 97};
  streamkl_shape r = shape(3, 8, 600, 600, 128, 128, STREAMKL_BF16);
  r.q_len = ql; r.k_len = kl;
  EXPECT(streamkl_fwd_workspace_bytes(&r, 1, NULL) != STREAMKL_INVALID_BYTES);
  EXPECT(streamkl_fwd_loss_workspace_bytes(&r, 1, NULL) != STREAMKL_INVALID_BYTES);
  EXPECT(streamkl_fwd_plan(&r, 1, NULL) >= 1);
  r.q_len = qbad; r.k_len = kzero;  /* query rows with no key */
  EXPECT(streamkl_fwd(p, p, p, p, 1, 0.f, 0.f, fp, fp, fp, &r, NULL, NULL) == STREAMKL_ERR_INVALID);
  EXPECT(streamkl_fwd_loss_workspace_bytes(&r, 1, NULL) == STREAMKL_INVALID_BYTES);

  /* packed batches: offsets from 0 to the totals, nondecreasing, both or neither, no lengths beside them */
  int64_t qo[4] = {0, 600, 600, 697}, ko[4] = {0, 600, 605, 702};
  streamkl_shape pk = shape(3, 8, 697, 702, 128, 128, STREAMKL_BF16);
  pk.q_off = qo; pk.k_off = ko;
  EXPECT(streamkl_fwd_workspace_bytes(&pk, 1, NULL) != STREAMKL_INVALID_BYTES);
  EXPECT(streamkl_fwd_loss_workspace_bytes(&pk, 1, NULL) != STREAMKL_INVALID_BYTES);
  EXPECT(streamkl_fwd_plan(&pk, 1, NULL) >= 1);
  pk.n_q = 700;  /* the total rows disagree with the offsets */
  EXPECT(streamkl_fwd(p, p, p, p, 1, 0.f, 0.f, fp, fp, fp, &pk, NULL, NULL) == STREAMKL_ERR_INVALID);
  pk.n_q = 697;
  int64_t qdown[4] = {0, 600, 500, 697};  /* decreasing */
  pk.q_off = qdown;
  EXPECT(streamkl_fwd(p, p, p, p, 1, 0.f, 0.f, fp, fp, fp, &pk, NULL, NULL) == STREAMKL_ERR_INVALID);
  pk.q_off = qo;
  pk.k_off = NULL;  /* one without the other */
  EXPECT(streamkl_fwd_workspace_bytes(&pk, 1, NULL) == STREAMKL_INVALID_BYTES);
  pk.k_off = ko;
  pk.q_len = ql;  /* lengths beside offsets */
  EXPECT(streamkl_fwd_workspace_bytes(&pk, 1, NULL) == STREAMKL_INVALID_BYTES);
  pk.q_len = NULL;
  int64_t kshort[4] = {0, 600, 605, 605};  /* element 2: 97 query rows, no key */
  pk.k_off = kshort;
  pk.n_k = 605;
  EXPECT(streamkl_fwd_workspace_bytes(&pk, 0, NULL) == STREAMKL_INVALID_BYTES);

  /* planning and sizing of valid shapes (no device: the planner assumes 256 compute units) */
  streamkl_shape dec = shape(1, 32, 16, 131072, 128, 128, STREAMKL_BF16);
  size_t ws = streamkl_fwd_workspace_bytes(&dec, 0, NULL);
  size_t wl = streamkl_fwd_loss_workspace_bytes(&dec, 0, NULL);
  EXPECT(ws > 0 && wl > ws);
  streamkl_launch withws = {0, 0, p, ws};
  EXPECT(streamkl_fwd_plan(&dec, 0, &withws) > 1);
  EXPECT(streamkl_fwd_plan(&dec, 0, NULL) == 1);
  streamkl_shape big = shape(1, 32, 65536, 65536, 128, 128, STREAMKL_BF16);
  EXPECT(streamkl_fwd_workspace_bytes(&big, 1, NULL) == 0);
  EXPECT(streamkl_fwd_loss_workspace_bytes(&big, 1, NULL) == 8u * 32u * 256u);
  EXPECT(streamkl_bwd_plan(&big, 1, 1, NULL) == STREAMKL_BWD_SEPARATE);
  EXPECT(streamkl_bwd_plan(&dec, 0, 1, NULL) == STREAMKL_BWD_FUSED);
  for (int st = 0; st < 6; ++st) EXPECT(streamkl_status_string(st) != NULL);
  EXPECT(streamkl_version() == 5);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks passed\n");
  return 0;
}
