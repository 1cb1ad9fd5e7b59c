/* A C11 caller of the reducer's C ABI, built and run by tests/test_host_c_abi.py
 * against the host-only library (same plan and state machine, a launcher that
 * enqueues nothing), so no GPU is needed. It checks that the header is valid
 * C and that the entry points behave as documented for a small model:
 * nn.Linear(10, 10) (bias 10, weight 100) plus a 2 x 3 x 4 tensor, and the
 * same three shapes with a cap that puts each in its own bucket. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ddpb.h"

static int failures = 0;

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond);  \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

int main(void) {
  /* v0 = bias [10], v1 = weight [10, 10], v2 = [2, 3, 4] */
  const int64_t shapes[] = {10, 10, 10, 2, 3, 4};
  const int32_t ndims[] = {1, 2, 3};
  ddpb_t h = NULL;

  /* argument errors leave no handle behind */
  CHECK(ddpb_reducer_create(shapes, ndims, 3, DDPB_F32, -1, 2, &h) == DDPB_E_ARG);
  CHECK(ddpb_reducer_create(shapes, ndims, 3, DDPB_F32, 1024, 0, &h) == DDPB_E_ARG);
  CHECK(strlen(ddpb_last_error()) > 0);

  /* one bucket: the cap (25 MiB) is never reached; members in reverse order */
  CHECK(ddpb_reducer_create(shapes, ndims, 3, DDPB_F32, 25 << 20, 2, &h) == DDPB_OK);
  int32_t B = -1;
  CHECK(ddpb_num_buckets(h, &B) == DDPB_OK && B == 1);
  int32_t nvars = 0, vars[3] = {-1, -1, -1};
  int64_t bytes = 0;
  CHECK(ddpb_get_bucket(h, 0, &nvars, &bytes, vars) == DDPB_OK);
  CHECK(nvars == 3 && bytes == 4 * (10 + 100 + 24));
  CHECK(vars[0] == 2 && vars[1] == 1 && vars[2] == 0);
  int32_t bucket = -1, intra = -1;
  int64_t offset = -1, length = -1;
  CHECK(ddpb_get_locator(h, 0, &bucket, &intra, &offset, &length) == DDPB_OK);
  CHECK(bucket == 0 && intra == 2 && offset == 24 + 100 && length == 10);
  CHECK(ddpb_get_locator(h, 3, &bucket, &intra, &offset, &length) == DDPB_E_INDEX);

  /* bind fake device pointers (the host-only launcher never reads them) */
  void* grads[6];
  for (int i = 0; i < 6; ++i) grads[i] = (void*)(uintptr_t)(0x10000 + 0x1000 * i);
  void* side[1] = {(void*)0};
  CHECK(ddpb_mark_ready(h, 0) == DDPB_E_STATE);                 /* not bound yet */
  CHECK(ddpb_bind(h, grads, NULL, 0, NULL, side, 1, DDPB_MODE_FUSED, 0) == DDPB_OK);

  /* one iteration: the bucket launches at the third hook */
  CHECK(ddpb_mark_ready(h, 2) == DDPB_OK);
  CHECK(ddpb_mark_ready(h, 2) == DDPB_E_DOUBLE_READY);
  CHECK(ddpb_mark_ready(h, 1) == DDPB_OK);
  CHECK(ddpb_mark_ready(h, 7) == DDPB_E_INDEX);
  CHECK(ddpb_mark_ready(h, 0) == DDPB_OK);
  int32_t lb[4], trig[4], n = -1;
  CHECK(ddpb_get_launch_log(h, lb, trig, NULL, NULL, 4, &n) == DDPB_OK);
  CHECK(n == 1 && lb[0] == 0 && trig[0] == 2);
  CHECK(ddpb_finalize(h) == DDPB_OK);

  /* an iteration left open is caught at the next forward, latched until reset */
  CHECK(ddpb_mark_ready(h, 1) == DDPB_OK);
  CHECK(ddpb_finalize(h) == DDPB_E_INCOMPLETE);
  CHECK(ddpb_ensure_prior_reduction_finished(h) == DDPB_E_INCOMPLETE);
  CHECK(ddpb_mark_ready(h, 2) == DDPB_E_INCOMPLETE);
  CHECK(ddpb_reset(h) == DDPB_OK);
  CHECK(ddpb_ensure_prior_reduction_finished(h) == DDPB_OK);

  /* no_sync: hooks are no-ops, finalize has nothing to do */
  CHECK(ddpb_set_sync(h, 0) == DDPB_OK);
  CHECK(ddpb_mark_ready(h, 0) == DDPB_OK);
  CHECK(ddpb_finalize(h) == DDPB_OK);
  CHECK(ddpb_set_sync(h, 1) == DDPB_OK);
  ddpb_destroy(h);

  /* cap 0: one bucket per tensor; hooks out of order park buckets */
  h = NULL;
  CHECK(ddpb_reducer_create(shapes, ndims, 3, DDPB_F32, 0, 2, &h) == DDPB_OK);
  CHECK(ddpb_num_buckets(h, &B) == DDPB_OK && B == 3);
  CHECK(ddpb_bind(h, grads, NULL, 0, NULL, side, 1, DDPB_MODE_FUSED, 0) == DDPB_OK);
  CHECK(ddpb_mark_ready(h, 0) == DDPB_OK);    /* bucket 2: parked */
  CHECK(ddpb_mark_ready(h, 1) == DDPB_OK);    /* bucket 1: parked */
  CHECK(ddpb_mark_ready(h, 2) == DDPB_OK);    /* bucket 0, then 1 and 2 */
  CHECK(ddpb_get_launch_log(h, lb, trig, NULL, NULL, 4, &n) == DDPB_OK);
  CHECK(n == 3 && lb[0] == 0 && lb[1] == 1 && lb[2] == 2);
  CHECK(trig[0] == 2 && trig[1] == 2 && trig[2] == 2);
  CHECK(ddpb_finalize(h) == DDPB_OK);

  /* the allocation-free binding: argument checks, then a sync; the calls that
     need pinned staging are refused on it */
  void* null_grads[6] = {0};
  CHECK(ddpb_bind_static(h, grads, NULL, 5) == DDPB_E_ARG);            /* bad mode */
  CHECK(ddpb_bind_static(h, null_grads, NULL, DDPB_MODE_FUSED) == DDPB_E_ARG);
  CHECK(ddpb_bind_static(NULL, grads, NULL, DDPB_MODE_FUSED) == DDPB_E_ARG);
  CHECK(ddpb_bind_static(h, grads, NULL, DDPB_MODE_STAGED) == DDPB_OK);
  CHECK(ddpb_no_sync_accumulate(h, grads, DDPB_F32, 1) == DDPB_E_STATE);
  uint8_t used[6] = {1, 1, 1, 1, 1, 1};
  CHECK(ddpb_set_local_used(h, used) == DDPB_E_STATE);
  CHECK(ddpb_mark_ready(h, 2) == DDPB_OK && ddpb_mark_ready(h, 1) == DDPB_OK && ddpb_mark_ready(h, 0) == DDPB_OK);
  CHECK(ddpb_finalize(h) == DDPB_OK);
  ddpb_destroy(h);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("c abi ok\n");
  return 0;
}
