/* A C11 program that drives one synchronisation through the reducer's C ABI
 * on the GPU, with no Python or torch in the data path. Built and run by
 * tests/test_gpu_c_abi.py, which writes the inputs and compares the outputs
 * with the oracle's; this program only moves data through the library.
 *
 *   abi_gpu <input file> <output file>
 *
 * Input (little-endian): int32 magic 0x44445042, int32 P, int32 R, int32 mode
 * (DDPB_MODE_FUSED or DDPB_MODE_STAGED, plus 2 to bind with ddpb_bind_static,
 * which allocates nothing and reduces on the compute stream), int64 cap, int64 numel[P], int32 n,
 * int32 order[n] (the hooks, in firing order), then float32 gradients of
 * replica 0 variable 0, replica 0 variable 1, ... replica R-1 variable P-1.
 * Output: the gradients after ddpb_finalize in the same layout, then int32 m
 * and m (bucket, trigger call) int32 pairs of the launch log. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ddpb.h"

#define HIPCHECK(x)                                                              \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
      return 2;                                                                  \
    }                                                                            \
  } while (0)

#define DDPBCHECK(x)                                                             \
  do {                                                                           \
    int rc_ = (x);                                                               \
    if (rc_ != DDPB_OK) {                                                        \
      fprintf(stderr, "%s failed: %d (%s)\n", #x, rc_, ddpb_last_error());       \
      return 3;                                                                  \
    }                                                                            \
  } while (0)

static int read_all(FILE* f, void* p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: abi_gpu <input> <output>\n");
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 1;
  int32_t magic = 0, P = 0, R = 0, mode = 0, n = 0;
  int64_t cap = 0;
  if (!read_all(in, &magic, 4) || magic != 0x44445042 || !read_all(in, &P, 4) || !read_all(in, &R, 4) ||
      !read_all(in, &mode, 4) || !read_all(in, &cap, 8) || P < 1 || P > 4096 || R < 1 || R > 64 ||
      mode < 0 || mode > 3) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const int use_static = (mode & 2) != 0;
  mode &= 1;
  int64_t* numel = malloc(sizeof(int64_t) * (size_t)P);
  int32_t* ndims = malloc(sizeof(int32_t) * (size_t)P);
  if (!numel || !ndims || !read_all(in, numel, sizeof(int64_t) * (size_t)P) || !read_all(in, &n, 4) || n < 0 ||
      n > P) {
    fprintf(stderr, "bad sizes\n");
    return 1;
  }
  int64_t total = 0;
  for (int32_t v = 0; v < P; ++v) {
    if (numel[v] < 0 || numel[v] > (1 << 26)) return 1;
    ndims[v] = 1;
    total += numel[v];
  }
  int32_t* order = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!order || !read_all(in, order, sizeof(int32_t) * (size_t)n)) return 1;
  for (int32_t i = 0; i < n; ++i)
    if (order[i] < 0 || order[i] >= P) return 1;
  float* host = malloc(sizeof(float) * (size_t)(total > 0 ? total : 1) * (size_t)R);
  if (!host || !read_all(in, host, sizeof(float) * (size_t)total * (size_t)R)) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  fclose(in);

  ddpb_t h = NULL;
  DDPBCHECK(ddpb_reducer_create(numel, ndims, P, DDPB_F32, cap, R, &h));

  /* one device allocation per replica and variable, as separate .grad fields are */
  void** grads = malloc(sizeof(void*) * (size_t)R * (size_t)P);
  if (!grads) return 1;
  int64_t at = 0;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t v = 0; v < P; ++v) {
      const size_t bytes = sizeof(float) * (size_t)numel[v];
      HIPCHECK(hipMalloc(&grads[(size_t)r * P + v], bytes > 0 ? bytes : 4));
      if (bytes) HIPCHECK(hipMemcpy(grads[(size_t)r * P + v], host + at, bytes, hipMemcpyHostToDevice));
      at += numel[v];
    }
  hipStream_t compute, side[2];
  HIPCHECK(hipStreamCreate(&compute));
  HIPCHECK(hipStreamCreate(&side[0]));
  HIPCHECK(hipStreamCreate(&side[1]));
  int64_t ws_bytes = 0;
  void* ws = NULL;
  if (use_static) {
    DDPBCHECK(ddpb_bind_static(h, grads, compute, mode));  /* no workspace, nothing allocated */
  } else {
    DDPBCHECK(ddpb_workspace_bytes(h, mode, &ws_bytes));
    if (ws_bytes > 0) HIPCHECK(hipMalloc(&ws, (size_t)ws_bytes));
    void* sides[2] = {side[0], side[1]};
    DDPBCHECK(ddpb_bind(h, grads, ws, ws_bytes, compute, sides, 2, mode, 0));
  }
  for (int32_t i = 0; i < n; ++i) DDPBCHECK(ddpb_mark_ready(h, order[i]));
  DDPBCHECK(ddpb_finalize(h));
  HIPCHECK(hipStreamSynchronize(compute));

  at = 0;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t v = 0; v < P; ++v) {
      const size_t bytes = sizeof(float) * (size_t)numel[v];
      if (bytes) HIPCHECK(hipMemcpy(host + at, grads[(size_t)r * P + v], bytes, hipMemcpyDeviceToHost));
      at += numel[v];
    }
  int32_t m = 0;
  DDPBCHECK(ddpb_get_launch_log(h, NULL, NULL, NULL, NULL, 0, &m));
  int32_t* lb = malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
  int32_t* lt = malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
  if (!lb || !lt) return 1;
  DDPBCHECK(ddpb_get_launch_log(h, lb, lt, NULL, NULL, m, &m));

  FILE* out = fopen(argv[2], "wb");
  if (!out) return 1;
  fwrite(host, sizeof(float), (size_t)total * (size_t)R, out);
  fwrite(&m, 4, 1, out);
  for (int32_t i = 0; i < m; ++i) {
    fwrite(&lb[i], 4, 1, out);
    fwrite(&lt[i], 4, 1, out);
  }
  fclose(out);

  ddpb_destroy(h);
  for (size_t i = 0; i < (size_t)R * (size_t)P; ++i) HIPCHECK(hipFree(grads[i]));
  if (ws) HIPCHECK(hipFree(ws));
  HIPCHECK(hipStreamDestroy(compute));
  HIPCHECK(hipStreamDestroy(side[0]));
  HIPCHECK(hipStreamDestroy(side[1]));
  free(grads);
  free(host);
  free(order);
  free(ndims);
  free(numel);
  free(lb);
  free(lt);
  return 0;
}
