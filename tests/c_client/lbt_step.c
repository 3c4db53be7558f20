/* A plain C99 client of include/lbt.h: one pass of the path (route, plan,
 * align, dispatch, combine with the identity expert) on device buffers it
 * allocates with the HIP runtime, driven without Python or torch.  Test
 * infrastructure: the GPU tests write its input file, run it and compare
 * what it writes back with the oracle.
 *
 *   lbt_step IN OUT
 *
 * IN  (little-endian): int32 E, K, R, S, H, B, blk, score_fn; then fp32
 *     logits [N][E]; then bf16 bits x [N][H]  (N = R*S).
 * OUT: int64 N, P, C, n_blocks, plan_words; then int32 ids [N][K]; fp32
 *      gates [N][K]; int32 counts [R][E]; int32 plan [plan_words]; int32
 *      slot [P]; int32 sorted_ids [R*C]; int32 block_wrow [R][n_blocks];
 *      int32 block_expert [R][n_blocks]; int32 status; fp32 y [N][H];
 *      bf16 bits recv [R*C][H].
 * Exit status: 0 ok, 1 usage or file error, 2 HIP error, 3 library error
 * (the message names the call). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lbt.h"

#define HIP_CHECK(call)                                                          \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));          \
      return 2;                                                                  \
    }                                                                            \
  } while (0)

#define LBT_CHECK(call)                                                          \
  do {                                                                           \
    int r_ = (call);                                                             \
    if (r_ != LBT_OK) {                                                          \
      fprintf(stderr, "%s failed: %s%s%s\n", #call, lbt_strerror(r_),             \
              r_ == LBT_EHIP ? ", " : "", r_ == LBT_EHIP ? lbt_last_hip_error() : ""); \
      return 3;                                                                  \
    }                                                                            \
  } while (0)

/* Device and host buffers of one output array. */
typedef struct {
  void* dev;
  void* host;
  size_t bytes;
} buffer;

static int alloc_pair(buffer* b, size_t bytes) {
  b->bytes = bytes;
  b->host = malloc(bytes > 0 ? bytes : 1);
  if (b->host == NULL) return 1;
  /* at least one word, so that every call gets a valid pointer */
  return hipMalloc(&b->dev, bytes > 16 ? bytes : 16) != hipSuccess;
}

static int read_all(FILE* f, void* p, size_t bytes) {
  return fread(p, 1, bytes, f) != bytes;
}

static int write_all(FILE* f, const void* p, size_t bytes) {
  return fwrite(p, 1, bytes, f) != bytes;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[8];
  if (read_all(in, hdr, sizeof hdr)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  lbt_shape s;
  memset(&s, 0, sizeof s);
  s.E = hdr[0];
  s.K = hdr[1];
  s.R = hdr[2];
  s.S = hdr[3];
  s.H = hdr[4];
  s.B = hdr[5];
  s.blk = hdr[6];
  s.score_fn = hdr[7];
  lbt_sizes z;
  LBT_CHECK(lbt_query_sizes(&s, &z));
  const int64_t N = z.N, P = z.P, C = z.C, nb = z.n_blocks;
  const int64_t E = s.E, K = s.K, R = s.R, H = s.H;

  buffer logits, x, ids, gates, counts, work, plan, status, slot, sorted_ids, bw, be, recv, y;
  if (alloc_pair(&logits, (size_t)(N * E) * 4) || alloc_pair(&x, (size_t)(N * H) * 2) ||
      alloc_pair(&ids, (size_t)(N * K) * 4) || alloc_pair(&gates, (size_t)(N * K) * 4) ||
      alloc_pair(&counts, (size_t)(R * E) * 4) || alloc_pair(&work, (size_t)z.work_words * 4) ||
      alloc_pair(&plan, (size_t)z.plan_words * 4) || alloc_pair(&status, 4) ||
      alloc_pair(&slot, (size_t)P * 4) || alloc_pair(&sorted_ids, (size_t)(R * C) * 4) ||
      alloc_pair(&bw, (size_t)(R * nb) * 4) || alloc_pair(&be, (size_t)(R * nb) * 4) ||
      alloc_pair(&recv, (size_t)(R * C * H) * 2) || alloc_pair(&y, (size_t)(N * H) * 4)) {
    fprintf(stderr, "allocation failed\n");
    return 2;
  }
  if (read_all(in, logits.host, logits.bytes) || read_all(in, x.host, x.bytes)) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  fclose(in);

  HIP_CHECK(hipMemcpy(logits.dev, logits.host, logits.bytes, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(x.dev, x.host, x.bytes, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemset(status.dev, 0, 4));

  /* one pass on the default stream; no call synchronises the host */
  LBT_CHECK(lbt_route_topk(&s, (const float*)logits.dev, NULL, (int32_t*)ids.dev,
                           (float*)gates.dev, (int32_t*)counts.dev, (int32_t*)work.dev, NULL));
  LBT_CHECK(lbt_plan_balance(&s, (const int32_t*)counts.dev, (int32_t*)plan.dev,
                             (int32_t*)status.dev, NULL));
  LBT_CHECK(lbt_align_sort(&s, (const int32_t*)ids.dev, (const int32_t*)work.dev,
                           (const int32_t*)plan.dev, (int32_t*)slot.dev, (int32_t*)sorted_ids.dev,
                           (int32_t*)bw.dev, (int32_t*)be.dev, (int32_t*)status.dev, NULL));
  LBT_CHECK(lbt_dispatch(&s, (const uint16_t*)x.dev, (const int32_t*)slot.dev,
                         (uint16_t*)recv.dev, NULL));
  LBT_CHECK(lbt_combine(&s, (const uint16_t*)recv.dev, (const int32_t*)slot.dev,
                        (const float*)gates.dev, LBT_Y_F32, y.dev, NULL));
  HIP_CHECK(hipDeviceSynchronize());

  buffer* outs[] = {&ids, &gates, &counts, &plan, &slot, &sorted_ids, &bw, &be, &status, &y, &recv};
  const size_t n_outs = sizeof outs / sizeof outs[0];
  for (size_t i = 0; i < n_outs; ++i)
    HIP_CHECK(hipMemcpy(outs[i]->host, outs[i]->dev, outs[i]->bytes, hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) {
    perror(argv[2]);
    return 1;
  }
  const int64_t sizes[5] = {N, P, C, nb, z.plan_words};
  int bad = write_all(out, sizes, sizeof sizes);
  for (size_t i = 0; i < n_outs; ++i) bad |= write_all(out, outs[i]->host, outs[i]->bytes);
  bad |= fclose(out) != 0;
  if (bad) {
    fprintf(stderr, "write failed\n");
    return 1;
  }
  buffer* all[] = {&logits, &x, &ids, &gates, &counts, &work, &plan, &status, &slot, &sorted_ids,
                   &bw, &be, &recv, &y};
  for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) {
    HIP_CHECK(hipFree(all[i]->dev));
    free(all[i]->host);
  }
  return 0;
}
