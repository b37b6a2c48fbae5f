/* Calls libcq's host-only entry points from C through include/libcq.h (no
 * GPU needed) and prints the results, one "key value..." line each. */
#include <stdint.h>
#include <stdio.h>

#include "libcq.h"

int main(void) {
  printf("version %s\n", cq_version());
  int64_t ng = 0, pb = 0;
  int rc = cq_layout(300, 1000, 2, 128, &ng, &pb);
  printf("layout %d %lld %lld\n", rc, (long long)ng, (long long)pb);
  const int64_t rows[3] = {4096, 300, 2};
  const int64_t cols[3] = {4096, 1000, 130};
  uint64_t bytes = 0;
  rc = cq_model_bytes(3, rows, cols, 2, 128, &bytes);
  printf("model_bytes %d %llu\n", rc, (unsigned long long)bytes);
  rc = cq_model_bytes(3, rows, cols, CQ_TERNARY_TRITS, 128, &bytes);
  printf("model_bytes_trits %d %llu\n", rc, (unsigned long long)bytes);
  int64_t po[3], no[3], total = 0;
  rc = cq_blob_layout(3, rows, cols, 2, 128, po, no, &total);
  printf("blob %d %lld %lld %lld %lld %lld %lld %lld\n", rc, (long long)po[0], (long long)po[1],
         (long long)po[2], (long long)no[0], (long long)no[1], (long long)no[2], (long long)total);
  float lv[CQ_MAX_LEVELS];
  int n = 0;
  rc = cq_codebook(CQ_TERNARY, lv, &n);
  printf("ternary %d %d %.7f %.7f %.7f\n", rc, n, lv[0], lv[1], lv[2]);
  rc = cq_codebook(2, lv, &n);
  printf("builtin2 %d %d %.7f %.7f %.7f %.7f\n", rc, n, lv[0], lv[1], lv[2], lv[3]);
  const double samples[4] = {-2.0, -1.0, 1.0, 3.0};
  rc = cq_codebook_train(1, samples, 4, 10, lv, &n);
  printf("lloyd1 %d %d %.7f %.7f\n", rc, n, lv[0], lv[1]);
  /* validation errors come back before any device work */
  rc = cq_quantize(NULL, CQ_F32, 4, 256, 5, 128, lv, 4, NULL, NULL, NULL);
  printf("bad_bits %d %s\n", rc, cq_status_str(rc));
  const float lv4[4] = {-1.5f, -0.45f, 0.45f, 1.5f};
  rc = cq_dequant_matvec(NULL, NULL, 8, 200, 2, 128, lv4, 4, NULL, 1, NULL, NULL);
  printf("bad_k %d\n", rc);
  return 0;
}
