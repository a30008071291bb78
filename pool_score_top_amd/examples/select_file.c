/*
 * select_file - the whole k-pool selection through the C ABI, with plain HIP
 * runtime calls and no framework: pool the keys, score and select every row,
 * expand to token ids.
 *
 *     select_file IN OUT
 *
 * IN, little-endian:
 *   int32 T, H, D, kpool, budget, nseq
 *   int32 cu_seqlens[nseq + 1]
 *   uint16 q[T * H * D]   bf16 bit patterns, row-major [T, H, D]
 *   uint16 k[T * D]       bf16 bit patterns, row-major [T, D]
 *   float  w[T * H]       row-major [T, H]
 * OUT:
 *   int32 pool_ids[T * budget], then int32 token_ids[T * budget * kpool]
 *
 * The scale is 1/sqrt(D) in fp32 and the workspace is the library's default
 * size for all rows (one chunk buffer).  Exit status 0 on success, 1 on a
 * library or HIP error (the message goes to stderr), 2 on bad usage or input.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "../../include/kpool.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

#define KPOOL_OK_OR_EXIT(call)                                                    \
  do {                                                                            \
    int rc_ = (call);                                                             \
    if (rc_ != KPOOL_OK) {                                                        \
      fprintf(stderr, "%s failed (%d): %s\n", #call, rc_, kpool_last_error());    \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

static void *read_or_exit(FILE *f, size_t bytes) {
  void *p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    exit(2);
  }
  return p;
}

static void *device_copy(const void *host, size_t bytes) {
  void *d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE *in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  int32_t hdr[6];
  if (fread(hdr, sizeof hdr, 1, in) != 1) {
    fprintf(stderr, "short input file\n");
    return 2;
  }
  const int32_t T = hdr[0], H = hdr[1], D = hdr[2], kpool = hdr[3], budget = hdr[4], nseq = hdr[5];
  if (T < 1 || H < 1 || D < 1 || kpool < 1 || budget < 1 || nseq < 1) {
    fprintf(stderr, "bad header\n");
    return 2;
  }
  int32_t *cu = (int32_t *)read_or_exit(in, sizeof(int32_t) * (size_t)(nseq + 1));
  uint16_t *q = (uint16_t *)read_or_exit(in, sizeof(uint16_t) * (size_t)T * H * D);
  uint16_t *k = (uint16_t *)read_or_exit(in, sizeof(uint16_t) * (size_t)T * D);
  float *w = (float *)read_or_exit(in, sizeof(float) * (size_t)T * H);
  fclose(in);

  /* pools per sequence (host), then device copies of everything */
  int32_t *cu_pools = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nseq + 1));
  int32_t max_pools = 0;
  const int64_t P = kpool_count_pools(cu, nseq, kpool, 0u, cu_pools, &max_pools);
  if (P < 0) {
    fprintf(stderr, "kpool_count_pools failed (%lld): %s\n", (long long)P, kpool_last_error());
    return 1;
  }
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  void *q_d = device_copy(q, sizeof(uint16_t) * (size_t)T * H * D);
  void *k_d = device_copy(k, sizeof(uint16_t) * (size_t)T * D);
  void *w_d = device_copy(w, sizeof(float) * (size_t)T * H);
  void *cu_d = device_copy(cu, sizeof(int32_t) * (size_t)(nseq + 1));
  void *cup_d = device_copy(cu_pools, sizeof(int32_t) * (size_t)(nseq + 1));
  void *kp_d = NULL, *ids_d = NULL, *tok_d = NULL, *ws_d = NULL;
  HIP_OK(hipMalloc(&kp_d, sizeof(uint16_t) * (size_t)(P ? P : 1) * D));
  HIP_OK(hipMalloc(&ids_d, sizeof(int32_t) * (size_t)T * budget));
  HIP_OK(hipMalloc(&tok_d, sizeof(int32_t) * (size_t)T * budget * kpool));
  const size_t ws_bytes = max_pools > 0 ? kpool_workspace_bytes(0, T, max_pools, 1) : 0;
  HIP_OK(hipMalloc(&ws_d, ws_bytes ? ws_bytes : 16));

  /* the three steps, in order on one stream */
  KPOOL_OK_OR_EXIT(kpool_pool_keys((const uint16_t *)k_d, cu, (const int32_t *)cu_d,
                                   (const int32_t *)cup_d, nseq, D, kpool, 0u, (uint16_t *)kp_d,
                                   (void *)stream));
  const float scale = 1.0f / sqrtf((float)D);
  KPOOL_OK_OR_EXIT(kpool_score_topk((const uint16_t *)q_d, (const uint16_t *)kp_d, (const float *)w_d,
                                    cu, (const int32_t *)cu_d, nseq, H, D, kpool, scale, 0, T, budget,
                                    ws_d, ws_bytes, 0u, (int32_t *)ids_d, NULL, (void *)stream));
  KPOOL_OK_OR_EXIT(kpool_expand((const int32_t *)ids_d, cu, (const int32_t *)cu_d, nseq, kpool, 0, T,
                                budget, 0u, (int32_t *)tok_d, (void *)stream));
  HIP_OK(hipStreamSynchronize(stream));

  const size_t n_ids = (size_t)T * budget, n_tok = (size_t)T * budget * kpool;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * n_ids);
  int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * n_tok);
  HIP_OK(hipMemcpy(ids, ids_d, sizeof(int32_t) * n_ids, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(tok, tok_d, sizeof(int32_t) * n_tok, hipMemcpyDeviceToHost));
  FILE *out = fopen(argv[2], "wb");
  if (!out || fwrite(ids, sizeof(int32_t), n_ids, out) != n_ids ||
      fwrite(tok, sizeof(int32_t), n_tok, out) != n_tok || fclose(out) != 0) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 2;
  }

  void *bufs[] = {q_d, k_d, w_d, cu_d, cup_d, kp_d, ids_d, tok_d, ws_d};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
  HIP_OK(hipStreamDestroy(stream));
  free(cu);
  free(q);
  free(k);
  free(w);
  free(cu_pools);
  free(ids);
  free(tok);
  return 0;
}
