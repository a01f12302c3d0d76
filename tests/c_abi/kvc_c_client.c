/* kvc_c_client.c -- a plain C consumer of libkvc: plans and compresses a
 * ragged pool-16 batch through the C ABI alone (HIP runtime for memory and a
 * stream; no Python, no torch), so the tests can show the boundary stands on
 * its own.
 *
 * usage: kvc_c_client DIR
 *   reads  DIR/seq_lens.i64 (int64 [B]), DIR/keys.u16 and DIR/scores.u16
 *          (bf16 bit patterns [T,128], rows packed by sequence),
 *          DIR/ape.f32 (fp32 [16,128])
 *   writes DIR/rows.i32 (pool start rows), DIR/codes.u8 (e4m3 [n,128]),
 *          DIR/scales.f32 ([n], power-of-two scales), DIR/pooled.f32
 *          (fp32 [n,128] means before the bf16 rounding)
 * Exit status 0 on success; 1 usage / file errors, 2 HIP errors, 3 library
 * errors (the library's message is printed). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvc.h"

static void* read_file(const char* dir, const char* name, size_t* bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* p = malloc(n > 0 ? (size_t)n : 1);
  if (p && n > 0 && fread(p, 1, (size_t)n, f) != (size_t)n) {
    free(p);
    p = NULL;
  }
  fclose(f);
  *bytes = n > 0 ? (size_t)n : 0;
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  const int ok = fwrite(p, 1, bytes, f) == bytes;
  return fclose(f) == 0 && ok;
}

#define HIP_CHECK(x)                                                     \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      return 2;                                                          \
    }                                                                    \
  } while (0)

#define KVC_CHECK(x)                                                     \
  do {                                                                   \
    int r_ = (x);                                                        \
    if (r_ != KVC_OK) {                                                  \
      fprintf(stderr, "%s: status %d: %s\n", #x, r_, kvc_last_error());  \
      return 3;                                                          \
    }                                                                    \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  size_t b_sl, b_k, b_s, b_a;
  int64_t* seq_lens = (int64_t*)read_file(dir, "seq_lens.i64", &b_sl);
  uint16_t* keys = (uint16_t*)read_file(dir, "keys.u16", &b_k);
  uint16_t* scores = (uint16_t*)read_file(dir, "scores.u16", &b_s);
  float* ape = (float*)read_file(dir, "ape.f32", &b_a);
  if (!seq_lens || !keys || !scores || !ape || b_sl % 8 || b_k % 256 || b_k != b_s ||
      b_a != 16 * 128 * 4) {
    fprintf(stderr, "missing or malformed input files in %s\n", dir);
    return 1;
  }
  const int64_t batch = (int64_t)(b_sl / 8), rows_total = (int64_t)(b_k / 256);

  /* host planner: the first row of every complete pool */
  int64_t cap = 0, n = 0;
  for (int64_t b = 0; b < batch; ++b) cap += seq_lens[b] > 0 ? seq_lens[b] / 16 : 0;
  int32_t* rows = (int32_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int32_t));
  KVC_CHECK(kvc_plan_pool_prefill(seq_lens, batch, 16, rows, cap, &n));

  void *d_keys, *d_scores, *d_ape, *d_rows, *d_codes, *d_scales, *d_pooled;
  const size_t nn = (size_t)(n > 0 ? n : 1);
  HIP_CHECK(hipMalloc(&d_keys, b_k));
  HIP_CHECK(hipMalloc(&d_scores, b_s));
  HIP_CHECK(hipMalloc(&d_ape, b_a));
  HIP_CHECK(hipMalloc(&d_rows, nn * 4));
  HIP_CHECK(hipMalloc(&d_codes, nn * 128));
  HIP_CHECK(hipMalloc(&d_scales, nn * 4));
  HIP_CHECK(hipMalloc(&d_pooled, nn * 128 * 4));
  HIP_CHECK(hipMemcpy(d_keys, keys, b_k, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_scores, scores, b_s, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_ape, ape, b_a, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_rows, rows, (size_t)n * 4, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));
  KVC_CHECK(kvc_compress_prefill((const uint16_t*)d_keys, 128, (const uint16_t*)d_scores, 128,
                                 rows_total, (const float*)d_ape, 16, (const int32_t*)d_rows, n,
                                 (uint8_t*)d_codes, (float*)d_scales, 1, (float*)d_pooled,
                                 stream));
  HIP_CHECK(hipStreamSynchronize(stream));

  uint8_t* codes = (uint8_t*)malloc(nn * 128);
  float* scales = (float*)malloc(nn * 4);
  float* pooled = (float*)malloc(nn * 128 * 4);
  HIP_CHECK(hipMemcpy(codes, d_codes, (size_t)n * 128, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(scales, d_scales, (size_t)n * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(pooled, d_pooled, (size_t)n * 128 * 4, hipMemcpyDeviceToHost));
  if (!write_file(dir, "rows.i32", rows, (size_t)n * 4) ||
      !write_file(dir, "codes.u8", codes, (size_t)n * 128) ||
      !write_file(dir, "scales.f32", scales, (size_t)n * 4) ||
      !write_file(dir, "pooled.f32", pooled, (size_t)n * 128 * 4)) {
    fprintf(stderr, "cannot write outputs to %s\n", dir);
    return 1;
  }
  HIP_CHECK(hipStreamDestroy(stream));
  HIP_CHECK(hipFree(d_keys));
  HIP_CHECK(hipFree(d_scores));
  HIP_CHECK(hipFree(d_ape));
  HIP_CHECK(hipFree(d_rows));
  HIP_CHECK(hipFree(d_codes));
  HIP_CHECK(hipFree(d_scales));
  HIP_CHECK(hipFree(d_pooled));
  free(seq_lens);
  free(keys);
  free(scores);
  free(ape);
  free(rows);
  free(codes);
  free(scales);
  free(pooled);
  printf("kvc_c_client: %lld pools from %lld rows\n", (long long)n, (long long)rows_total);
  return 0;
}
