/*
 * c_abi_demo.c - a plain C consumer of the exact-attention library (no C++, no Python, no
 * torch): it allocates device memory with the HIP runtime, fills seeded inputs, calls attn_fwd
 * and attn_fwd_varlen through include/exact_attn.h, checks one error path, and writes inputs
 * and outputs to a directory so that they can be compared with a reference.
 *
 *   c_abi_demo OUT_DIR        exit status 0 on success
 *
 * Files written per case NAME: NAME.bin (the arrays below, back to back, little-endian) and
 * NAME.json (shapes, arguments and the byte offset of each array).  Inputs are bf16 values
 * drawn from a 32-bit linear congruential generator (multiplier 1664525, increment 1013904223)
 * as uniform floats in [-2, 2), rounded to bf16 (round to nearest even).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "exact_attn.h"

static uint32_t lcg_next(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return *s;
}

/* float -> bf16 bits, round to nearest even (inputs are finite) */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void fill(uint16_t* p, size_t n, uint32_t seed) {
  uint32_t s = seed;
  for (size_t i = 0; i < n; ++i) {
    const float u = (float)(lcg_next(&s) >> 8) * (1.0f / 16777216.0f); /* [0, 1) */
    p[i] = to_bf16(4.0f * u - 2.0f);
  }
}

#define CHECK_HIP(x)                                                       \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      exit(2);                                                             \
    }                                                                      \
  } while (0)

typedef struct {
  FILE* bin;
  FILE* js;
  long offset;
  int first;
} Out;

static void out_open(Out* o, const char* dir, const char* name) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  o->bin = fopen(path, "wb");
  snprintf(path, sizeof path, "%s/%s.json", dir, name);
  o->js = fopen(path, "w");
  if (!o->bin || !o->js) {
    fprintf(stderr, "cannot write to %s\n", dir);
    exit(3);
  }
  o->offset = 0;
  o->first = 1;
  fprintf(o->js, "{\"arrays\": {");
}

static void out_array(Out* o, const char* name, const char* dtype, const void* p, size_t n,
                      size_t elem) {
  fwrite(p, elem, n, o->bin);
  fprintf(o->js, "%s\"%s\": {\"dtype\": \"%s\", \"offset\": %ld, \"count\": %zu}",
          o->first ? "" : ", ", name, dtype, o->offset, n);
  o->offset += (long)(n * elem);
  o->first = 0;
}

static void out_close(Out* o, const char* args_json) {
  fprintf(o->js, "}, \"args\": %s}\n", args_json);
  fclose(o->bin);
  fclose(o->js);
}

static int dense_case(const char* dir) {
  const int B = 1, H = 2, N = 200, D = 128, causal = 1, wl = -1, wr = -1;
  const float scale = 0.08838834764831845f; /* 1 / sqrt(128) */
  const size_t n = (size_t)B * H * N * D, rows = (size_t)B * H * N;
  uint16_t* hq = malloc(n * 2);
  uint16_t* hk = malloc(n * 2);
  uint16_t* hv = malloc(n * 2);
  uint16_t* ho = malloc(n * 2);
  float* hl = malloc(rows * 4);
  fill(hq, n, 11u);
  fill(hk, n, 12u);
  fill(hv, n, 13u);
  void *dq, *dk, *dv, *dout;
  float* dl;
  CHECK_HIP(hipMalloc(&dq, n * 2));
  CHECK_HIP(hipMalloc(&dk, n * 2));
  CHECK_HIP(hipMalloc(&dv, n * 2));
  CHECK_HIP(hipMalloc(&dout, n * 2));
  CHECK_HIP(hipMalloc((void**)&dl, rows * 4));
  CHECK_HIP(hipMemcpy(dq, hq, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, n * 2, hipMemcpyHostToDevice));
  int st = attn_fwd(dq, dk, dv, dout, dl, B, H, N, D, ATTN_DTYPE_BF16, scale, causal, wl, wr,
                    NULL);
  if (st != ATTN_OK) {
    fprintf(stderr, "attn_fwd: %s\n", attn_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho, dout, n * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hl, dl, rows * 4, hipMemcpyDeviceToHost));
  /* an unsupported head dim is rejected on the host, before anything runs */
  st = attn_fwd(dq, dk, dv, dout, dl, B, H, N, 96, ATTN_DTYPE_BF16, scale, causal, wl, wr, NULL);
  if (st != ATTN_ERR_UNSUPPORTED_HEAD_DIM) {
    fprintf(stderr, "head_dim 96: expected ATTN_ERR_UNSUPPORTED_HEAD_DIM, got %d\n", st);
    return 1;
  }
  Out o;
  out_open(&o, dir, "dense");
  out_array(&o, "q", "bf16", hq, n, 2);
  out_array(&o, "k", "bf16", hk, n, 2);
  out_array(&o, "v", "bf16", hv, n, 2);
  out_array(&o, "o", "bf16", ho, n, 2);
  out_array(&o, "lse", "f32", hl, rows, 4);
  char args[512];
  snprintf(args, sizeof args,
           "{\"batch\": %d, \"heads\": %d, \"seqlen\": %d, \"head_dim\": %d, \"scale\": %.9g, "
           "\"causal\": %d, \"window_left\": %d, \"window_right\": %d}",
           B, H, N, D, (double)scale, causal, wl, wr);
  out_close(&o, args);
  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dl));
  free(hq), free(hk), free(hv), free(ho), free(hl);
  return 0;
}

static int varlen_case(const char* dir) {
  const int H = 2, D = 64, causal = 1, wl = 20, wr = -1, num_seqs = 3, max_len = 130;
  const int32_t cu[4] = {0, 50, 50, 180};
  const int total = cu[3];
  const float scale = 0.125f; /* 1 / sqrt(64) */
  const size_t n = (size_t)H * total * D, rows = (size_t)H * total;
  uint16_t* hq = malloc(n * 2);
  uint16_t* hk = malloc(n * 2);
  uint16_t* hv = malloc(n * 2);
  uint16_t* ho = malloc(n * 2);
  float* hl = malloc(rows * 4);
  fill(hq, n, 21u);
  fill(hk, n, 22u);
  fill(hv, n, 23u);
  void *dq, *dk, *dv, *dout, *dcu;
  float* dl;
  CHECK_HIP(hipMalloc(&dq, n * 2));
  CHECK_HIP(hipMalloc(&dk, n * 2));
  CHECK_HIP(hipMalloc(&dv, n * 2));
  CHECK_HIP(hipMalloc(&dout, n * 2));
  CHECK_HIP(hipMalloc((void**)&dl, rows * 4));
  CHECK_HIP(hipMalloc(&dcu, sizeof cu));
  CHECK_HIP(hipMemcpy(dq, hq, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dcu, cu, sizeof cu, hipMemcpyHostToDevice));
  const int st = attn_fwd_varlen(dq, dk, dv, dout, dl, (const int32_t*)dcu, num_seqs, max_len,
                                 total, H, D, ATTN_DTYPE_BF16, scale, causal, wl, wr, NULL);
  if (st != ATTN_OK) {
    fprintf(stderr, "attn_fwd_varlen: %s\n", attn_status_string(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(ho, dout, n * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hl, dl, rows * 4, hipMemcpyDeviceToHost));
  Out o;
  out_open(&o, dir, "varlen");
  out_array(&o, "q", "bf16", hq, n, 2);
  out_array(&o, "k", "bf16", hk, n, 2);
  out_array(&o, "v", "bf16", hv, n, 2);
  out_array(&o, "o", "bf16", ho, n, 2);
  out_array(&o, "lse", "f32", hl, rows, 4);
  out_array(&o, "cu_seqlens", "i32", cu, 4, 4);
  char args[512];
  snprintf(args, sizeof args,
           "{\"heads\": %d, \"total_tokens\": %d, \"head_dim\": %d, \"scale\": %.9g, "
           "\"causal\": %d, \"window_left\": %d, \"window_right\": %d, \"max_seqlen\": %d}",
           H, total, D, (double)scale, causal, wl, wr, max_len);
  out_close(&o, args);
  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dl));
  CHECK_HIP(hipFree(dcu));
  free(hq), free(hk), free(hv), free(ho), free(hl);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUT_DIR\n", argv[0]);
    return 64;
  }
  if (dense_case(argv[1]) != 0) return 1;
  if (varlen_case(argv[1]) != 0) return 1;
  printf("c_abi_demo: ok\n");
  return 0;
}
