/*
 * abi_demo.c -- a plain C consumer of libmxattn.so (include/mxattn.h), with
 * no Python and no torch: HIP runtime calls for memory and a stream, then the
 * library's calls.  Run by tests/test_gpu_abi_c.py; prints one line starting
 * with "abi_demo ok" and exits 0 when every check holds.
 *
 * Checks:
 *   - mxattn_fwd (bf16 Q, K, V) equals, bit for bit, mxq_quantize of Q, K, V
 *     followed by mxattn_fwd_quantized, as the header states;
 *   - rejected calls return their documented status and enqueue nothing;
 *   - mxq_dump writes the 256-byte header plus codes and scales.
 * Usage: abi_demo DUMP_PATH
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxattn.h"

#define CHECK_HIP(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define CHECK_MXQ(x, want)                                                       \
  do {                                                                           \
    int s_ = (x);                                                                \
    if (s_ != (want)) {                                                          \
      fprintf(stderr, "line %d: got %s, want %s\n", __LINE__, mxq_status_string(s_), \
              mxq_status_string(want));                                          \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

/* bf16 bit pattern of a float, round to nearest even */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* xorshift32, mapped to [-2, 2) */
static float next_value(uint32_t* s) {
  uint32_t x = *s;
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  *s = x;
  return (float)(x >> 8) / 16777216.0f * 4.0f - 2.0f;
}

int main(int argc, char** argv) {
  if (argc < 2) {
    fprintf(stderr, "usage: abi_demo DUMP_PATH\n");
    return 2;
  }
  const int64_t B = 1, H = 2, N = 300, d = 128;
  const size_t n = (size_t)(B * H * N * d);
  uint16_t* host = (uint16_t*)malloc(3 * n * sizeof(uint16_t));
  uint16_t* out1 = (uint16_t*)malloc(n * sizeof(uint16_t));
  uint16_t* out2 = (uint16_t*)malloc(n * sizeof(uint16_t));
  if (!host || !out1 || !out2) return 1;
  uint32_t seed = 12345u;
  for (size_t i = 0; i < 3 * n; ++i) host[i] = to_bf16(next_value(&seed));

  void *q, *k, *v, *o1, *o2, *ws;
  CHECK_HIP(hipMalloc(&q, n * 2));
  CHECK_HIP(hipMalloc(&k, n * 2));
  CHECK_HIP(hipMalloc(&v, n * 2));
  CHECK_HIP(hipMalloc(&o1, n * 2));
  CHECK_HIP(hipMalloc(&o2, n * 2));
  CHECK_HIP(hipMemcpy(q, host, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, host + n, n * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, host + 2 * n, n * 2, hipMemcpyHostToDevice));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  /* 1. the whole path */
  const size_t wsb = mxattn_workspace_bytes(B, H, N, d);
  if (wsb == 0) return 1;
  CHECK_HIP(hipMalloc(&ws, wsb));
  CHECK_MXQ(mxattn_fwd(q, k, v, B, H, N, d, MXQ_MODE_UOS, 1, 0.0f, o1, ws, wsb, stream), MXQ_OK);

  /* 2. quantize the three operands, then the attention kernel on codes */
  const int64_t nbk = d / 32, nbv = (N + 31) / 32;
  uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  CHECK_HIP(hipMalloc((void**)&qc, (size_t)(B * H * N * nbk * 16)));
  CHECK_HIP(hipMalloc((void**)&qs, (size_t)(B * H * N * nbk)));
  CHECK_HIP(hipMalloc((void**)&kc, (size_t)(B * H * N * nbk * 16)));
  CHECK_HIP(hipMalloc((void**)&ks, (size_t)(B * H * N * nbk)));
  CHECK_HIP(hipMalloc((void**)&vc, (size_t)(B * H * d * nbv * 16)));
  CHECK_HIP(hipMalloc((void**)&vs, (size_t)(B * H * d * nbv)));
  CHECK_MXQ(mxq_quantize(q, B * H, N, d, 1, MXQ_MODE_UOS, qc, qs, stream), MXQ_OK);
  CHECK_MXQ(mxq_quantize(k, B * H, N, d, 1, MXQ_MODE_UOS, kc, ks, stream), MXQ_OK);
  CHECK_MXQ(mxq_quantize(v, B * H, N, d, 0, MXQ_MODE_UOS, vc, vs, stream), MXQ_OK);
  CHECK_MXQ(mxattn_fwd_quantized(qc, qs, kc, ks, vc, vs, B, H, N, d, MXQ_MODE_UOS, 1, 0.0f, o2, stream), MXQ_OK);

  /* 3. rejected calls */
  CHECK_MXQ(mxattn_fwd(q, k, v, B, H, N, 96, MXQ_MODE_UOS, 1, 0.0f, o1, ws, wsb, stream), MXQ_ERR_UNSUPPORTED);
  CHECK_MXQ(mxattn_fwd(q, k, v, B, H, N, d, MXQ_MODE_UOS, 1, 0.0f, o1, ws, wsb - 1, stream), MXQ_ERR_WORKSPACE);
  CHECK_MXQ(mxq_quantize(q, B * H, N, d, 2, MXQ_MODE_UOS, qc, qs, stream), MXQ_ERR_INVALID_ARG);

  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(out1, o1, n * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out2, o2, n * 2, hipMemcpyDeviceToHost));
  if (memcmp(out1, out2, n * 2) != 0) {
    fprintf(stderr, "mxattn_fwd and mxattn_fwd_quantized differ\n");
    return 1;
  }
  uint64_t sum = 0;
  int finite = 1;
  for (size_t i = 0; i < n; ++i) {
    sum = sum * 1000003u + out1[i];
    if ((out1[i] & 0x7F80u) == 0x7F80u) finite = 0;
  }
  if (!finite) {
    fprintf(stderr, "non-finite output\n");
    return 1;
  }

  /* 4. dump the V codes and check the file's size */
  CHECK_MXQ(mxq_dump(argv[1], vc, vs, B * H, d, N, 0, MXQ_MODE_UOS, stream), MXQ_OK);
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 1;
  fseek(f, 0, SEEK_END);
  const long size = ftell(f);
  fclose(f);
  const long want = 256 + (long)(B * H * d * nbv * 17);
  if (size != want) {
    fprintf(stderr, "dump has %ld bytes, want %ld\n", size, want);
    return 1;
  }

  printf("abi_demo ok: %lld outputs equal on both paths, checksum %016llx, %s\n", (long long)n,
         (unsigned long long)sum, mxq_status_string(MXQ_OK));
  hipFree(q); hipFree(k); hipFree(v); hipFree(o1); hipFree(o2); hipFree(ws);
  hipFree(qc); hipFree(qs); hipFree(kc); hipFree(ks); hipFree(vc); hipFree(vs);
  hipStreamDestroy(stream);
  free(host); free(out1); free(out2);
  return 0;
}
