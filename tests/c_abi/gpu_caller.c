/*
 * A C99 program that drives the library with no Python and no torch: HIP's C
 * runtime API for device memory and a stream, the library's C ABI for the
 * work.  Reads raw bf16 inputs from a file, runs add_rmsnorm_fwd over them
 * and qk_rmsnorm_fwd in place on a fused qkv tensor, and writes the raw
 * outputs to another file.
 *
 *   gpu_caller <in> <out> <n_rows> <hidden> <tokens> <q_heads> <k_heads> <head_dim>
 *
 * <in>:  x, residual [n_rows * hidden], weight [hidden], then qkv
 *        [tokens * (q_heads + 2 k_heads) * head_dim], q_weight, k_weight
 *        [head_dim], all uint16.
 * <out>: out, residual_out [n_rows * hidden], then qkv after the in-place
 *        q/k norm.
 * Exit status 0 on success; otherwise a message names the failing step.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "add_rmsnorm.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static int read_all(const char* path, void* buf, size_t bytes) {
  FILE* f = fopen(path, "rb");
  size_t got;
  if (!f) return 1;
  got = fread(buf, 1, bytes, f);
  fclose(f);
  return got != bytes;
}

int main(int argc, char** argv) {
  int64_t n, h, t, hq, hk, d, width;
  size_t tb, wb, qb, hb;
  uint16_t *host, *dx, *dr, *dw, *dout, *dres, *dqkv, *dqw, *dkw;
  hipStream_t stream;
  int rc;
  FILE* f;

  if (argc != 9) {
    fprintf(stderr, "usage: gpu_caller in out n_rows hidden tokens q_heads k_heads head_dim\n");
    return 2;
  }
  n = atoll(argv[3]);
  h = atoll(argv[4]);
  t = atoll(argv[5]);
  hq = atoll(argv[6]);
  hk = atoll(argv[7]);
  d = atoll(argv[8]);
  width = (hq + 2 * hk) * d;
  tb = (size_t)(n * h) * 2;
  wb = (size_t)h * 2;
  qb = (size_t)(t * width) * 2;
  hb = (size_t)d * 2;
  host = (uint16_t*)malloc(2 * tb + wb + qb + 2 * hb);
  if (!host || read_all(argv[1], host, 2 * tb + wb + qb + 2 * hb)) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }

  HIP_OK(hipMalloc((void**)&dx, tb));
  HIP_OK(hipMalloc((void**)&dr, tb));
  HIP_OK(hipMalloc((void**)&dw, wb));
  HIP_OK(hipMalloc((void**)&dout, tb));
  HIP_OK(hipMalloc((void**)&dres, tb));
  HIP_OK(hipMalloc((void**)&dqkv, qb));
  HIP_OK(hipMalloc((void**)&dqw, hb));
  HIP_OK(hipMalloc((void**)&dkw, hb));
  HIP_OK(hipStreamCreate(&stream));
  HIP_OK(hipMemcpy(dx, host, tb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dr, (char*)host + tb, tb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, (char*)host + 2 * tb, wb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dqkv, (char*)host + 2 * tb + wb, qb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dqw, (char*)host + 2 * tb + wb + qb, hb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkw, (char*)host + 2 * tb + wb + qb + hb, hb, hipMemcpyHostToDevice));

  rc = add_rmsnorm_fwd(dout, dres, dx, dr, dw, n, h, 1e-6f, stream);
  if (rc != ADD_RMSNORM_OK) {
    fprintf(stderr, "add_rmsnorm_fwd: %s\n", add_rmsnorm_strerror(rc));
    return 1;
  }
  rc = qk_rmsnorm_fwd(dqkv, dqkv + hq * d, dqkv, dqkv + hq * d, dqw, dkw, t, hq, hk, d, width,
                      width, width, width, 1e-6f, stream);
  if (rc != ADD_RMSNORM_OK) {
    fprintf(stderr, "qk_rmsnorm_fwd: %s\n", add_rmsnorm_strerror(rc));
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(host, dout, tb, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy((char*)host + tb, dres, tb, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy((char*)host + 2 * tb, dqkv, qb, hipMemcpyDeviceToHost));
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dr));
  HIP_OK(hipFree(dw));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dres));
  HIP_OK(hipFree(dqkv));
  HIP_OK(hipFree(dqw));
  HIP_OK(hipFree(dkw));

  f = fopen(argv[2], "wb");
  if (!f || fwrite(host, 1, 2 * tb + qb, f) != 2 * tb + qb) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(f);
  free(host);
  return 0;
}
