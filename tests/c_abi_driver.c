/*
 * Plain C caller of libvcattn.so: the C ABI used without Python or torch.
 * Device buffers come from hipMalloc, the work runs on a stream this program
 * creates, and the output is copied back and written raw.
 *
 *   c_abi_driver <inputs> <output> B H N C flags
 *
 * <inputs> holds Q, K and V one after the other, bf16 [B][H][N][128] each;
 * <output> receives O, bf16 [B][H][N][128].  Before the real calls the program
 * checks two error paths (a null input pointer, a short workspace), which must
 * be refused before any device work.  Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "vc_attn.h"

#define HIP_OK(x)                                                             \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      return 3;                                                               \
    }                                                                         \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s <inputs> <output> B H N C flags\n", argv[0]);
    return 2;
  }
  vc_attn_params p;
  vc_attn_default_params(&p);
  p.B = atoi(argv[3]);
  p.H = atoi(argv[4]);
  p.N = atoi(argv[5]);
  p.n_clusters = atoi(argv[6]);
  p.flags = (uint32_t)strtoul(argv[7], NULL, 0);
  vc_status st = vc_attn_check_params(&p);
  if (st != VC_OK) {
    fprintf(stderr, "parameters refused: %s\n", vc_attn_status_string(st));
    return 2;
  }
  const size_t n = (size_t)p.B * p.H * p.N * 128, bytes = n * 2;
  unsigned char* host = (unsigned char*)malloc(3 * bytes);
  FILE* f = fopen(argv[1], "rb");
  if (!host || !f || fread(host, 1, 3 * bytes, f) != 3 * bytes) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", 3 * bytes, argv[1]);
    return 2;
  }
  fclose(f);

  void *q, *k, *v, *o, *ws;
  const size_t ws_bytes = vc_attn_workspace_size(&p);
  HIP_OK(hipMalloc(&q, bytes));
  HIP_OK(hipMalloc(&k, bytes));
  HIP_OK(hipMalloc(&v, bytes));
  HIP_OK(hipMalloc(&o, bytes));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(q, host, bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, host + bytes, bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, host + 2 * bytes, bytes, hipMemcpyHostToDevice));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  /* error paths: refused before any device work */
  st = vc_attn_prepare(&p, NULL, k, v, ws, ws_bytes, s);
  if (st != VC_ERR_INVALID_ARG) {
    fprintf(stderr, "null Q: expected VC_ERR_INVALID_ARG, got %s\n", vc_attn_status_string(st));
    return 4;
  }
  st = vc_attn_prepare(&p, q, k, v, ws, ws_bytes - 1, s);
  if (st != VC_ERR_WORKSPACE) {
    fprintf(stderr, "short workspace: expected VC_ERR_WORKSPACE, got %s\n", vc_attn_status_string(st));
    return 4;
  }

  st = vc_attn_prepare(&p, q, k, v, ws, ws_bytes, s);
  if (st != VC_OK) {
    fprintf(stderr, "vc_attn_prepare: %s\n", vc_attn_status_string(st));
    return 5;
  }
  st = vc_attn_forward(&p, ws, ws_bytes, o, s);
  if (st != VC_OK) {
    fprintf(stderr, "vc_attn_forward: %s\n", vc_attn_status_string(st));
    return 5;
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(host, o, bytes, hipMemcpyDeviceToHost));
  f = fopen(argv[2], "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 2;
  }
  fclose(f);
  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(ws));
  free(host);
  printf("c_abi_driver: library version %d, workspace %zu bytes, ok\n", (int)vc_attn_version(), ws_bytes);
  return 0;
}
