/*
 * A plain C consumer of the boundary library, with no torch in the process:
 * it allocates device memory with hipMalloc, calls one entry point of
 * include/fused_boundary.h on a stream of its own, and writes the outputs back.
 * It holds none of the method's arithmetic; tests/test_gpu_c_consumer.py writes
 * its input file and checks its outputs against the oracle.
 *
 *   c_abi_consumer IN OUT
 *
 * IN  (little-endian): int64 T, H, R, K, N, has_shared, has_gate, finalize;
 *     float32 eps, weight_bias; bf16 partials [R][T][H]; bf16 residual [T][H];
 *     bf16 gamma [H]; with finalize: bf16 expert [N][H], int32 idx [T][K],
 *     float32 weights [T][K], bf16 shared [T][H] if has_shared, float32
 *     gate [T] if has_gate.
 * OUT: int32 status; bf16 normed [T][H]; bf16 residual_out [T][H].
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fused_boundary.h"

#define CHECK(x)                                                        \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));    \
      exit(3);                                                          \
    }                                                                   \
  } while (0)

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p == NULL || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input (%zu bytes wanted)\n", bytes);
    exit(2);
  }
  return p;
}

/* Copies a host block to a new device allocation (NULL for an empty block). */
static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (bytes == 0) return NULL;
  CHECK(hipMalloc(&d, bytes));
  CHECK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  int64_t hdr[8];
  float scal[2];
  FILE* f;
  int64_t T, H, R, K, N, r;
  int has_shared, has_gate, finalize, status;
  size_t act, ws_bytes;
  const void* parts[FB_MAX_PARTIALS];
  void *d_res, *d_gamma, *d_exp = NULL, *d_idx = NULL, *d_w = NULL, *d_sh = NULL, *d_gate = NULL;
  void *d_normed, *d_rout, *d_ws;
  void *h_normed, *h_rout;
  hipStream_t stream;

  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  f = fopen(argv[1], "rb");
  if (f == NULL || fread(hdr, sizeof hdr, 1, f) != 1 || fread(scal, sizeof scal, 1, f) != 1) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 2;
  }
  T = hdr[0], H = hdr[1], R = hdr[2], K = hdr[3], N = hdr[4];
  has_shared = (int)hdr[5], has_gate = (int)hdr[6], finalize = (int)hdr[7];
  if (T < 1 || H < 1 || R < 0 || R > FB_MAX_PARTIALS || K < 0 || N < 0) {
    fprintf(stderr, "bad header\n");
    return 2;
  }
  act = (size_t)T * (size_t)H * 2u;

  for (r = 0; r < R; ++r) {
    void* h = read_block(f, act);
    parts[r] = to_device(h, act);
    free(h);
  }
  {
    void* h = read_block(f, act);
    d_res = to_device(h, act);
    free(h);
    h = read_block(f, (size_t)H * 2u);
    d_gamma = to_device(h, (size_t)H * 2u);
    free(h);
  }
  if (finalize) {
    void* h = read_block(f, (size_t)N * (size_t)H * 2u);
    d_exp = to_device(h, (size_t)N * (size_t)H * 2u);
    free(h);
    h = read_block(f, (size_t)T * (size_t)K * 4u);
    d_idx = to_device(h, (size_t)T * (size_t)K * 4u);
    free(h);
    h = read_block(f, (size_t)T * (size_t)K * 4u);
    d_w = to_device(h, (size_t)T * (size_t)K * 4u);
    free(h);
    if (has_shared) {
      h = read_block(f, act);
      d_sh = to_device(h, act);
      free(h);
    }
    if (has_gate) {
      h = read_block(f, (size_t)T * 4u);
      d_gate = to_device(h, (size_t)T * 4u);
      free(h);
    }
  }
  fclose(f);

  CHECK(hipMalloc(&d_normed, act));
  CHECK(hipMalloc(&d_rout, act));
  ws_bytes = fused_boundary_workspace_bytes(T, H);
  CHECK(hipMalloc(&d_ws, ws_bytes));
  CHECK(hipMemset(d_ws, 0, ws_bytes)); /* zero-filled once before first use */
  CHECK(hipStreamCreate(&stream));

  if (finalize)
    status = fused_moe_finalize_rmsnorm(parts, (int32_t)R, d_exp, N, (const int32_t*)d_idx,
                                        (const float*)d_w, (int32_t)K, d_sh, (const float*)d_gate,
                                        d_res, d_gamma, scal[1], scal[0], T, H, d_normed, d_rout,
                                        d_ws, ws_bytes, (void*)stream);
  else
    status = fused_reduce_rmsnorm(parts, (int32_t)R, d_res, d_gamma, scal[1], scal[0], T, H,
                                  d_normed, d_rout, d_ws, ws_bytes, (void*)stream);
  CHECK(hipStreamSynchronize(stream));

  h_normed = malloc(act);
  h_rout = malloc(act);
  if (h_normed == NULL || h_rout == NULL) return 2;
  CHECK(hipMemcpy(h_normed, d_normed, act, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(h_rout, d_rout, act, hipMemcpyDeviceToHost));
  f = fopen(argv[2], "wb");
  if (f == NULL || fwrite(&status, sizeof status, 1, f) != 1 || fwrite(h_normed, 1, act, f) != act ||
      fwrite(h_rout, 1, act, f) != act) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 2;
  }
  fclose(f);
  printf("status %d (%s)\n", status, fused_boundary_status_string(status));

  for (r = 0; r < R; ++r) CHECK(hipFree((void*)parts[r]));
  CHECK(hipFree(d_res));
  CHECK(hipFree(d_gamma));
  if (d_exp) CHECK(hipFree(d_exp));
  if (d_idx) CHECK(hipFree(d_idx));
  if (d_w) CHECK(hipFree(d_w));
  if (d_sh) CHECK(hipFree(d_sh));
  if (d_gate) CHECK(hipFree(d_gate));
  CHECK(hipFree(d_normed));
  CHECK(hipFree(d_rout));
  CHECK(hipFree(d_ws));
  CHECK(hipStreamDestroy(stream));
  free(h_normed);
  free(h_rout);
  return 0;
}
