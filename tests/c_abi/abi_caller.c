/*
 * A caller of libprune24.so written in C99 against include/prune24.h and the
 * HIP runtime API only, with no Python or torch in between.  It runs the 2:4
 * path (compression in both layouts, then spmm24) and the TVW path
 * (tvw_compress, then spmm_tvw) on host inputs and copies the results back to
 * host buffers.  It allocates its device buffers, its TVW workspace and its
 * stream itself, as a C application using the library would.
 *
 * Test infrastructure: the GPU tests load this file's shared library with
 * ctypes, after PyTorch, so that it binds to the HIP runtime already in the
 * process, and compare its outputs with the CPU oracle.
 *
 * Return value of every function: 0, the p24_status of the first failing
 * library call (< 0), or -1000 - hipError_t for a failing runtime call.
 */
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "prune24.h"

#define HIP_TRY(x)                                   \
  do {                                               \
    hipError_t e_ = (x);                             \
    if (e_ != hipSuccess) {                          \
      rc = -1000 - (int)e_;                          \
      goto done;                                     \
    }                                                \
  } while (0)

#define P24_TRY(x)                                   \
  do {                                               \
    p24_status s_ = (x);                             \
    if (s_ != P24_OK) {                              \
      rc = s_;                                       \
      goto done;                                     \
    }                                                \
  } while (0)

static void release(void** bufs, int n, hipStream_t st) {
  int i;
  if (st) hipStreamSynchronize(st);
  for (i = 0; i < n; ++i)
    if (bufs[i]) hipFree(bufs[i]);
  if (st) hipStreamDestroy(st);
}

/*
 * 2:4 path.  W: M x K fp32 row-major; X: K x N bf16 bits row-major (N % 8 == 0).
 * Outputs: the canonical values (M x K/2 bf16 bits) and metadata
 * (M x ceil(K/32) words), and Y = W' X as M x N fp32, where W' is W pruned,
 * compressed in the device layout and multiplied by spmm24.
 */
int p24c_run_24(const float* W, int64_t M, int64_t K, const uint16_t* X, int64_t N,
                uint16_t* values_canonical, uint32_t* meta_canonical, float* Y) {
  int rc = 0;
  hipStream_t st = NULL;
  void* b[7] = {NULL, NULL, NULL, NULL, NULL, NULL, NULL};
  const size_t cvb = prune24_values_bytes(M, K, P24_LAYOUT_CANONICAL);
  const size_t cmb = prune24_meta_bytes(M, K, P24_LAYOUT_CANONICAL);
  const size_t dvb = prune24_values_bytes(M, K, P24_LAYOUT_DEVICE);
  const size_t dmb = prune24_meta_bytes(M, K, P24_LAYOUT_DEVICE);
  if (!cvb || !cmb || !dvb || !dmb) return P24_ERR_SHAPE;
  HIP_TRY(hipStreamCreate(&st));
  HIP_TRY(hipMalloc(&b[0], (size_t)(M * K) * sizeof(float)));
  HIP_TRY(hipMalloc(&b[1], (size_t)(K * N) * sizeof(uint16_t)));
  HIP_TRY(hipMalloc(&b[2], (size_t)(M * N) * sizeof(float)));
  HIP_TRY(hipMalloc(&b[3], cvb));
  HIP_TRY(hipMalloc(&b[4], cmb));
  HIP_TRY(hipMalloc(&b[5], dvb));
  HIP_TRY(hipMalloc(&b[6], dmb));
  HIP_TRY(hipMemcpyAsync(b[0], W, (size_t)(M * K) * sizeof(float), hipMemcpyHostToDevice, st));
  HIP_TRY(hipMemcpyAsync(b[1], X, (size_t)(K * N) * sizeof(uint16_t), hipMemcpyHostToDevice, st));
  P24_TRY(prune24_compress(b[0], P24_F32, M, K, K, b[3], b[4], P24_LAYOUT_CANONICAL, st));
  P24_TRY(prune24_compress(b[0], P24_F32, M, K, K, b[5], b[6], P24_LAYOUT_DEVICE, st));
  P24_TRY(spmm24(b[5], b[6], P24_LAYOUT_DEVICE, M, K, b[1], N, N, b[2], P24_F32, N, P24_ALGO_AUTO, st));
  HIP_TRY(hipMemcpyAsync(values_canonical, b[3], cvb, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipMemcpyAsync(meta_canonical, b[4], cmb, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipMemcpyAsync(Y, b[2], (size_t)(M * N) * sizeof(float), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
done:
  release(b, 7, st);
  return rc;
}

/*
 * TVW path.  W: M x K fp32; X: K x N bf16 bits (N % 8 == 0).  Outputs: the
 * kept columns of every tile (ceil(M / tile_m) x keep_k, ascending) and
 * Y = W_tvw X as M x N fp32.
 */
int p24c_run_tvw(const float* W, int64_t M, int64_t K, int64_t tile_m, int64_t keep_k,
                 const uint16_t* X, int64_t N, int32_t* kept, float* Y) {
  int rc = 0;
  hipStream_t st = NULL;
  void* b[7] = {NULL, NULL, NULL, NULL, NULL, NULL, NULL};
  const int64_t tiles = (M + tile_m - 1) / tile_m;
  const size_t vb = prune24_values_bytes(M, keep_k, P24_LAYOUT_DEVICE);
  const size_t mb = prune24_meta_bytes(M, keep_k, P24_LAYOUT_DEVICE);
  const size_t wsb = tvw_workspace_bytes(M, K, tile_m, keep_k);
  const size_t kb = (size_t)(tiles * keep_k) * sizeof(int32_t);
  if (!vb || !mb || !wsb) return P24_ERR_SHAPE;
  HIP_TRY(hipStreamCreate(&st));
  HIP_TRY(hipMalloc(&b[0], (size_t)(M * K) * sizeof(float)));
  HIP_TRY(hipMalloc(&b[1], (size_t)(K * N) * sizeof(uint16_t)));
  HIP_TRY(hipMalloc(&b[2], (size_t)(M * N) * sizeof(float)));
  HIP_TRY(hipMalloc(&b[3], kb));
  HIP_TRY(hipMalloc(&b[4], vb));
  HIP_TRY(hipMalloc(&b[5], mb));
  HIP_TRY(hipMalloc(&b[6], wsb));
  HIP_TRY(hipMemcpyAsync(b[0], W, (size_t)(M * K) * sizeof(float), hipMemcpyHostToDevice, st));
  HIP_TRY(hipMemcpyAsync(b[1], X, (size_t)(K * N) * sizeof(uint16_t), hipMemcpyHostToDevice, st));
  P24_TRY(tvw_compress(b[0], P24_F32, M, K, K, tile_m, keep_k, (int32_t*)b[3], b[4], b[5],
                       P24_LAYOUT_DEVICE, b[6], wsb, st));
  P24_TRY(spmm_tvw((const int32_t*)b[3], b[4], b[5], P24_LAYOUT_DEVICE, M, K, tile_m, keep_k, b[1], N, N,
                   b[2], P24_F32, N, st));
  HIP_TRY(hipMemcpyAsync(kept, b[3], kb, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipMemcpyAsync(Y, b[2], (size_t)(M * N) * sizeof(float), hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
done:
  release(b, 7, st);
  return rc;
}

/*
 * Argument checks seen from C: each request below is invalid (or empty) and is
 * answered before anything is enqueued, so no pointer is dereferenced.
 * codes[0..5] receive the statuses; the function returns the ABI version.
 */
int p24c_error_paths(int32_t* codes) {
  static float host_dummy[16];
  void* p = host_dummy;
  codes[0] = spmm24(p, p, P24_LAYOUT_DEVICE, 64, 100, p, 64, 64, p, P24_F32, 64, P24_ALGO_AUTO, NULL);
  codes[1] = spmm24(p, p, P24_LAYOUT_CANONICAL, 64, 128, p, 64, 64, p, P24_F32, 64, P24_ALGO_AUTO, NULL);
  codes[2] = prune24_compress(p, P24_F32, 4, 6, 6, p, p, P24_LAYOUT_CANONICAL, NULL);
  codes[3] = prune24_compress(NULL, P24_F32, 4, 8, 8, p, p, P24_LAYOUT_CANONICAL, NULL);
  codes[4] = spmm24(p, p, P24_LAYOUT_DEVICE, 0, 128, p, 64, 64, p, P24_F32, 64, P24_ALGO_AUTO, NULL);
  codes[5] = prune24_compress(p, 7, 4, 8, 8, p, p, P24_LAYOUT_CANONICAL, NULL);
  return prune24_abi_version();
}
