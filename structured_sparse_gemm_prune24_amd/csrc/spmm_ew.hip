// Unstructured (element-wise) sparse x dense product, the comparison point
// for the structured patterns ("Accelerating Sparse DNNs Based on Tiled GEMM",
// Abstract: TVW against unstructured sparsity).  W is in CSR form with bf16
// values; the product runs on the fp32 vector ALUs: the scattered columns of
// an unstructured row give the matrix cores no fixed operand shape.
#include "p24_api_internal.hpp"
#include "p24_device.hpp"

namespace p24 {

constexpr int EW_WAVES = 4;
constexpr int EW_COLS = 512;          // columns per wave: 8 per lane

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <typename OutT> __device__ __forceinline__ void ew_store(OutT* p, const float (&acc)[8], int n_valid, bool vec);
template <> __device__ __forceinline__ void ew_store<float>(float* p, const float (&acc)[8], int n_valid, bool vec) {
  if (vec) {
    reinterpret_cast<float4*>(p)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    for (int i = 0; i < n_valid; ++i) p[i] = acc[i];
  }
}
template <> __device__ __forceinline__ void ew_store<uint16_t>(uint16_t* p, const float (&acc)[8], int n_valid,
                                                              bool vec) {
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = f32_to_bf16_rne(__float_as_uint(acc[i]));
  if (vec) {
    *reinterpret_cast<u32x4*>(p) = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                         h[6] | (h[7] << 16)};
  } else {
    for (int i = 0; i < n_valid; ++i) p[i] = (uint16_t)h[i];
  }
}

// One wave per (row m, 512-column slice of N); lane l owns columns n0 + 8l ..
// +8.  Each stored entry (k, w) of the row adds w * X[k][n .. n+8) (one 16 B
// read per lane, the wave's 1 KiB coalesced) in fp32, in column order.  Four
// entries are fetched ahead so that their X reads overlap.
template <typename OutT>
__global__ __launch_bounds__(64 * EW_WAVES) void k_spmm_ew(const int64_t* __restrict__ row_ptr,
                                                           const int32_t* __restrict__ cols,
                                                           const uint16_t* __restrict__ vals,
                                                           const uint16_t* __restrict__ X, int64_t ldx, int64_t M,
                                                           int64_t K, int64_t N, OutT* __restrict__ Y, int64_t ldy,
                                                           bool y_vec) {
  const int lane = threadIdx.x & 63;
  const int64_t nchunk = (N + EW_COLS - 1) / EW_COLS;
  const int64_t wid = (int64_t)blockIdx.x * EW_WAVES + (threadIdx.x >> 6);
  if (wid >= M * nchunk) return;                         // wave-uniform
  const int64_t m = wid / nchunk, n = (wid % nchunk) * EW_COLS + 8 * lane;
  const int n_valid = N - n >= 8 ? 8 : (N - n > 0 ? (int)(N - n) : 0);
  const int64_t p0 = row_ptr[m], p1 = row_ptr[m + 1];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](int64_t p) {
    int64_t k = cols[p];
    k = k < 0 ? 0 : (k >= K ? K - 1 : k);
    const float w = bf16_to_f32(vals[p]);
    const uint16_t* xr = X + k * ldx + n;
    uint32_t xb[8];
    if (n_valid == 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xr);
      xb[0] = v.x & 0xFFFFu; xb[1] = v.x >> 16; xb[2] = v.y & 0xFFFFu; xb[3] = v.y >> 16;
      xb[4] = v.z & 0xFFFFu; xb[5] = v.z >> 16; xb[6] = v.w & 0xFFFFu; xb[7] = v.w >> 16;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xb[i] = i < n_valid ? xr[i] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, bf16_to_f32(xb[i]), acc[i]);
  };
  int64_t p = p0;
  for (; p + 4 <= p1; p += 4) {
    add(p);
    add(p + 1);
    add(p + 2);
    add(p + 3);
  }
  for (; p < p1; ++p) add(p);
  if (n_valid > 0) ew_store<OutT>(Y + m * ldy + n, acc, n_valid, y_vec && n_valid == 8);
}

}  // namespace p24

using namespace p24;

extern "C" P24_API p24_status spmm_ew(const int64_t* row_ptr, const int32_t* cols, const void* vals, int64_t M,
                                      int64_t K, const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                                      int64_t ldy, void* stream) {
  if (y_dtype != P24_F32 && y_dtype != P24_BF16) return P24_ERR_DTYPE;
  if (M < 0 || K <= 0 || N < 0 || ldx < N || ldy < N || M > INT32_MAX || K > INT32_MAX || N > INT32_MAX)
    return P24_ERR_SHAPE;
  if (M == 0 || N == 0) return P24_OK;
  if (!row_ptr || !cols || !vals || !X || !Y) return P24_ERR_NULL;
  if (!aligned(row_ptr, 8) || !aligned(cols, 4) || !aligned(vals, 2) || !aligned(X, 16) || ldx % 8 ||
      !aligned(Y, y_dtype == P24_F32 ? 4 : 2))
    return P24_ERR_ALIGN;
  const size_t es = y_dtype == P24_F32 ? 4 : 2;
  const bool y_vec = aligned(Y, 16) && ((size_t)ldy * es) % 16 == 0;
  const int64_t waves = M * ((N + EW_COLS - 1) / EW_COLS);
  const dim3 grid((unsigned)((waves + EW_WAVES - 1) / EW_WAVES)), block(64 * EW_WAVES);
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == P24_F32)
    hipLaunchKernelGGL(k_spmm_ew<float>, grid, block, 0, st, row_ptr, cols, (const uint16_t*)vals,
                       (const uint16_t*)X, ldx, M, K, N, (float*)Y, ldy, y_vec);
  else
    hipLaunchKernelGGL(k_spmm_ew<uint16_t>, grid, block, 0, st, row_ptr, cols, (const uint16_t*)vals,
                       (const uint16_t*)X, ldx, M, K, N, (uint16_t*)Y, ldy, y_vec);
  return launch_status();
}
