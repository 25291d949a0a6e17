// Unstructured (element-wise) sparse x dense product, the comparison point
// for the structured patterns ("Accelerating Sparse DNNs Based on Tiled GEMM",
// Abstract: TVW against unstructured sparsity).  W is in CSR form with bf16
// values; the product runs on the fp32 vector ALUs: the scattered columns of
// an unstructured row give the matrix cores no fixed operand shape.
#include "p24_api_internal.hpp"
#include "p24_device.hpp"

namespace p24 {

constexpr int EW_WAVES = 4;
constexpr int EW_ROWS_PER_WAVE = 8;
constexpr int EW_ROWS = EW_WAVES * EW_ROWS_PER_WAVE;   // W rows per block
constexpr int EW_NB = 256;                              // columns per block: 4 per lane
constexpr int EW_KB = 128;                              // X rows staged in LDS at a time
constexpr int EW_ROWB = EW_NB * 2;                      // bytes per staged X row

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

template <typename OutT> __device__ __forceinline__ void ew_store(OutT* p, const float (&acc)[4], int n_valid, bool vec);
template <> __device__ __forceinline__ void ew_store<float>(float* p, const float (&acc)[4], int n_valid, bool vec) {
  if (vec) {
    *reinterpret_cast<float4*>(p) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
    for (int i = 0; i < n_valid; ++i) p[i] = acc[i];
  }
}
template <> __device__ __forceinline__ void ew_store<uint16_t>(uint16_t* p, const float (&acc)[4], int n_valid,
                                                              bool vec) {
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = f32_to_bf16_rne(__float_as_uint(acc[i]));
  if (vec) {
    *reinterpret_cast<u32x2*>(p) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  } else {
    for (int i = 0; i < n_valid; ++i) p[i] = (uint16_t)h[i];
  }
}

// One block per (32 rows of W, 256 columns of N).  The block walks K in
// chunks of 128: the chunk X[k0 .. k0+128)[n0 .. n0+256) is staged in LDS
// (64 KiB, rows past K and columns past N zero), then each wave takes its 8
// rows.  For a row, 64 stored entries at a time are read one per lane; those
// inside the chunk (columns ascending, so a prefix of the lanes) are
// broadcast one by one, and each adds w * X[k][4 lane .. +4] from LDS to the
// lane's fp32 accumulators, in column order.  Every X element is read from
// L2 once per block instead of once per stored entry.
template <typename OutT>
__global__ __launch_bounds__(64 * EW_WAVES) void k_spmm_ew(const int64_t* __restrict__ row_ptr,
                                                           const int32_t* __restrict__ cols,
                                                           const uint16_t* __restrict__ vals,
                                                           const uint16_t* __restrict__ X, int64_t ldx, int64_t M,
                                                           int64_t K, int64_t N, OutT* __restrict__ Y, int64_t ldy,
                                                           bool y_vec) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[EW_KB * EW_ROWB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nch = (N + EW_NB - 1) / EW_NB;
  const int64_t m0 = (int64_t)(blockIdx.x / nch) * EW_ROWS, n0 = (int64_t)(blockIdx.x % nch) * EW_NB;
  const int64_t mw = m0 + wave * EW_ROWS_PER_WAVE;         // this wave's first row

  int64_t pos[EW_ROWS_PER_WAVE], end[EW_ROWS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < EW_ROWS_PER_WAVE; ++i) {
    const int64_t m = mw + i < M ? mw + i : M - 1;
    pos[i] = mw + i < M ? row_ptr[m] : 0;
    end[i] = mw + i < M ? row_ptr[m + 1] : 0;
  }
  float acc[EW_ROWS_PER_WAVE][4];
#pragma unroll
  for (int i = 0; i < EW_ROWS_PER_WAVE; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += EW_KB) {
    __syncthreads();                                      // the previous chunk is consumed
    // stage the chunk: piece q = tid + 256 j is row q / 32, 16 B piece q % 32
#pragma unroll 4
    for (int j = 0; j < EW_KB * EW_ROWB / 16 / (64 * EW_WAVES); ++j) {
      const int q = tid + 64 * EW_WAVES * j;
      const int r = q / (EW_ROWB / 16), pc = q % (EW_ROWB / 16);
      const int64_t k = k0 + r, n = n0 + 8 * pc;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k < K) {
        const uint16_t* src = X + k * ldx + n;
        if (n + 8 <= N) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint32_t h[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) h[i] = n + i < N ? src[i] : 0u;
          v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
      *reinterpret_cast<u32x4*>(xs + r * EW_ROWB + pc * 16) = v;
    }
    __syncthreads();
    const int64_t k_hi = k0 + EW_KB;
#pragma unroll
    for (int i = 0; i < EW_ROWS_PER_WAVE; ++i) {
      int64_t p = pos[i];
      const int64_t e = end[i];
      while (p < e) {
        const int64_t q = p + lane;
        const bool valid = q < e;
        const int32_t c = valid ? cols[q] : 0x7FFFFFFF;
        const uint32_t w = valid ? vals[q] : 0u;
        const bool in = valid && c < k_hi;
        const int n_in = __popcll(__ballot(in));
        // row offset of each entry inside the staged chunk, clamped into it
        int32_t kk = c - (int32_t)k0;
        kk = kk < 0 ? 0 : (kk >= EW_KB ? EW_KB - 1 : kk);
        const uint32_t roff = (uint32_t)kk * EW_ROWB;
        // eight entries at a time: their LDS reads are all issued before the
        // multiply-adds, which then run in entry (column) order
        auto fma4 = [&](float wf, u32x2 xv) {
          acc[i][0] = fmaf(wf, bf16_to_f32(xv.x & 0xFFFFu), acc[i][0]);
          acc[i][1] = fmaf(wf, bf16_to_f32(xv.x >> 16), acc[i][1]);
          acc[i][2] = fmaf(wf, bf16_to_f32(xv.y & 0xFFFFu), acc[i][2]);
          acc[i][3] = fmaf(wf, bf16_to_f32(xv.y >> 16), acc[i][3]);
        };
        int j = 0;
        for (; j + 8 <= n_in; j += 8) {
          u32x2 xv[8];
          float wf[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)roff, j + u) + lane * 8;
            wf[u] = bf16_to_f32((uint32_t)__builtin_amdgcn_readlane((int)w, j + u));
            xv[u] = *reinterpret_cast<const u32x2*>(xs + a);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) fma4(wf[u], xv[u]);
        }
        for (; j < n_in; ++j) {
          const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)roff, j) + lane * 8;
          fma4(bf16_to_f32((uint32_t)__builtin_amdgcn_readlane((int)w, j)), *reinterpret_cast<const u32x2*>(xs + a));
        }
        p += n_in;
        if (n_in < 64) break;
      }
      pos[i] = p;
    }
  }
  const int64_t n = n0 + 4 * lane;
  const int n_valid = N - n >= 4 ? 4 : (N - n > 0 ? (int)(N - n) : 0);
#pragma unroll
  for (int i = 0; i < EW_ROWS_PER_WAVE; ++i)
    if (mw + i < M && n_valid > 0) ew_store<OutT>(Y + (mw + i) * ldy + n, acc[i], n_valid, y_vec && n_valid == 4);
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
  const bool y_vec = aligned(Y, 16) && ((size_t)ldy * es) % (4 * es) == 0;
  const int64_t blocks = ((M + EW_ROWS - 1) / EW_ROWS) * ((N + EW_NB - 1) / EW_NB);
  if (blocks > INT32_MAX) return P24_ERR_SHAPE;
  const dim3 grid((unsigned)blocks), block(64 * EW_WAVES);
  hipStream_t st = (hipStream_t)stream;
  if (y_dtype == P24_F32)
    hipLaunchKernelGGL(k_spmm_ew<float>, grid, block, 0, st, row_ptr, cols, (const uint16_t*)vals,
                       (const uint16_t*)X, ldx, M, K, N, (float*)Y, ldy, y_vec);
  else
    hipLaunchKernelGGL(k_spmm_ew<uint16_t>, grid, block, 0, st, row_ptr, cols, (const uint16_t*)vals,
                       (const uint16_t*)X, ldx, M, K, N, (uint16_t*)Y, ldy, y_vec);
  return launch_status();
}
