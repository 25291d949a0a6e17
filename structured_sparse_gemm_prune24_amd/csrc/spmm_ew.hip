// Unstructured (element-wise) sparse x dense product, the comparison point
// for the structured patterns ("Accelerating Sparse DNNs Based on Tiled GEMM",
// Abstract: TVW against unstructured sparsity).  W is in CSR form with bf16
// values; the product runs on the fp32 vector ALUs: the scattered columns of
// an unstructured row give the matrix cores no fixed operand shape.
#include "p24_api_internal.hpp"
#include "p24_device.hpp"

namespace p24 {

constexpr int EW_WAVES = 8;
constexpr int EW_ROWS_PER_WAVE = 8;
constexpr int EW_ROWS = EW_WAVES * EW_ROWS_PER_WAVE;   // W rows per block
constexpr int EW_NB = 256;                              // columns per block: 4 per lane
constexpr int EW_KB = 32;                               // X rows staged in LDS at a time
constexpr int EW_ROWB = EW_NB * 4;                      // bytes per staged X row (fp32)

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

// One block per (64 rows of W, 256 columns of N), 8 waves.  The block walks K
// in chunks of 32: the chunk X[k0 .. k0+32)[n0 .. n0+256) is staged in LDS as
// fp32 (32 KiB, rows past K and columns past N zero; converted once per
// element here instead of once per stored entry below), then each wave takes
// its 8 rows.  The small chunk leaves room for two blocks per CU, whose 16
// waves hide each other's LDS and lane-broadcast latencies (64 KiB chunks and
// one block of 4 waves less per CU measured 17 % slower; 4-wave blocks of 32
// rows, which stage each chunk for half as many rows, 7 % slower; 16-wave
// blocks of 128 rows, one per CU, 2 % slower).  For a row, 64 stored entries at a time are read one per lane;
// those inside the chunk (columns ascending, so a prefix of the lanes) are
// broadcast one by one as one word (bf16 value in the high half, chunk row in
// the low half: the value is that word with the low half cleared), and each
// adds w * X[k][4 lane .. +4] from LDS to the lane's fp32 accumulators, in
// column order.  Every X element is read from L2 once per block instead of
// once per stored entry.
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
    // The first window of stored entries (64, one per lane) of each of the
    // wave's rows, loaded for all rows before any is used: the loads overlap
    // each other and the staging below instead of costing one latency per row.
    int32_t cwin[EW_ROWS_PER_WAVE];
    uint32_t wwin[EW_ROWS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < EW_ROWS_PER_WAVE; ++i) {
      const int64_t q = pos[i] + lane;
      const bool valid = q < end[i];
      cwin[i] = valid ? cols[q] : 0x7FFFFFFF;
      wwin[i] = valid ? vals[q] : 0u;
    }
    __syncthreads();                                      // the previous chunk is consumed
    // stage the chunk: piece q = tid + 64 EW_WAVES j is row q / 32, 8 bf16 columns
    // 8 (q % 32) .. +8; every piece is loaded before any is written, so all
    // loads are in flight at once
    constexpr int PIECES = EW_KB * EW_NB / 8 / (64 * EW_WAVES);
    u32x4 pv[PIECES];
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int q = tid + 64 * EW_WAVES * j;
      const int r = q / (EW_NB / 8), pc = q % (EW_NB / 8);
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
      pv[j] = v;
    }
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int q = tid + 64 * EW_WAVES * j;
      const int r = q / (EW_NB / 8), pc = q % (EW_NB / 8);
      const u32x4 v = pv[j];
      const u32x4 lo = {v[0] << 16, v[0] & 0xFFFF0000u, v[1] << 16, v[1] & 0xFFFF0000u};
      const u32x4 hi = {v[2] << 16, v[2] & 0xFFFF0000u, v[3] << 16, v[3] & 0xFFFF0000u};
      *reinterpret_cast<u32x4*>(xs + r * EW_ROWB + pc * 32) = lo;
      *reinterpret_cast<u32x4*>(xs + r * EW_ROWB + pc * 32 + 16) = hi;
    }
    __syncthreads();
    const int64_t k_hi = k0 + EW_KB;
#pragma unroll
    for (int i = 0; i < EW_ROWS_PER_WAVE; ++i) {
      int64_t p = pos[i];
      const int64_t e = end[i];
      int32_t c_next = cwin[i];
      uint32_t w_next = wwin[i];
      while (p < e) {
        const int64_t q = p + lane;
        const bool valid = q < e;
        const int32_t c = c_next;
        const uint32_t w = w_next;
        const bool in = valid && c < k_hi;
        const int n_in = __popcll(__ballot(in));
        // chunk row of each entry (clamped into the chunk) in the low half, the
        // bf16 value in the high half
        int32_t kk = c - (int32_t)k0;
        kk = kk < 0 ? 0 : (kk >= EW_KB ? EW_KB - 1 : kk);
        const uint32_t packed = (w << 16) | (uint32_t)kk;
        const uint32_t lane_off = (uint32_t)lane * 16;
        auto fma4 = [&](uint32_t word, f32x4 xv) {
          const float wf = __uint_as_float(word & 0xFFFF0000u);
          acc[i][0] = fmaf(wf, xv[0], acc[i][0]);
          acc[i][1] = fmaf(wf, xv[1], acc[i][1]);
          acc[i][2] = fmaf(wf, xv[2], acc[i][2]);
          acc[i][3] = fmaf(wf, xv[3], acc[i][3]);
        };
        auto xrow = [&](uint32_t word) {
          return *reinterpret_cast<const f32x4*>(xs + (word & 0xFFFFu) * EW_ROWB + lane_off);
        };
        // eight entries at a time: their LDS reads are all issued before the
        // multiply-adds, which then run in entry (column) order
        int j = 0;
        for (; j + 8 <= n_in; j += 8) {
          uint32_t wd[8];
          f32x4 xv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            wd[u] = (uint32_t)__builtin_amdgcn_readlane((int)packed, j + u);
            xv[u] = xrow(wd[u]);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) fma4(wd[u], xv[u]);
        }
        for (; j < n_in; ++j) {
          const uint32_t wd = (uint32_t)__builtin_amdgcn_readlane((int)packed, j);
          fma4(wd, xrow(wd));
        }
        p += n_in;
        if (n_in < 64) break;
        // a full window inside the chunk: the next one
        const int64_t qn = p + lane;
        c_next = qn < e ? cols[qn] : 0x7FFFFFFF;
        w_next = qn < e ? vals[qn] : 0u;
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
