// Test infrastructure: one wavefront runs one matrix instruction on operands
// given lane by lane, so a GPU test can compare the hardware's lane mapping with
// the lane-level models the CPU tests drive the device layouts through.
//   p24probe_smfmac32: v_smfmac_f32_32x32x32_bf16, A = a[64][8] (compressed
//     bf16 values), B = b[64][16] bf16, index word idx[64] (its 16-bit half
//     `abid` is used), zero accumulator; d[64][16] fp32 in the instruction's
//     output lane order.
//   p24probe_mfma32x32x16: v_mfma_f32_32x32x16_bf16, A = a[64][8], B = b[64][8].
// Both return 0, or -1 if the launch failed.  All pointers are device pointers.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16v __attribute__((ext_vector_type(16)));
typedef float f16v __attribute__((ext_vector_type(16)));

template <int ABID>
__global__ __launch_bounds__(64) void k_smfmac(const uint16_t* a, const uint16_t* b, const uint32_t* idx, float* d) {
  const int l = threadIdx.x;
  s16x8 av;
  s16x16 bv;
  for (int i = 0; i < 8; ++i) av[i] = (short)a[l * 8 + i];
  for (int i = 0; i < 16; ++i) bv[i] = (short)b[l * 16 + i];
  f16v acc = {};
  acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf8, av), __builtin_bit_cast(bf16v, bv), acc,
                                                  (int)idx[l], 0, ABID);
  for (int i = 0; i < 16; ++i) d[l * 16 + i] = acc[i];
}

__global__ __launch_bounds__(64) void k_mfma(const uint16_t* a, const uint16_t* b, float* d) {
  const int l = threadIdx.x;
  s16x8 av, bv;
  for (int i = 0; i < 8; ++i) {
    av[i] = (short)a[l * 8 + i];
    bv[i] = (short)b[l * 8 + i];
  }
  f16v acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, av), __builtin_bit_cast(bf8, bv), acc, 0, 0, 0);
  for (int i = 0; i < 16; ++i) d[l * 16 + i] = acc[i];
}

extern "C" __attribute__((visibility("default"))) int p24probe_smfmac32(const uint16_t* a, const uint16_t* b,
                                                                       const uint32_t* idx, int abid, float* d,
                                                                       void* stream) {
  if (abid == 0)
    hipLaunchKernelGGL(k_smfmac<0>, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, idx, d);
  else
    hipLaunchKernelGGL(k_smfmac<1>, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, idx, d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" __attribute__((visibility("default"))) int p24probe_mfma32x32x16(const uint16_t* a, const uint16_t* b,
                                                                           float* d, void* stream) {
  hipLaunchKernelGGL(k_mfma, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
