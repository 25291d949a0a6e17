// Device-side building blocks shared by the prune24 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace p24 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 32-row blocks of the device layout: M rounded up to whole groups of four
// blocks, so the metadata of one 128-row group for one K-pair is a single
// contiguous 1 KiB piece ([rb / 4][t][rb % 4][lane]).
__host__ __device__ inline int64_t device_row_blocks(int64_t M) { return ((M + 127) / 128) * 4; }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN -> 0x7FC0 | sign.
// Both results are computed and one is selected (no branch).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(uint32_t u) {
  const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rne);
}

// 2-of-4 selection under (magnitude key descending, index ascending).
// Entry i beats entry j (i < j) when key_i >= key_j.  An entry is kept when at
// most one other entry beats it.  Returns p0 | p1 << 2 with p0 < p1 the kept
// positions.
__device__ __forceinline__ uint32_t select_2of4(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  const uint32_t b01 = k0 >= k1, b02 = k0 >= k2, b03 = k0 >= k3;
  const uint32_t b12 = k1 >= k2, b13 = k1 >= k3, b23 = k2 >= k3;
  const uint32_t beaten0 = (1 - b01) + (1 - b02) + (1 - b03);
  const uint32_t beaten1 = b01 + (1 - b12) + (1 - b13);
  const uint32_t beaten2 = b02 + b12 + (1 - b23);
  const uint32_t keep = (beaten0 < 2 ? 1u : 0u) | (beaten1 < 2 ? 2u : 0u) | (beaten2 < 2 ? 4u : 0u) |
                        ((b03 + b13 + b23) < 2 ? 8u : 0u);
  // keep has exactly two bits set
  const uint32_t p0 = __builtin_ctz(keep);
  const uint32_t p1 = __builtin_ctz(keep & (keep - 1));
  return p0 | (p1 << 2);
}

// One group of four as raw bits plus magnitude keys.
template <typename T> struct GroupIO;

template <> struct GroupIO<float> {
  // key = bits with the sign cleared; value cast = RNE to bf16
  static __device__ __forceinline__ uint32_t key(uint32_t bits) { return bits & 0x7FFFFFFFu; }
  static __device__ __forceinline__ uint16_t to_bf16(uint32_t bits) { return f32_to_bf16_rne(bits); }
};
template <> struct GroupIO<uint16_t> {
  static __device__ __forceinline__ uint32_t key(uint32_t bits) { return bits & 0x7FFFu; }
  static __device__ __forceinline__ uint16_t to_bf16(uint32_t bits) { return (uint16_t)bits; }
};

// Compress one group given its four raw bit patterns.  Writes the two kept
// bf16 values and returns the 4-bit position code p0 | p1 << 2.
template <typename T>
__device__ __forceinline__ uint32_t compress_group(const uint32_t b[4], uint16_t& v0, uint16_t& v1) {
  const uint32_t code = select_2of4(GroupIO<T>::key(b[0]), GroupIO<T>::key(b[1]),
                                    GroupIO<T>::key(b[2]), GroupIO<T>::key(b[3]));
  const uint32_t p0 = code & 3u, p1 = code >> 2;
  // select by position with masks (no dynamic register indexing, no branches)
  const uint32_t w0 = (b[0] & (0u - (uint32_t)(p0 == 0))) | (b[1] & (0u - (uint32_t)(p0 == 1))) |
                      (b[2] & (0u - (uint32_t)(p0 == 2)));
  const uint32_t w1 = (b[1] & (0u - (uint32_t)(p1 == 1))) | (b[2] & (0u - (uint32_t)(p1 == 2))) |
                      (b[3] & (0u - (uint32_t)(p1 == 3)));
  v0 = GroupIO<T>::to_bf16(w0);
  v1 = GroupIO<T>::to_bf16(w1);
  return code;
}

// XCD-aware block order.  Workgroups are handed to the 8 XCDs round-robin, so
// block b runs on XCD b % 8.  Renumbering so that each XCD receives one
// contiguous range of logical tiles keeps neighbouring tiles (which share rows
// of W and columns of X) in the same XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
  constexpr uint32_t NXCD = 8;
  const uint32_t per = nblocks / NXCD;          // full rounds
  const uint32_t full = per * NXCD;
  if (b >= full) return b;                      // the ragged last round keeps its ids
  return (b % NXCD) * per + (b / NXCD);
}

}  // namespace p24
