// 2:4 magnitude prune + compress, decompress, dense operand packing and TVW
// column selection (gfx950).  All kernels here are HBM-bound scans.
#include "p24_api_internal.hpp"
#include "p24_device.hpp"

#include <algorithm>
#include <mutex>

namespace p24 {

// --------------------------------------------------------------------------
// Loading one group of four raw bit patterns
// --------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void load_group(const T* p, uint32_t b[4]);

template <> __device__ __forceinline__ void load_group<float>(const float* p, uint32_t b[4]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);   // 16 B aligned by contract
  b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
}
template <> __device__ __forceinline__ void load_group<uint16_t>(const uint16_t* p, uint32_t b[4]) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);   // 8 B aligned by contract
  b[0] = v.x & 0xFFFFu; b[1] = v.x >> 16; b[2] = v.y & 0xFFFFu; b[3] = v.y >> 16;
}

template <typename T> __device__ __forceinline__ uint32_t raw_bits(T v);
template <> __device__ __forceinline__ uint32_t raw_bits<float>(float v) { return __float_as_uint(v); }
template <> __device__ __forceinline__ uint32_t raw_bits<uint16_t>(uint16_t v) { return v; }

// Row m, compacted group g.  Without a gather the group is W[m][4g .. 4g+4);
// with one (TVW) its columns are kept[tile(m)][4g .. 4g+4).
// Gathered columns are clamped into [0, kmax) so that no read leaves the row.
template <typename T, bool GATHER>
__device__ __forceinline__ void fetch_group(const T* __restrict__ W, int64_t ldw, int64_t m, int64_t g,
                                            const int32_t* __restrict__ kept_row, int64_t kmax, uint32_t b[4]) {
  const T* row = W + m * ldw;
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t k = kept_row[4 * g + i];
      k = k < 0 ? 0 : (k >= kmax ? kmax - 1 : k);
      b[i] = raw_bits<T>(row[k]);
    }
  } else {
    load_group<T>(row + 4 * g, b);
  }
}

// The group of four back in place with only positions p0 = code & 3 and
// p1 = code >> 2 kept: the other two become +0 (masked fine-tuning).
template <typename T> __device__ __forceinline__ void store_masked_group(T* p, const uint32_t b[4], uint32_t code);
template <> __device__ __forceinline__ void store_masked_group<float>(float* p, const uint32_t b[4], uint32_t code) {
  const uint32_t p0 = code & 3u, p1 = code >> 2;
  uint32_t o[4];
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i) o[i] = (i == p0 || i == p1) ? b[i] : 0u;
  __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4*>(p));
}
template <> __device__ __forceinline__ void store_masked_group<uint16_t>(uint16_t* p, const uint32_t b[4],
                                                                         uint32_t code) {
  const uint32_t p0 = code & 3u, p1 = code >> 2;
  uint32_t o[4];
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i) o[i] = (i == p0 || i == p1) ? b[i] : 0u;
  __builtin_nontemporal_store(u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)}, reinterpret_cast<u32x2*>(p));
}

// --------------------------------------------------------------------------
// Canonical layout: one thread per (row, metadata word) = 8 groups.
// With WB (re-prune in place) the dropped entries of W are also set to +0:
// W is then read and written through the same rows, hence no restrict on it.
// --------------------------------------------------------------------------
template <typename T, bool GATHER, bool WB = false>
__global__ __launch_bounds__(256) void k_compress_canonical(const T* W, int64_t ldw, int64_t M,
                                                            int64_t K, uint16_t* __restrict__ values,
                                                            uint32_t* __restrict__ meta,
                                                            const int32_t* __restrict__ kept, int64_t tile_m,
                                                            int64_t kmax, T* Wout) {
  const int64_t nw = (K + 31) / 32;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= M * nw) return;
  const int64_t m = id / nw, w = id % nw;
  const int64_t G = K / 4;
  const int32_t* kept_row = GATHER ? kept + (m / tile_m) * K : nullptr;
  uint32_t word = 0;
  uint32_t* vrow = reinterpret_cast<uint32_t*>(values + m * (K / 2));   // 4 B per group
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t g = 8 * w + q;
    if (g < G) {
      uint32_t b[4];
      fetch_group<T, GATHER>(W, ldw, m, g, kept_row, kmax, b);
      uint16_t v0, v1;
      const uint32_t code = compress_group<T>(b, v0, v1);
      vrow[g] = (uint32_t)v0 | ((uint32_t)v1 << 16);
      if constexpr (WB) store_masked_group<T>(Wout + m * ldw + 4 * g, b, code);
      word |= code << (4 * q);
    }
  }
  meta[m * nw + w] = word;
}

// --------------------------------------------------------------------------
// Device layout: one wave per (row block rb, chunk of 256 columns).  Lane l
// owns group 64 c + l of every row, so each row is one contiguous read (1 KiB
// of fp32).  The device layout puts that group at step s = 8 c + l / 8, lane
// half h = (l / 4) % 2, pair q = l % 4 of lane L = r + 32 h of block (rb, s):
// the wave collects its up-to-8 value blocks and 4 metadata blocks in LDS.
// Every 8 rows complete two whole 128 B lines of each value block (lanes r and
// r + 32), which are written right away so that stores interleave with the
// loads; the metadata goes out at the end as contiguous 4 B pieces.
// Staging pads (4 words after every 32 lanes of a block, 8 per block, one
// per metadata row) spread one row's writes over distinct banks.
// Rows M..Mp-1 (Mp = M rounded up to 128) are padding: zero values, positions
// (0, 1).  Every output (values, metadata, the re-pruned weights) is written
// once and read by a later kernel, so it goes out as non-temporal stores that
// do not take L2 space from the weight stream (82 -> 58 us on 8192 x 8192
// fp32, 5.9 TB/s).  Metadata words are stored [rb / 4][t][rb % 4][L]: the four row
// blocks of a group side by side per K-pair, one 1 KiB load for the GEMM.
// --------------------------------------------------------------------------
constexpr int CMP_WAVES = 4;
constexpr int CMP_BLK_WORDS = 264;    // 64 lanes x 4 words + 2 pads of 4
constexpr int CMP_META_PITCH = 65;

// Gather modes: none; one kept list of K columns per tile_m rows; per-tile
// keep counts (128-row tiles, tile t's list and storage start at column
// offsets[t] of the concatenation, its compacted K is offsets[t+1] - offsets[t]).
enum GatherMode { G_NONE = 0, G_FIXED = 1, G_VAR = 2 };

// rq: waves per (row block, chunk); each takes 32 / rq of the block's rows
// (1, or 4 when there are too few (row block, chunk) pairs to fill the chip).
template <typename T, int GM, bool WB = false>
__global__ __launch_bounds__(64 * CMP_WAVES) void k_compress_device(const T* W, int64_t ldw, int64_t M,
                                                                    int64_t K, uint16_t* __restrict__ dvals,
                                                                    uint32_t* __restrict__ dmeta,
                                                                    const int32_t* __restrict__ kept,
                                                                    const int64_t* __restrict__ offsets,
                                                                    int64_t tile_m, int64_t kmax, T* Wout, int rq) {
  constexpr bool GATHER = GM != G_NONE;
  static_assert(!WB || GM == G_NONE, "re-prune in place works on the whole matrix");
  __shared__ uint32_t sv[CMP_WAVES][8 * CMP_BLK_WORDS];
  __shared__ uint32_t sm[CMP_WAVES][4 * CMP_META_PITCH];
  const int64_t RB = device_row_blocks(M);
  const int64_t NC = (K + 255) / 256;    // K: the widest compacted row
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t wq = (int64_t)blockIdx.x * CMP_WAVES + wv;
  if (wq >= RB * NC * rq) return;        // wave-uniform
  const int64_t wid = wq / rq, rb = wid / NC, c = wid % NC;
  const int r_begin = (int)(wq % rq) * (32 / rq), r_end = r_begin + 32 / rq;
  int64_t Kc = K, rbl = rb;              // compacted K, row block inside the storage
  const int32_t* kept_tile = nullptr;
  if constexpr (GM == G_VAR) {
    const int64_t t = rb >> 2, p = offsets[t];
    Kc = offsets[t + 1] - p;
    if (256 * c >= Kc) return;           // wave-uniform: past this tile's columns
    rbl = rb & 3;
    kept_tile = kept + p;
    dvals += p * 64;                     // 128 rows x Kc/2 values per tile
    dmeta += p * 4;                      // 16 B of metadata per kept column
  }
  const int64_t S = Kc / 32, T_ = Kc / 64, G = Kc / 4;
  const int64_t g = 64 * c + lane;
  const bool gv = g < G;
  const int ns = (int)(S - 8 * c < 8 ? S - 8 * c : 8);     // steps in this chunk (even: K % 64 == 0)
  const int sl = lane >> 3, hl = (lane >> 2) & 1, ql = lane & 3;
  uint32_t* vst = sv[wv];
  uint32_t* mst = sm[wv];
  // Branch-free rows: padding rows and lanes past K read a clamped in-range
  // group and then take the padding result (zero values, positions (0, 1)).
  const int64_t g_rd = gv ? g : G - 1;
  u32x4* vout = reinterpret_cast<u32x4*>(dvals + (rbl * S + 8 * c) * 64 * 8);
  // Gathered columns: tile heights are multiples of 32 (the host checks), so
  // the block's 32 rows lie in one tile and the lane's four kept columns are
  // read once; each row's loads then depend on nothing else.  Padding rows
  // read the last row, which lies in the tile of the block's first row.
  int64_t kcol[4] = {0, 0, 0, 0};
  if constexpr (GATHER) {
    const int64_t m_first = rb * 32 < M ? rb * 32 : M - 1;
    const int32_t* kr = GM == G_FIXED ? kept + (m_first / tile_m) * K : kept_tile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k = kr[4 * g_rd + i];
      kcol[i] = k < 0 ? 0 : (k >= kmax ? kmax - 1 : k);
    }
  }
  for (int r0 = r_begin; r0 < r_end; r0 += 8) {
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = r0 + rr;
      const int64_t m = rb * 32 + r;
      const bool live = m < M && gv;
      const int64_t m_rd = m < M ? m : M - 1;
      uint32_t b[4];
      if constexpr (GATHER) {
        const T* row = W + m_rd * ldw;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = raw_bits<T>(row[kcol[i]]);
      } else {
        fetch_group<T, false>(W, ldw, m_rd, g_rd, nullptr, kmax, b);
      }
      uint16_t v0, v1;
      uint32_t code = compress_group<T>(b, v0, v1);
      if constexpr (WB) {
        if (live) store_masked_group<T>(Wout + m * ldw + 4 * g, b, code);
      }
      const uint32_t packed = live ? ((uint32_t)v0 | ((uint32_t)v1 << 16)) : 0u;
      code = live ? code : 0x4u;
      const int L = r + 32 * hl;
      vst[sl * CMP_BLK_WORDS + L * 4 + hl * 4 + ql] = packed;
      // 16-bit code of (step, half): the 4 pairs' nibbles, gathered with DPP
      // lane permutes inside each quad; the metadata word of K-pair t holds step
      // 2t in bits 0-15 and step 2t+1 (the lanes 8 higher) in bits 16-31
      uint32_t c16 = code << (4 * ql);
      c16 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)c16, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]: lane ^ 1
      c16 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)c16, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]: lane ^ 2
      const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)c16, 0x128, 0xF, 0xF, false);  // row_ror:8: lane ^ 8
      if (ql == 0 && (sl & 1) == 0) mst[(sl >> 1) * CMP_META_PITCH + L] = c16 | (hi << 16);
    }
    // rows r0..r0+7 complete lanes r0..r0+7 and r0+32..r0+39 of every block:
    // two whole 128 B lines per block, written now
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = t * 64 + lane, j = q >> 4, idx = q & 15;
      const int L = r0 + (idx & 7) + 32 * (idx >> 3);
      if (j < ns) {
        const uint32_t* e = vst + j * CMP_BLK_WORDS + L * 4 + (L >> 5) * 4;
        __builtin_nontemporal_store(u32x4{e[0], e[1], e[2], e[3]}, &vout[j * 64 + L]);
      }
    }
  }
  // the metadata words of this wave's rows: lanes r and r + 32 for its rows r
  uint32_t* mout = dmeta + (((rbl >> 2) * T_ + 4 * c) * 4 + (rbl & 3)) * 64;
  if ((lane & 31) >= r_begin && (lane & 31) < r_end)
    for (int j = 0; j < ns / 2; ++j) __builtin_nontemporal_store(mst[j * CMP_META_PITCH + lane], &mout[j * 256 + lane]);
}

// --------------------------------------------------------------------------
// Decompress: one thread per (row, group) -> 4 dense bf16 entries.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_decompress(const uint16_t* __restrict__ values,
                                                    const uint32_t* __restrict__ meta, int layout, int64_t M,
                                                    int64_t K, uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t G = K / 4;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= M * G) return;
  const int64_t m = id / G, g = id % G;
  uint32_t code;
  uint16_t v0, v1;
  if (layout == P24_LAYOUT_CANONICAL) {
    const int64_t nw = (K + 31) / 32;
    code = (meta[m * nw + g / 8] >> (4 * (g % 8))) & 0xFu;
    v0 = values[m * (K / 2) + 2 * g];
    v1 = values[m * (K / 2) + 2 * g + 1];
  } else {
    const int64_t S = K / 32, T_ = K / 64;
    const int64_t s = g / 8, h = (g % 8) / 4, q = g % 4;
    const int64_t rb = m / 32, L = m % 32 + 32 * h;
    code = (meta[(((rb >> 2) * T_ + s / 2) * 4 + (rb & 3)) * 64 + L] >> (16 * (s % 2) + 4 * q)) & 0xFu;
    const uint16_t* v = values + ((rb * S + s) * 64 + L) * 8 + 2 * q;
    v0 = v[0];
    v1 = v[1];
  }
  const uint32_t p0 = code & 3u, p1 = code >> 2;
  uint16_t* o = out + m * ldo + 4 * g;
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i) o[i] = (i == p0) ? v0 : ((i == p1) ? v1 : (uint16_t)0);
}

// --------------------------------------------------------------------------
// Masked fine-tuning: W keeps only the positions the stored metadata selects.
// One thread per (row, group): the group's 16 B (fp32) or 8 B (bf16) are read
// and written back with the two unselected entries set to +0.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_mask_apply(T* W, int64_t ldw, int64_t M, int64_t K,
                                                    const uint32_t* __restrict__ meta, int layout) {
  const int64_t G = K / 4;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= M * G) return;
  const int64_t m = id / G, g = id % G;
  uint32_t code;
  if (layout == P24_LAYOUT_CANONICAL) {
    code = (meta[m * ((K + 31) / 32) + g / 8] >> (4 * (g % 8))) & 0xFu;
  } else {
    const int64_t T_ = K / 64, s = g / 8, h = (g % 8) / 4, q = g % 4;
    const int64_t rb = m / 32, L = m % 32 + 32 * h;
    code = (meta[(((rb >> 2) * T_ + s / 2) * 4 + (rb & 3)) * 64 + L] >> (16 * (s % 2) + 4 * q)) & 0xFu;
  }
  T* p = W + m * ldw + 4 * g;
  uint32_t b[4];
  load_group<T>(p, b);
  store_masked_group<T>(p, b, code);
}

// --------------------------------------------------------------------------
// Dense operand packing for the MFMA 32x32x16 bf16 tile loop.
// One thread per (row block, K16 step, lane): one 16 B chunk.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack_dense(const uint16_t* __restrict__ W, int64_t ldw, int64_t M,
                                                    int64_t K, uint16_t* __restrict__ Wp) {
  const int64_t RB = (M + 31) / 32, S = K / 16;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= RB * S * 64) return;
  const int64_t L = id % 64, s = (id / 64) % S, rb = id / (64 * S);
  const int64_t m = rb * 32 + L % 32, k = 16 * s + 8 * (L / 32);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M) v = *reinterpret_cast<const u32x4*>(W + m * ldw + k);
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Wp + id * 8));
}

// --------------------------------------------------------------------------
// TVW column scores: one thread per (tile, column); fp64 sum of |W| over the
// tile's rows, one row at a time in ascending order (fixed order -> the same
// correctly rounded sums as a sequential host loop).
// A NaN sum is stored as the one quiet NaN 0x7FF8000000000000: IEEE 754 does
// not fix the payload an addition passes on, and the selections rank scores by
// their bit patterns, so every NaN score must carry the same bits (above
// +Inf; NaN columns then tie and go to the lower index).
// --------------------------------------------------------------------------
// The state of a global radix select (the per-tile-keep cut, the
// unstructured plan), kept in the caller's workspace between its launches.
template <int BINS>
struct VarSel {
  uint64_t prefix;        // the cut's digits found so far
  int64_t need;           // rank of the cut among the keys matching the prefix
  uint32_t ticket;        // blocks done in the current pass
  uint32_t done;          // a pass found the cut's bin kept whole: later passes do nothing
  uint32_t hist[BINS];    // digit histogram of the current pass
};
// 8-bit digits (the unstructured plan's four passes over 32-bit keys) and
// 11-bit digits (the per-tile-keep cut over 64-bit scores: six passes of
// 11, 11, 11, 11, 11 and 9 bits instead of eight of 8; each pass is one launch)
using VarSelect = VarSel<256>;
constexpr int VAR_DIGIT = 11;
using VarSelectW = VarSel<1 << VAR_DIGIT>;
constexpr int VAR_THREADS = 256;
constexpr int64_t VAR_STEP = 64;

// A fresh select state, by the threads tid = 0 .. nthreads-1 of one block.
template <int BINS>
__device__ __forceinline__ void var_init(VarSel<BINS>* vs, int64_t total_keep, int tid, int nthreads) {
  for (int i = tid; i < BINS; i += nthreads) vs->hist[i] = 0u;
  if (tid == 0) {
    vs->prefix = 0ull;
    vs->need = total_keep;
    vs->ticket = 0u;
    vs->done = 0u;
  }
}

__device__ __forceinline__ double canonical_score(double s) {
  return s != s ? __longlong_as_double(0x7FF8000000000000ll) : s;
}

// vs (optional): a per-tile-keep select state that block 0 initialises for the
// digit passes that follow (one launch less).
__global__ __launch_bounds__(256) void k_tvw_scores(const float* __restrict__ W, int64_t ldw, int64_t M,
                                                    int64_t K, int64_t tile_m, double* __restrict__ scores,
                                                    VarSelectW* __restrict__ vs, int64_t total_keep) {
  if (vs != nullptr && blockIdx.x == 0) var_init(vs, total_keep, (int)threadIdx.x, (int)blockDim.x);
  const int64_t T_ = (M + tile_m - 1) / tile_m;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= T_ * K) return;
  const int64_t t = id / K, k = id % K;
  const int64_t r1 = (t + 1) * tile_m < M ? (t + 1) * tile_m : M;
  double acc = 0.0;
  int64_t m = t * tile_m;
  for (; m + 16 <= r1; m += 16) {        // 16 loads in flight, then the adds in row order
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = W[(m + u) * ldw + k];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc = acc + fabs((double)v[u]);
  }
  for (; m < r1; ++m) acc = acc + fabs((double)W[m * ldw + k]);
  scores[id] = canonical_score(acc);
}

// The same scores four columns per thread with 16-byte loads (K and the row
// stride multiples of 4, W 16-byte aligned); each column's sum still runs
// over its rows in order.
__global__ __launch_bounds__(256) void k_tvw_scores4(const float* __restrict__ W, int64_t ldw, int64_t M,
                                                     int64_t K, int64_t tile_m, double* __restrict__ scores,
                                                     VarSelectW* __restrict__ vs, int64_t total_keep) {
  if (vs != nullptr && blockIdx.x == 0) var_init(vs, total_keep, (int)threadIdx.x, (int)blockDim.x);
  const int64_t T_ = (M + tile_m - 1) / tile_m, K4 = K / 4;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= T_ * K4) return;
  const int64_t t = id / K4, k = 4 * (id % K4);
  const int64_t r1 = (t + 1) * tile_m < M ? (t + 1) * tile_m : M;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t m = t * tile_m;
  for (; m + 8 <= r1; m += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(W + (m + u) * ldw + k);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc[0] = acc[0] + fabs((double)v[u].x);
      acc[1] = acc[1] + fabs((double)v[u].y);
      acc[2] = acc[2] + fabs((double)v[u].z);
      acc[3] = acc[3] + fabs((double)v[u].w);
    }
  }
  for (; m < r1; ++m) {
    const float4 v = *reinterpret_cast<const float4*>(W + m * ldw + k);
    acc[0] = acc[0] + fabs((double)v.x);
    acc[1] = acc[1] + fabs((double)v.y);
    acc[2] = acc[2] + fabs((double)v.z);
    acc[3] = acc[3] + fabs((double)v.w);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) scores[t * K + k + c] = canonical_score(acc[c]);
}


// --------------------------------------------------------------------------
// TVW selection: one block per tile.  The kept set is the keep_k largest
// scores, ties to the lower column.  Scores are non-negative fp64 sums with
// one NaN pattern, so their bit patterns order like the values (NaN above
// +Inf).  An MSB-first radix select (up to six passes of 11-bit digits, a
// 2048-bin histogram over the keys that still match the prefix found so far)
// finds the keep_k-th largest key v and how many of the keys equal to v are
// kept; a block-wide scan in column order then writes every column with
// key > v and the first `need` columns with key == v.
// --------------------------------------------------------------------------
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_DIGIT = 11;            // select digits: 11, 11, 11, 11, 11 and 9 bits from the top
constexpr int64_t SEL_LDS_KEYS = 8192;   // 64 KiB of fp64 keys per block

// Exclusive block-wide prefix of per-thread counts in thread order (blocks of
// SEL_THREADS); returns this thread's prefix and writes the block total.
template <typename U>
__device__ __forceinline__ int64_t block_exclusive_scan(U v, int64_t* total, U* wave_sums) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  U incl = v;
  static_assert(sizeof(U) == 4 || sizeof(U) == 8, "32- or 64-bit counts");
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const U o = __shfl_up(incl, d);      // full width: 64-bit partial sums stay whole
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < SEL_WAVES; ++w) {
    if (w < wave) before += wave_sums[w];
    all += wave_sums[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Lane l of one wave holds bins 4l .. 4l+3 of a 256-bin digit histogram.
// The need-th largest key (need >= 1, at most the histogram total) has the
// digit d at which the keys of bins >= d first reach `need`; the lane that
// owns d returns true with d and that key's rank among the keys of bin d.
__device__ __forceinline__ bool find_cut(const uint32_t (&hb)[4], int64_t need, int l, int* digit, int64_t* rest,
                                         uint32_t* bin = nullptr) {
  const uint32_t own = hb[0] + hb[1] + hb[2] + hb[3];
  uint32_t incl = own;                 // inclusive suffix sum over lanes l .. 63
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_down(incl, d);
    if (l + d < 64) incl += o;
  }
  const int64_t above = incl - own;
  if (!(above < need && above + own >= need)) return false;
  // the cut lies in this lane's bins: walk them from the highest
  int64_t a = above;
  int d = 4 * l + 3;
  uint32_t cnt = hb[3];
  for (int i = 3; i > 0 && a + hb[i] < need; --i) {
    a += hb[i];
    --d;
    cnt = hb[i - 1];
  }
  *digit = d;
  *rest = need - a;
  if (bin) *bin = cnt;
  return true;
}

__global__ __launch_bounds__(SEL_THREADS) void k_tvw_select(const double* __restrict__ scores, int64_t K,
                                                            int64_t keep_k, const int64_t* __restrict__ offsets,
                                                            int32_t* __restrict__ kept) {
  constexpr int BINS = 1 << SEL_DIGIT, PER = BINS / SEL_THREADS;
  __shared__ uint32_t hist[BINS];
  __shared__ uint32_t wave_sums[SEL_WAVES];
  __shared__ uint64_t sh_prefix;
  __shared__ int64_t sh_need;
  __shared__ uint32_t sh_whole;
  __shared__ uint64_t skey[SEL_LDS_KEYS];
  const int64_t t = blockIdx.x;
  const uint64_t* gkey = reinterpret_cast<const uint64_t*>(scores + t * K);
  const int tid = threadIdx.x;
  // A tile's keys are read from memory once into LDS when they fit (every
  // pass below then reads LDS), else each pass reads them from memory.
  const bool in_lds = K <= SEL_LDS_KEYS;
  if (in_lds) {
    for (int64_t k = tid; k < K; k += SEL_THREADS) skey[k] = gkey[k];
    __syncthreads();
  }
  auto key = [&](int64_t k) -> uint64_t { return in_lds ? skey[k] : gkey[k]; };
  // per-tile keep counts: this tile's count and list position from the offsets
  int32_t* kept_out = kept + t * keep_k;
  if (offsets) {
    keep_k = offsets[t + 1] - offsets[t];
    kept_out = kept + offsets[t];
  }
  uint64_t prefix = 0;        // digits of the threshold found so far (high bits)
  int64_t need = keep_k;      // rank of the threshold among keys matching the prefix
  for (int top = 64; top > 0; top -= SEL_DIGIT) {
    const int width = top < SEL_DIGIT ? top : SEL_DIGIT, shift = top - width;
    for (int i = tid; i < BINS; i += SEL_THREADS) hist[i] = 0u;
    __syncthreads();
    const uint64_t hi_mask = top == 64 ? 0ull : (~0ull << top);
    const uint32_t dmask = (1u << width) - 1u;
    // A tile's keys mostly share their high digits: when every matching key
    // of a wave has the same digit, one lane adds them all (one LDS address
    // hit by each lane in turn would serialise the wave).
    for (int64_t k0 = 0; k0 < K; k0 += SEL_THREADS) {
      const int64_t k = k0 + tid;
      const uint64_t x = k < K ? key(k) : 0ull;
      const bool match = k < K && (x & hi_mask) == prefix;
      const uint32_t d = (uint32_t)(x >> shift) & dmask;
      const uint64_t mm = __ballot(match);
      if (!mm) continue;                                    // wave-uniform
      const int l0 = __builtin_ffsll((long long)mm) - 1;
      const uint32_t d0 = (uint32_t)__shfl((int)d, l0);
      if (__ballot(match && d == d0) == mm) {
        if ((tid & 63) == l0) atomicAdd(&hist[d0], (uint32_t)__builtin_popcountll(mm));
      } else if (match) {
        atomicAdd(&hist[d], 1u);
      }
    }
    __syncthreads();
    // Thread tid holds the digits [PER tid, PER tid + PER): a suffix sum over
    // the threads (higher digits first: the lanes of a wave, then the waves)
    // gives the count above them; the one thread whose digits hold the rank
    // `need` walks them from the highest.
    uint32_t hb[PER], own = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      hb[i] = hist[PER * tid + i];
      own += hb[i];
    }
    const int lane = tid & 63, wv = tid >> 6;
    uint32_t incl = own;
#pragma unroll
    for (int dd = 1; dd < 64; dd <<= 1) {
      const uint32_t o = __shfl_down(incl, dd);
      if (lane + dd < 64) incl += o;
    }
    if (lane == 0) wave_sums[wv] = incl;
    __syncthreads();
    int64_t above = (int64_t)incl - own;
    for (int w = wv + 1; w < SEL_WAVES; ++w) above += wave_sums[w];
    if (above < need && above + own >= need) {
      int64_t a = above;
      int dsel = PER * tid;
      uint32_t bin = hb[0];
      bool found = false;
#pragma unroll
      for (int i = PER - 1; i >= 0; --i) {
        if (!found) {
          if (a + hb[i] >= need) {
            dsel = PER * tid + i;
            bin = hb[i];
            found = true;
          } else {
            a += hb[i];
          }
        }
      }
      sh_prefix = prefix | ((uint64_t)dsel << shift);
      sh_need = need - a;
      sh_whole = need - a == (int64_t)bin ? 1u : 0u;
    }
    __syncthreads();
    prefix = sh_prefix;
    need = sh_need;
    // Every key of the cut's bin is kept: the kept set is then every key >= the
    // bin's lowest value (prefix, lower bits zero), which the scan below takes
    // as the keys above prefix plus all keys equal to it.  No later digit can
    // change that set, so the remaining passes are skipped.
    if (sh_whole) {
      need = K;
      break;
    }
  }
  // prefix is the threshold key; `need` columns equal to it are kept, lowest
  // first.  Thread tid takes the columns [tid * C, tid * C + C): a scan of the
  // per-thread counts of keys equal to the threshold gives each thread the rank
  // of its first such key, a second scan of the kept counts its first output
  // position, and the thread then writes its kept columns in order.
  const int64_t C = (K + SEL_THREADS - 1) / SEL_THREADS;
  const int64_t k_lo = tid * C < K ? tid * C : K, k_hi = k_lo + C < K ? k_lo + C : K;
  uint32_t n_gt = 0, n_eq = 0;
  for (int64_t k = k_lo; k < k_hi; ++k) {
    const uint64_t x = key(k);
    n_gt += x > prefix ? 1u : 0u;
    n_eq += x == prefix ? 1u : 0u;
  }
  int64_t total;
  const int64_t eq_rank0 = block_exclusive_scan<uint32_t>(n_eq, &total, wave_sums);
  const int64_t eq_kept = need - eq_rank0 <= 0 ? 0 : (need - eq_rank0 < n_eq ? need - eq_rank0 : n_eq);
  int64_t pos = block_exclusive_scan<uint32_t>(n_gt + (uint32_t)eq_kept, &total, wave_sums);
  int64_t eq_left = eq_kept;
  for (int64_t k = k_lo; k < k_hi; ++k) {
    const uint64_t x = key(k);
    const bool keep = x > prefix || (x == prefix && eq_left-- > 0);
    if (keep && pos < keep_k) kept_out[pos] = (int32_t)k;   // exactly keep_k keys are kept; the bound is a guard
    pos += keep ? 1 : 0;
  }
}

// --------------------------------------------------------------------------
// TVW with per-tile keep counts (128-row tiles).  Every (tile, column) score
// of the matrix is ranked, score descending and then flat index t*K + k
// ascending, and the top total_keep are taken; tile t keeps its number of
// those rounded to a multiple of 64 (halves up), clamped to [64, K].
//   * the global cut: the same MSB-first radix select as above, over all T*K
//     keys, with 11-bit digits; one launch per digit (six), each block adds
//     its LDS histogram to a global one and the last block to finish picks
//     the digit;
//   * per tile: keys above the cut and keys equal to it; the equal keys are
//     taken in flat order, so tile t gets min(eq_t, need - (eq of tiles < t));
//   * keep counts, their running sum (the tiles' column offsets in the
//     concatenated storage) and the order of the tiles by count, heaviest first.
// --------------------------------------------------------------------------
template <int BINS>
__global__ __launch_bounds__(VAR_THREADS) void k_var_init(VarSel<BINS>* __restrict__ vs, int64_t total_keep) {
  var_init(vs, total_keep, (int)threadIdx.x, VAR_THREADS);
}

// One digit pass of the global cut: digit (x >> shift) & (2^width - 1) of the
// keys whose higher digits equal the prefix found so far.
__global__ __launch_bounds__(VAR_THREADS) void k_var_radix(const uint64_t* __restrict__ keys, int64_t n, int shift,
                                                           int width, VarSelectW* __restrict__ vs) {
  constexpr int BINS = 1 << VAR_DIGIT, PER = BINS / VAR_THREADS, NW = VAR_THREADS / 64;
  __shared__ uint32_t h[BINS];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t last;
  // An earlier pass kept the cut's whole bin: the prefix found so far already
  // separates the kept keys (every key >= it), so no digit is left to pick.
  if (vs->done) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t prefix = vs->prefix;
  const int64_t need = vs->need;
  for (int i = tid; i < BINS; i += VAR_THREADS) h[i] = 0u;
  __syncthreads();
  const uint64_t hi_mask = shift + width >= 64 ? 0ull : (~0ull << (shift + width));
  const uint32_t dmask = (1u << width) - 1u;
  // as in the per-tile select: a wave whose matching keys share one digit adds
  // them with one atomic
  for (int64_t i0 = (int64_t)blockIdx.x * VAR_THREADS; i0 < n; i0 += (int64_t)gridDim.x * VAR_THREADS) {
    const int64_t i = i0 + tid;
    const uint64_t x = i < n ? keys[i] : 0ull;
    const bool match = i < n && (x & hi_mask) == prefix;
    const uint32_t d = (uint32_t)(x >> shift) & dmask;
    const uint64_t mm = __ballot(match);
    if (!mm) continue;                                      // wave-uniform
    const int l0 = __builtin_ffsll((long long)mm) - 1;
    const uint32_t d0 = (uint32_t)__shfl((int)d, l0);
    if (__ballot(match && d == d0) == mm) {
      if (lane == l0) atomicAdd(&h[d0], (uint32_t)__builtin_popcountll(mm));
    } else if (match) {
      atomicAdd(&h[d], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < BINS; i += VAR_THREADS)
    if (h[i]) atomicAdd(&vs->hist[i], h[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(&vs->ticket, 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!last) return;
  // The last block sees every block's histogram.  Thread tid holds the
  // digits [PER tid, PER tid + PER); a suffix sum over the threads (higher
  // digits first) gives the count above each thread's digits, and the one
  // thread whose digits hold the rank `need` walks them from the highest.
  // Then the histogram and the ticket are cleared for the next pass.
  __threadfence();
  uint32_t hb[PER];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    hb[i] = __hip_atomic_load(&vs->hist[PER * tid + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    own += hb[i];
  }
  uint32_t incl = own;                  // inclusive suffix sum over the wave's lanes lane .. 63
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_down(incl, d);
    if (lane + d < 64) incl += o;
  }
  if (lane == 0) wsum[wave] = incl;     // the wave's total
  __syncthreads();
  int64_t above = (int64_t)incl - own;
  for (int w = wave + 1; w < NW; ++w) above += wsum[w];
  if (above < need && above + own >= need) {
    int64_t a = above;
    int dsel = PER * tid;
    uint32_t bin = hb[0];
    bool found = false;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (!found) {
        if (a + hb[i] >= need) {
          dsel = PER * tid + i;
          bin = hb[i];
          found = true;
        } else {
          a += hb[i];
        }
      }
    }
    vs->prefix = prefix | ((uint64_t)dsel << shift);
    // Every key of the cut's bin is kept: the kept keys are then those >= the
    // bin's lowest value (the prefix, lower bits zero), i.e. the keys above it
    // and all keys equal to it (need = n takes every equal key).
    const bool whole = need - a == (int64_t)bin;
    vs->need = whole ? n : need - a;
    if (whole) vs->done = 1u;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) vs->hist[PER * tid + i] = 0u;
  if (tid == 0) vs->ticket = 0u;
}

// keys of tile t above the cut and equal to it; one block per tile
__global__ __launch_bounds__(VAR_THREADS) void k_var_tile_counts(const uint64_t* __restrict__ keys, int64_t K,
                                                                 const VarSelectW* __restrict__ vs,
                                                                 int32_t* __restrict__ gt, int32_t* __restrict__ eq) {
  __shared__ uint32_t sg[VAR_THREADS / 64], se[VAR_THREADS / 64];
  const int64_t t = blockIdx.x;
  const uint64_t v = vs->prefix;
  const uint64_t* key = keys + t * K;
  uint32_t g = 0, e = 0;
  for (int64_t k = threadIdx.x; k < K; k += VAR_THREADS) {
    const uint64_t x = key[k];
    g += x > v ? 1u : 0u;
    e += x == v ? 1u : 0u;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    g += __shfl_xor(g, d);
    e += __shfl_xor(e, d);
  }
  if ((threadIdx.x & 63) == 0) {
    sg[threadIdx.x >> 6] = g;
    se[threadIdx.x >> 6] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t G = 0, E = 0;
    for (int w = 0; w < VAR_THREADS / 64; ++w) {
      G += sg[w];
      E += se[w];
    }
    gt[t] = (int32_t)G;
    eq[t] = (int32_t)E;
  }
}

// keep counts and their offsets; one block of SEL_THREADS.  With order given
// (T <= SEL_THREADS: one tile per thread) also the order of the tiles, as
// k_var_order computes it.
__global__ __launch_bounds__(SEL_THREADS) void k_var_plan(int64_t T, int64_t K, const VarSelectW* __restrict__ vs,
                                                          const int32_t* __restrict__ gt,
                                                          const int32_t* __restrict__ eq,
                                                          int64_t* __restrict__ offsets, int32_t* __restrict__ order) {
  __shared__ int64_t wave_sums[SEL_WAVES];
  __shared__ int64_t sk[SEL_THREADS];
  const int64_t need = vs->need;
  int64_t eq_base = 0, off_base = 0, my_keep = 0;
  for (int64_t t0 = 0; t0 < T; t0 += SEL_THREADS) {
    const int64_t t = t0 + threadIdx.x;
    const bool live = t < T;
    const int64_t e = live ? eq[t] : 0;
    int64_t eq_total, keep_total;
    const int64_t before = eq_base + block_exclusive_scan<int64_t>(e, &eq_total, wave_sums);
    int64_t take = need - before;
    take = take < 0 ? 0 : (take > e ? e : take);
    const int64_t c = live ? gt[t] + take : 0;
    int64_t keep = VAR_STEP * ((c + VAR_STEP / 2) / VAR_STEP);
    keep = keep < VAR_STEP ? VAR_STEP : (keep > K ? K : keep);
    keep = live ? keep : 0;
    const int64_t off = off_base + block_exclusive_scan<int64_t>(keep, &keep_total, wave_sums);
    if (live) offsets[t] = off;
    eq_base += eq_total;
    off_base += keep_total;
    my_keep = keep;
  }
  if (threadIdx.x == 0) offsets[T] = off_base;
  if (order != nullptr) {
    // rank r = the tiles with a larger count, or an equal count and a lower index
    sk[threadIdx.x] = my_keep;
    __syncthreads();
    const int64_t t = threadIdx.x;
    if (t < T) {
      int64_t rank = 0;
      for (int64_t u = 0; u < T; ++u) {
        const int64_t cu = sk[u];
        rank += (cu > my_keep || (cu == my_keep && u < t)) ? 1 : 0;
      }
      order[rank] = (int32_t)t;
    }
  }
}

// order[r] = the tile of rank r by keep count descending, then tile ascending
__global__ __launch_bounds__(VAR_THREADS) void k_var_order(const int64_t* __restrict__ offsets, int64_t T,
                                                           int32_t* __restrict__ order) {
  __shared__ int64_t sc[VAR_THREADS];
  const int64_t t = (int64_t)blockIdx.x * VAR_THREADS + threadIdx.x;
  const int64_t ct = t < T ? offsets[t + 1] - offsets[t] : 0;
  int64_t rank = 0;
  for (int64_t u0 = 0; u0 < T; u0 += VAR_THREADS) {
    const int64_t u = u0 + threadIdx.x;
    sc[threadIdx.x] = u < T ? offsets[u + 1] - offsets[u] : 0;
    __syncthreads();
    const int64_t n = T - u0 < VAR_THREADS ? T - u0 : VAR_THREADS;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t cu = sc[i];
      rank += (cu > ct || (cu == ct && u0 + i < t)) ? 1 : 0;
    }
    __syncthreads();
  }
  if (t < T) order[rank] = (int32_t)t;
}

// --------------------------------------------------------------------------
// TW: a tile's rows on its kept columns, rounded to bf16, in the dense MFMA
// operand order (block (rb, s) of 64 lanes x 8 values, lane L holding row
// 32 rb + L % 32, columns 16 s + 8 (L / 32) .. +8).  One thread per (row, 8
// consecutive kept columns): its 8 gathered reads walk one row in ascending
// column order and its result is one 16 B store.  With one kept list per tile
// (VAR false) the rows are padded to 32 and row m uses kept[m / tile_m][0 ..
// Kc); with per-tile counts each 128-row tile is laid out on its own from
// element 128 * offsets[t] and Kc is the widest tile (K).  Padding rows are zero.
// --------------------------------------------------------------------------
template <bool VAR>
__global__ __launch_bounds__(256) void k_pack_tw(const float* __restrict__ W, int64_t ldw, int64_t M, int64_t K,
                                                 int64_t Kc, const int32_t* __restrict__ kept,
                                                 const int64_t* __restrict__ offsets, int64_t tile_m, int64_t rows,
                                                 uint16_t* __restrict__ Wp) {
  const int64_t C8 = Kc / 8;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= rows * C8) return;
  const int64_t m = id / C8, j8 = id % C8;
  int64_t kc = Kc, r = m;
  const int32_t* kr;
  uint16_t* out = Wp;
  if constexpr (VAR) {
    const int64_t t = m / 128, p = offsets[t];
    kc = offsets[t + 1] - p;
    if (8 * j8 >= kc) return;
    kr = kept + p;
    r = m % 128;
    out += p * 128;               // 128 rows x kc bf16 per tile
  } else {
    kr = kept + (m < M ? m / tile_m : 0) * Kc;
  }
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t k = kr[8 * j8 + i];
      k = k < 0 ? 0 : (k >= K ? K - 1 : k);
      b[i] = f32_to_bf16_rne(__float_as_uint(W[m * ldw + k]));
    }
    v = u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
  }
  const int64_t S = kc / 16, rb = r / 32, st = j8 / 2, L = 32 * (j8 % 2) + r % 32;
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + ((rb * S + st) * 64 + L) * 8));
}

// --------------------------------------------------------------------------
// Comparison patterns.
// BW: the score of block (tile t, 64 columns j) is the fp64 sum of the tile's
// column scores 64j .. 64j+63 in ascending order (one thread per block); the
// kept blocks (k_tvw_select over the block scores) expand to their columns.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bw_block_scores(const double* __restrict__ scores, int64_t T, int64_t K,
                                                         double* __restrict__ bscores) {
  const int64_t nb = K / 64;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= T * nb) return;
  const int64_t t = id / nb, j = id % nb;
  const double* sc = scores + t * K + 64 * j;
  double acc = 0.0;
  for (int c = 0; c < 64; ++c) acc = acc + sc[c];
  bscores[id] = canonical_score(acc);
}

__global__ __launch_bounds__(256) void k_bw_expand(const int32_t* __restrict__ kept_blocks, int64_t T,
                                                   int64_t keep_blocks, int32_t* __restrict__ kept) {
  const int64_t n = keep_blocks * 64;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= T * n) return;
  const int64_t t = id / n, i = id % n;
  kept[id] = kept_blocks[t * keep_blocks + i / 64] * 64 + (int32_t)(i % 64);
}

// EW: the magnitude keys (sign-cleared fp32 bits) of the whole matrix; the
// same MSB-first radix select as the per-tile-keep plan (4 digit passes), then
// per row the keys above the cut and equal to it, the row pointers (equal keys
// taken in row-major order), and a per-row compaction into CSR.
__device__ __forceinline__ uint32_t ew_key(const float* W, int64_t ldw, int64_t K, int64_t i) {
  return __float_as_uint(W[(i / K) * ldw + i % K]) & 0x7FFFFFFFu;
}

__global__ __launch_bounds__(VAR_THREADS) void k_ew_radix(const float* __restrict__ W, int64_t ldw, int64_t M,
                                                          int64_t K, int shift, VarSelect* __restrict__ vs) {
  __shared__ uint32_t h[256];
  __shared__ uint32_t last;
  const int tid = threadIdx.x;
  const uint64_t prefix = vs->prefix;
  const int64_t need = vs->need;
  h[tid] = 0u;
  __syncthreads();
  const uint64_t hi_mask = shift == 24 ? 0ull : (0xFFFFFFFFull << (shift + 8)) & 0xFFFFFFFFull;
  const int64_t n = M * K;
  for (int64_t i = (int64_t)blockIdx.x * VAR_THREADS + tid; i < n; i += (int64_t)gridDim.x * VAR_THREADS) {
    const uint64_t x = ew_key(W, ldw, K, i);
    if ((x & hi_mask) == prefix) atomicAdd(&h[(x >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (h[tid]) atomicAdd(&vs->hist[tid], h[tid]);
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(&vs->ticket, 1u) == gridDim.x - 1 ? 1u : 0u;
  __syncthreads();
  if (!last) return;
  __threadfence();
  if (tid < 64) {
    uint32_t hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      hb[i] = __hip_atomic_load(&vs->hist[4 * tid + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int d;
    int64_t rest;
    if (find_cut(hb, need, tid, &d, &rest)) {
      vs->prefix = prefix | ((uint64_t)d << shift);
      vs->need = rest;
    }
  }
  __syncthreads();
  vs->hist[tid] = 0u;
  if (tid == 0) vs->ticket = 0u;
}

__global__ __launch_bounds__(VAR_THREADS) void k_ew_row_counts(const float* __restrict__ W, int64_t ldw, int64_t K,
                                                               const VarSelect* __restrict__ vs,
                                                               int32_t* __restrict__ gt, int32_t* __restrict__ eq) {
  __shared__ uint32_t sg[VAR_THREADS / 64], se[VAR_THREADS / 64];
  const int64_t m = blockIdx.x;
  const uint32_t v = (uint32_t)vs->prefix;
  const float* row = W + m * ldw;
  uint32_t g = 0, e = 0;
  for (int64_t k = threadIdx.x; k < K; k += VAR_THREADS) {
    const uint32_t x = __float_as_uint(row[k]) & 0x7FFFFFFFu;
    g += x > v ? 1u : 0u;
    e += x == v ? 1u : 0u;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    g += __shfl_xor(g, d);
    e += __shfl_xor(e, d);
  }
  if ((threadIdx.x & 63) == 0) {
    sg[threadIdx.x >> 6] = g;
    se[threadIdx.x >> 6] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t G = 0, E = 0;
    for (int w = 0; w < VAR_THREADS / 64; ++w) {
      G += sg[w];
      E += se[w];
    }
    gt[m] = (int32_t)G;
    eq[m] = (int32_t)E;
  }
}

// row pointers; eq[m] is replaced by the number of row m's equal keys taken
__global__ __launch_bounds__(SEL_THREADS) void k_ew_plan(int64_t M, const VarSelect* __restrict__ vs,
                                                         const int32_t* __restrict__ gt, int32_t* __restrict__ eq,
                                                         int64_t* __restrict__ row_ptr) {
  __shared__ int64_t wave_sums[SEL_WAVES];
  const int64_t need = vs->need;
  int64_t eq_base = 0, off_base = 0;
  for (int64_t m0 = 0; m0 < M; m0 += SEL_THREADS) {
    const int64_t m = m0 + threadIdx.x;
    const bool live = m < M;
    const int64_t e = live ? eq[m] : 0;
    int64_t eq_total, cnt_total;
    const int64_t before = eq_base + block_exclusive_scan<int64_t>(e, &eq_total, wave_sums);
    int64_t take = need - before;
    take = take < 0 ? 0 : (take > e ? e : take);
    const int64_t cnt = live ? gt[m] + take : 0;
    const int64_t off = off_base + block_exclusive_scan<int64_t>(cnt, &cnt_total, wave_sums);
    if (live) {
      row_ptr[m] = off;
      eq[m] = (int32_t)take;
    }
    eq_base += eq_total;
    off_base += cnt_total;
  }
  if (threadIdx.x == 0) row_ptr[M] = off_base;
}

__global__ __launch_bounds__(SEL_THREADS) void k_ew_compact(const float* __restrict__ W, int64_t ldw, int64_t K,
                                                            const VarSelect* __restrict__ vs,
                                                            const int32_t* __restrict__ take,
                                                            const int64_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ cols, uint16_t* __restrict__ vals) {
  __shared__ uint32_t wave_sums[SEL_WAVES];
  const int64_t m = blockIdx.x;
  const uint32_t v = (uint32_t)vs->prefix;
  const int64_t need = take[m];
  const float* row = W + m * ldw;
  int64_t eq_base = 0, out_base = row_ptr[m];
  for (int64_t k0 = 0; k0 < K; k0 += SEL_THREADS) {
    const int64_t k = k0 + threadIdx.x;
    const uint32_t bits = k < K ? __float_as_uint(row[k]) : 0u;
    const uint32_t x = bits & 0x7FFFFFFFu;
    const bool gt = k < K && x > v;
    const bool eqk = k < K && x == v;
    int64_t eq_total, keep_total;
    const int64_t eq_rank = eq_base + block_exclusive_scan<uint32_t>(eqk ? 1u : 0u, &eq_total, wave_sums);
    const bool keep = gt || (eqk && eq_rank < need);
    const int64_t pos = out_base + block_exclusive_scan<uint32_t>(keep ? 1u : 0u, &keep_total, wave_sums);
    if (keep) {
      cols[pos] = (int32_t)k;
      vals[pos] = f32_to_bf16_rne(bits);
    }
    eq_base += eq_total;
    out_base += keep_total;
  }
}

}  // namespace p24

// ============================================================================
// C ABI
// ============================================================================
using namespace p24;

static inline unsigned grid1d(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

// vs (optional): a per-tile-keep select state to initialise with need =
// total_keep (the scores launch has at least one block).
static void launch_tvw_scores(const float* W, int64_t ldw, int64_t M, int64_t K, int64_t tile_m, double* scores,
                              hipStream_t st, VarSelectW* vs = nullptr, int64_t total_keep = 0) {
  const int64_t T_ = (M + tile_m - 1) / tile_m;
  // blocks of 128 threads: on 4096 x 4096 (tile 128) that is 256 blocks, one
  // per CU; measured 14.2 -> 12.0 us against 128 blocks of 256 threads (512
  // blocks of 64 threads: 18.8 us)
  if (K % 4 == 0 && ldw % 4 == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0)
    hipLaunchKernelGGL(k_tvw_scores4, dim3(grid1d(T_ * (K / 4), 128)), dim3(128), 0, st, W, ldw, M, K, tile_m, scores,
                       vs, total_keep);
  else
    hipLaunchKernelGGL(k_tvw_scores, dim3(grid1d(T_ * K, 256)), dim3(256), 0, st, W, ldw, M, K, tile_m, scores, vs,
                       total_keep);
}

extern "C" P24_API size_t prune24_values_bytes(int64_t M, int64_t K, int32_t layout) {
  if (M < 0 || K < 0 || K % 4) return 0;
  if (layout == P24_LAYOUT_CANONICAL) return (size_t)M * (size_t)(K / 2) * 2;
  if (layout == P24_LAYOUT_DEVICE) {
    if (K % 64) return 0;
    return (size_t)device_row_blocks(M) * 32 * (size_t)(K / 2) * 2;
  }
  return 0;
}

extern "C" P24_API size_t prune24_meta_bytes(int64_t M, int64_t K, int32_t layout) {
  if (M < 0 || K < 0 || K % 4) return 0;
  if (layout == P24_LAYOUT_CANONICAL) return (size_t)M * (size_t)((K + 31) / 32) * 4;
  if (layout == P24_LAYOUT_DEVICE) {
    if (K % 64) return 0;
    return (size_t)device_row_blocks(M) * (size_t)(K / 64) * 64 * 4;
  }
  return 0;
}

static p24_status check_compress_args(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                      const void* values, const void* meta, int32_t layout) {
  if (w_dtype != P24_F32 && w_dtype != P24_BF16) return P24_ERR_DTYPE;
  if (layout != P24_LAYOUT_CANONICAL && layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (M < 0 || K < 0 || K % 4 || ldw < K) return P24_ERR_SHAPE;
  if (M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (layout == P24_LAYOUT_DEVICE && K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return P24_OK;
  if (!W || !values || !meta) return P24_ERR_NULL;
  const size_t wal = w_dtype == P24_F32 ? 16 : 8;
  if (!aligned(W, wal) || ldw % 4 || !aligned(values, 16) || !aligned(meta, 16)) return P24_ERR_ALIGN;
  return P24_OK;
}

template <int GM, bool WB = false>
static p24_status launch_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                  void* values, void* meta, int32_t layout, const int32_t* kept,
                                  int64_t tile_m, int64_t kmax, hipStream_t st, const int64_t* offsets = nullptr) {
  constexpr bool GATHER = GM != G_NONE;
  // WB: W is written back in place (dropped entries -> +0)
  if (M == 0 || K == 0) return P24_OK;
  if (layout == P24_LAYOUT_CANONICAL) {
    const int64_t n = M * ((K + 31) / 32);
    if (w_dtype == P24_F32)
      hipLaunchKernelGGL((k_compress_canonical<float, GATHER, WB>), dim3(grid1d(n, 256)), dim3(256), 0, st,
                         (const float*)W, ldw, M, K, (uint16_t*)values, (uint32_t*)meta, kept, tile_m, kmax,
                         WB ? (float*)W : nullptr);
    else
      hipLaunchKernelGGL((k_compress_canonical<uint16_t, GATHER, WB>), dim3(grid1d(n, 256)), dim3(256), 0, st,
                         (const uint16_t*)W, ldw, M, K, (uint16_t*)values, (uint32_t*)meta, kept, tile_m, kmax,
                         WB ? (uint16_t*)W : nullptr);
  } else {
    // A (row block, 256-column chunk) pair is one wave, or four of 8 rows
    // each when the pairs would give fewer than 16 waves per CU (the gathered
    // compression of 4096 x 4096, keep 2048: 1024 pairs).
    const int64_t pairs = device_row_blocks(M) * ((K + 255) / 256);
    const int rq = pairs < 4096 ? 4 : 1;
    const dim3 grid(grid1d(pairs * rq, CMP_WAVES)), block(64 * CMP_WAVES);
    if (w_dtype == P24_F32)
      hipLaunchKernelGGL((k_compress_device<float, GM, WB>), grid, block, 0, st, (const float*)W, ldw, M, K,
                         (uint16_t*)values, (uint32_t*)meta, kept, offsets, tile_m, kmax, WB ? (float*)W : nullptr,
                         rq);
    else
      hipLaunchKernelGGL((k_compress_device<uint16_t, GM, WB>), grid, block, 0, st, (const uint16_t*)W, ldw, M, K,
                         (uint16_t*)values, (uint32_t*)meta, kept, offsets, tile_m, kmax,
                         WB ? (uint16_t*)W : nullptr, rq);
  }
  return launch_status();
}

extern "C" P24_API p24_status prune24_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K,
                                               int64_t ldw, void* values, void* meta, int32_t layout,
                                               void* stream) {
  const p24_status s = check_compress_args(W, w_dtype, M, K, ldw, values, meta, layout);
  if (s != P24_OK) return s;
  return launch_compress<G_NONE>(W, w_dtype, M, K, ldw, values, meta, layout, nullptr, 1, K,
                                (hipStream_t)stream);
}

extern "C" P24_API p24_status prune24_refresh(void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                              void* values, void* meta, int32_t layout, void* stream) {
  const p24_status s = check_compress_args(W, w_dtype, M, K, ldw, values, meta, layout);
  if (s != P24_OK) return s;
  return launch_compress<G_NONE, true>(W, w_dtype, M, K, ldw, values, meta, layout, nullptr, 1, K,
                                       (hipStream_t)stream);
}

extern "C" P24_API p24_status prune24_mask_apply(void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                                 const void* meta, int32_t layout, void* stream) {
  if (w_dtype != P24_F32 && w_dtype != P24_BF16) return P24_ERR_DTYPE;
  if (layout != P24_LAYOUT_CANONICAL && layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (M < 0 || K < 0 || K % 4 || ldw < K || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (layout == P24_LAYOUT_DEVICE && K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return P24_OK;
  if (!W || !meta) return P24_ERR_NULL;
  const size_t wal = w_dtype == P24_F32 ? 16 : 8;
  if (!aligned(W, wal) || ldw % 4 || !aligned(meta, 4)) return P24_ERR_ALIGN;
  const int64_t n = M * (K / 4);
  if (w_dtype == P24_F32)
    hipLaunchKernelGGL(k_mask_apply<float>, dim3(grid1d(n, 256)), dim3(256), 0, (hipStream_t)stream, (float*)W,
                       ldw, M, K, (const uint32_t*)meta, (int)layout);
  else
    hipLaunchKernelGGL(k_mask_apply<uint16_t>, dim3(grid1d(n, 256)), dim3(256), 0, (hipStream_t)stream,
                       (uint16_t*)W, ldw, M, K, (const uint32_t*)meta, (int)layout);
  return launch_status();
}

extern "C" P24_API p24_status prune24_decompress(const void* values, const void* meta, int32_t layout,
                                                 int64_t M, int64_t K, void* W_out, int64_t ldo,
                                                 void* stream) {
  if (layout != P24_LAYOUT_CANONICAL && layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (M < 0 || K < 0 || K % 4 || ldo < K || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (layout == P24_LAYOUT_DEVICE && K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return P24_OK;
  if (!values || !meta || !W_out) return P24_ERR_NULL;
  if (!aligned(values, 4) || !aligned(meta, 4) || !aligned(W_out, 2)) return P24_ERR_ALIGN;
  const int64_t n = M * (K / 4);
  hipLaunchKernelGGL(k_decompress, dim3(grid1d(n, 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)values, (const uint32_t*)meta, (int)layout, M, K, (uint16_t*)W_out, ldo);
  return launch_status();
}

extern "C" P24_API size_t gemm_bf16_packed_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || K % 64) return 0;
  return (size_t)((M + 31) / 32) * 32 * (size_t)K * 2;
}

extern "C" P24_API p24_status gemm_bf16_pack(const void* W, int64_t M, int64_t K, int64_t ldw, void* Wp,
                                             void* stream) {
  if (M < 0 || K < 0 || ldw < K || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return P24_OK;
  if (!W || !Wp) return P24_ERR_NULL;
  if (!aligned(W, 16) || ldw % 8 || !aligned(Wp, 16)) return P24_ERR_ALIGN;
  const int64_t n = ((M + 31) / 32) * (K / 16) * 64;
  hipLaunchKernelGGL(k_pack_dense, dim3(grid1d(n, 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)W, ldw, M, K, (uint16_t*)Wp);
  return launch_status();
}

extern "C" P24_API size_t tvw_workspace_bytes(int64_t M, int64_t K, int64_t tile_m, int64_t keep_k) {
  (void)keep_k;
  if (M < 0 || K <= 0 || tile_m <= 0) return 0;
  return (size_t)((M + tile_m - 1) / tile_m) * (size_t)K * sizeof(double);
}

// Argument checks of tvw_compress and its no-allocation variant (everything but
// the workspace), in the order the header gives the errors.
static p24_status tvw_check(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw, int64_t tile_m,
                            int64_t keep_k, const int32_t* kept, const void* values, const void* meta,
                            int32_t layout) {
  if (w_dtype != P24_F32) return P24_ERR_DTYPE;
  if (layout != P24_LAYOUT_CANONICAL && layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (M < 0 || K <= 0 || ldw < K || tile_m <= 0 || tile_m % 32 || keep_k <= 0 || keep_k > K || keep_k % 4)
    return P24_ERR_SHAPE;
  if (M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;    // kept lists are int32
  if (layout == P24_LAYOUT_DEVICE && keep_k % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0) return P24_OK;
  if (!W || !kept || !values || !meta) return P24_ERR_NULL;
  if (!aligned(W, 16) || ldw % 4 || !aligned(values, 16) || !aligned(meta, 16) || !aligned(kept, 4))
    return P24_ERR_ALIGN;
  return P24_OK;
}

// Scores into `workspace` (T x K doubles, every entry written before it is read),
// per-tile selection, then 2:4 compression of the kept columns.
static p24_status tvw_launch(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw, int64_t tile_m,
                             int64_t keep_k, int32_t* kept, void* values, void* meta, int32_t layout,
                             void* workspace, hipStream_t st) {
  const int64_t T_ = (M + tile_m - 1) / tile_m;
  double* scores = (double*)workspace;
  launch_tvw_scores((const float*)W, ldw, M, K, tile_m, scores, st);
  p24_status s = launch_status();
  if (s != P24_OK) return s;
  hipLaunchKernelGGL(k_tvw_select, dim3((unsigned)T_), dim3(SEL_THREADS), 0, st, (const double*)scores, K,
                     keep_k, (const int64_t*)nullptr, kept);
  s = launch_status();
  if (s != P24_OK) return s;
  // 2:4 along the compacted axis, reading W through the kept column lists
  return launch_compress<G_FIXED>(W, w_dtype, M, keep_k, ldw, values, meta, layout, kept, tile_m, K, st);
}

extern "C" P24_API p24_status tvw_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                           int64_t tile_m, int64_t keep_k, int32_t* kept, void* values,
                                           void* meta, int32_t layout, void* workspace, size_t ws_bytes,
                                           void* stream) {
  p24_status s = tvw_check(W, w_dtype, M, K, ldw, tile_m, keep_k, kept, values, meta, layout);
  if (s != P24_OK || M == 0) return s;
  if (!workspace || ws_bytes < tvw_workspace_bytes(M, K, tile_m, keep_k)) return P24_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return P24_ERR_ALIGN;
  return tvw_launch(W, w_dtype, M, K, ldw, tile_m, keep_k, kept, values, meta, layout, workspace,
                    (hipStream_t)stream);
}

// --------------------------------------------------------------------------
// tvw_compress without an allocation or a workspace argument: the column
// scores go to `scratch`, a fixed array in device memory (each GPU holds its
// own copy for the life of the process).  Host code reaches it only through
// the address hipGetSymbolAddress returns for the current device, looked up
// once per device and kept; the array's name itself is not a device address
// on the host.  Nothing in it has to start at zero: the score kernel writes
// every entry the selection reads.  Calls that overlap on one GPU share it and
// race.
// --------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MAX_DEVICES];

// The scratch address on the current device, looked up on the first call there.
static p24_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return P24_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return P24_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return P24_OK;
}

extern "C" P24_API size_t tvw_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" P24_API p24_status tvw_compress_noalloc(const void* W, int32_t w_dtype, int64_t M, int64_t K,
                                                   int64_t ldw, int64_t tile_m, int64_t keep_k, int32_t* kept,
                                                   void* values, void* meta, int32_t layout, void* stream) {
  p24_status s = tvw_check(W, w_dtype, M, K, ldw, tile_m, keep_k, kept, values, meta, layout);
  if (s != P24_OK || M == 0) return s;
  if (tvw_workspace_bytes(M, K, tile_m, keep_k) > NOALLOC_SCRATCH_BYTES) return P24_ERR_SCRATCH;
  // the stream must belong to the current device, whose copy of the scratch is used
  if (stream) {
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess || hipGetDevice(&cur) != hipSuccess)
      return P24_ERR_HIP;
    if (sdev != cur) return P24_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != P24_OK) return s;
  return tvw_launch(W, w_dtype, M, K, ldw, tile_m, keep_k, kept, values, meta, layout, ws, (hipStream_t)stream);
}

static int64_t var_tiles(int64_t M) { return (M + 127) / 128; }

extern "C" P24_API size_t tvw_var_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K <= 0) return 0;
  const int64_t T_ = var_tiles(M);
  const size_t scores = ((size_t)T_ * (size_t)K * sizeof(double) + 255) & ~(size_t)255;
  const size_t sel = (sizeof(VarSelectW) + 255) & ~(size_t)255;
  return scores + sel + 2 * (size_t)T_ * sizeof(int32_t);
}

// Scores, the global cut, keep counts, offsets, order and the kept lists of
// per-tile-keep TVW / TW (arguments already validated).
static p24_status launch_var_plan(const void* W, int64_t M, int64_t K, int64_t ldw, int64_t total_keep,
                                  int64_t* offsets, int32_t* order, int32_t* kept, void* workspace,
                                  hipStream_t st) {
  const int64_t T_ = var_tiles(M);
  uint8_t* ws = (uint8_t*)workspace;
  double* scores = (double*)ws;
  ws += ((size_t)T_ * (size_t)K * sizeof(double) + 255) & ~(size_t)255;
  VarSelectW* vs = (VarSelectW*)ws;
  ws += (sizeof(VarSelectW) + 255) & ~(size_t)255;
  int32_t* gt = (int32_t*)ws;
  int32_t* eq = gt + T_;
  const int64_t n = T_ * K;
  launch_tvw_scores((const float*)W, ldw, M, K, 128, scores, st, vs, total_keep);   // also initialises vs
  const int64_t per_block = (int64_t)VAR_THREADS * 8;
  const unsigned radix_blocks = (unsigned)std::min<int64_t>((n + per_block - 1) / per_block, 1024);
  // digits of 11 bits from the top (bits 53..63, 42..52, ...), the last one
  // the 9 bits left
  for (int top = 64; top > 0; top -= VAR_DIGIT) {
    const int width = top < VAR_DIGIT ? top : VAR_DIGIT;
    hipLaunchKernelGGL(k_var_radix, dim3(radix_blocks), dim3(VAR_THREADS), 0, st, (const uint64_t*)scores, n,
                       top - width, width, vs);
  }
  hipLaunchKernelGGL(k_var_tile_counts, dim3((unsigned)T_), dim3(VAR_THREADS), 0, st, (const uint64_t*)scores, K,
                     (const VarSelectW*)vs, gt, eq);
  // up to SEL_THREADS tiles the plan kernel also orders them (one launch less)
  const bool plan_orders = T_ <= SEL_THREADS;
  hipLaunchKernelGGL(k_var_plan, dim3(1), dim3(SEL_THREADS), 0, st, T_, K, (const VarSelectW*)vs,
                     (const int32_t*)gt, (const int32_t*)eq, offsets, plan_orders ? order : nullptr);
  if (!plan_orders)
    hipLaunchKernelGGL(k_var_order, dim3(grid1d(T_, VAR_THREADS)), dim3(VAR_THREADS), 0, st,
                       (const int64_t*)offsets, T_, order);
  hipLaunchKernelGGL(k_tvw_select, dim3((unsigned)T_), dim3(SEL_THREADS), 0, st, (const double*)scores, K,
                     (int64_t)0, (const int64_t*)offsets, kept);
  return launch_status();
}

static p24_status check_var_args(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                 int64_t total_keep, const void* offsets, const void* order, const void* kept,
                                 const void* values, const void* meta, const void* workspace, size_t ws_bytes) {
  if (w_dtype != P24_F32) return P24_ERR_DTYPE;
  if (M < 0 || K <= 0 || ldw < K || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0) return P24_OK;
  const int64_t T_ = var_tiles(M);
  if (T_ * K > INT32_MAX || total_keep <= 0 || total_keep > T_ * K) return P24_ERR_SHAPE;
  if (!W || !offsets || !order || !kept || !values || !meta) return P24_ERR_NULL;
  if (!workspace || ws_bytes < tvw_var_workspace_bytes(M, K)) return P24_ERR_WORKSPACE;
  if (!aligned(W, 16) || ldw % 4 || !aligned(values, 16) || !aligned(meta, 16) || !aligned(kept, 4) ||
      !aligned(offsets, 8) || !aligned(order, 4) || !aligned(workspace, 256))
    return P24_ERR_ALIGN;
  return P24_OK;
}

extern "C" P24_API p24_status tvw_var_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                               int64_t total_keep, int64_t* offsets, int32_t* order,
                                               int32_t* kept, void* values, void* meta, void* workspace,
                                               size_t ws_bytes, void* stream) {
  p24_status s = check_var_args(W, w_dtype, M, K, ldw, total_keep, offsets, order, kept, values, meta, workspace,
                                ws_bytes);
  if (s != P24_OK || M == 0) return s;
  hipStream_t st = (hipStream_t)stream;
  s = launch_var_plan(W, M, K, ldw, total_keep, offsets, order, kept, workspace, st);
  if (s != P24_OK) return s;
  // 2:4 along each tile's compacted axis; K bounds the widest tile
  return launch_compress<G_VAR>(W, w_dtype, M, K, ldw, values, meta, P24_LAYOUT_DEVICE, kept, 128, K, st, offsets);
}

extern "C" P24_API p24_status tw_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                          int64_t tile_m, int64_t keep_k, int32_t* kept, void* Wp,
                                          void* workspace, size_t ws_bytes, void* stream) {
  if (w_dtype != P24_F32) return P24_ERR_DTYPE;
  if (M < 0 || K <= 0 || ldw < K || tile_m <= 0 || tile_m % 32 || keep_k <= 0 || keep_k > K)
    return P24_ERR_SHAPE;
  if (M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (keep_k % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0) return P24_OK;
  if (!W || !kept || !Wp) return P24_ERR_NULL;
  if (!workspace || ws_bytes < tvw_workspace_bytes(M, K, tile_m, keep_k)) return P24_ERR_WORKSPACE;
  if (!aligned(W, 16) || ldw % 4 || !aligned(Wp, 16) || !aligned(kept, 4) || !aligned(workspace, 8))
    return P24_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const int64_t T_ = (M + tile_m - 1) / tile_m;
  double* scores = (double*)workspace;
  launch_tvw_scores((const float*)W, ldw, M, K, tile_m, scores, st);
  hipLaunchKernelGGL(k_tvw_select, dim3((unsigned)T_), dim3(SEL_THREADS), 0, st, (const double*)scores, K,
                     keep_k, (const int64_t*)nullptr, kept);
  const int64_t rows = (M + 31) / 32 * 32;
  hipLaunchKernelGGL(k_pack_tw<false>, dim3(grid1d(rows * (keep_k / 8), 256)), dim3(256), 0, st, (const float*)W,
                     ldw, M, K, keep_k, (const int32_t*)kept, (const int64_t*)nullptr, tile_m, rows,
                     (uint16_t*)Wp);
  return launch_status();
}

extern "C" P24_API p24_status tw_var_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                              int64_t total_keep, int64_t* offsets, int32_t* order,
                                              int32_t* kept, void* Wp, void* workspace, size_t ws_bytes,
                                              void* stream) {
  p24_status s = check_var_args(W, w_dtype, M, K, ldw, total_keep, offsets, order, kept, Wp, Wp, workspace,
                                ws_bytes);
  if (s != P24_OK || M == 0) return s;
  hipStream_t st = (hipStream_t)stream;
  s = launch_var_plan(W, M, K, ldw, total_keep, offsets, order, kept, workspace, st);
  if (s != P24_OK) return s;
  const int64_t rows = var_tiles(M) * 128;
  hipLaunchKernelGGL(k_pack_tw<true>, dim3(grid1d(rows * (K / 8), 256)), dim3(256), 0, st, (const float*)W, ldw,
                     M, K, K, (const int32_t*)kept, (const int64_t*)offsets, (int64_t)128, rows, (uint16_t*)Wp);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Comparison patterns (block-wise, unstructured)
// ---------------------------------------------------------------------------
extern "C" P24_API size_t bw_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K <= 0) return 0;
  const int64_t T_ = var_tiles(M);
  return (size_t)T_ * (size_t)K * sizeof(double) + (size_t)T_ * (size_t)(K / 64) * (sizeof(double) + 4);
}

extern "C" P24_API p24_status bw_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                          int64_t keep_blocks, int32_t* kept, void* Wp, void* workspace,
                                          size_t ws_bytes, void* stream) {
  if (w_dtype != P24_F32) return P24_ERR_DTYPE;
  if (M < 0 || K <= 0 || ldw < K || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (keep_blocks <= 0 || keep_blocks > K / 64) return P24_ERR_SHAPE;
  if (M == 0) return P24_OK;
  if (!W || !kept || !Wp) return P24_ERR_NULL;
  if (!workspace || ws_bytes < bw_workspace_bytes(M, K)) return P24_ERR_WORKSPACE;
  if (!aligned(W, 16) || ldw % 4 || !aligned(Wp, 16) || !aligned(kept, 4) || !aligned(workspace, 8))
    return P24_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const int64_t T_ = var_tiles(M), nb = K / 64, keep = keep_blocks * 64;
  double* scores = (double*)workspace;
  double* bscores = scores + T_ * K;
  int32_t* kept_blocks = (int32_t*)(bscores + T_ * nb);
  launch_tvw_scores((const float*)W, ldw, M, K, 128, scores, st);
  hipLaunchKernelGGL(k_bw_block_scores, dim3(grid1d(T_ * nb, 256)), dim3(256), 0, st, (const double*)scores, T_, K,
                     bscores);
  hipLaunchKernelGGL(k_tvw_select, dim3((unsigned)T_), dim3(SEL_THREADS), 0, st, (const double*)bscores, nb,
                     keep_blocks, (const int64_t*)nullptr, kept_blocks);
  hipLaunchKernelGGL(k_bw_expand, dim3(grid1d(T_ * keep, 256)), dim3(256), 0, st, (const int32_t*)kept_blocks, T_,
                     keep_blocks, kept);
  const int64_t rows = (M + 31) / 32 * 32;
  hipLaunchKernelGGL(k_pack_tw<false>, dim3(grid1d(rows * (keep / 8), 256)), dim3(256), 0, st, (const float*)W, ldw,
                     M, K, keep, (const int32_t*)kept, (const int64_t*)nullptr, (int64_t)128, rows, (uint16_t*)Wp);
  return launch_status();
}

extern "C" P24_API size_t ew_workspace_bytes(int64_t M, int64_t K) {
  (void)K;
  if (M < 0) return 0;
  return ((sizeof(VarSelect) + 255) & ~(size_t)255) + 2 * (size_t)M * sizeof(int32_t);
}

extern "C" P24_API p24_status ew_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                          int64_t keep_total, int64_t* row_ptr, int32_t* cols, void* vals,
                                          void* workspace, size_t ws_bytes, void* stream) {
  if (w_dtype != P24_F32) return P24_ERR_DTYPE;
  if (M < 0 || K <= 0 || ldw < K || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (M * K > UINT32_MAX || keep_total <= 0 || keep_total > M * K) return P24_ERR_SHAPE;
  if (M == 0) return P24_OK;
  if (!W || !row_ptr || !cols || !vals) return P24_ERR_NULL;
  if (!workspace || ws_bytes < ew_workspace_bytes(M, K)) return P24_ERR_WORKSPACE;
  if (!aligned(W, 4) || !aligned(row_ptr, 8) || !aligned(cols, 4) || !aligned(vals, 2) || !aligned(workspace, 256))
    return P24_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  VarSelect* vs = (VarSelect*)ws;
  ws += (sizeof(VarSelect) + 255) & ~(size_t)255;
  int32_t* gt = (int32_t*)ws;
  int32_t* eq = gt + M;
  hipLaunchKernelGGL(k_var_init<256>, dim3(1), dim3(VAR_THREADS), 0, st, vs, keep_total);
  const int64_t n = M * K, per_block = (int64_t)VAR_THREADS * 16;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + per_block - 1) / per_block, 2048);
  for (int shift = 24; shift >= 0; shift -= 8)
    hipLaunchKernelGGL(k_ew_radix, dim3(blocks), dim3(VAR_THREADS), 0, st, (const float*)W, ldw, M, K, shift, vs);
  hipLaunchKernelGGL(k_ew_row_counts, dim3((unsigned)M), dim3(VAR_THREADS), 0, st, (const float*)W, ldw, K,
                     (const VarSelect*)vs, gt, eq);
  hipLaunchKernelGGL(k_ew_plan, dim3(1), dim3(SEL_THREADS), 0, st, M, (const VarSelect*)vs, (const int32_t*)gt, eq,
                     row_ptr);
  hipLaunchKernelGGL(k_ew_compact, dim3((unsigned)M), dim3(SEL_THREADS), 0, st, (const float*)W, ldw, K,
                     (const VarSelect*)vs, (const int32_t*)eq, (const int64_t*)row_ptr, cols, (uint16_t*)vals);
  return launch_status();
}
