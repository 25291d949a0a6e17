// Tile loop for Y = W X on gfx950: 2:4-sparse W on the sparse MFMA
// (v_smfmac_f32_32x32x32_bf16), optionally with a TVW row gather of X, and the
// dense bf16 baseline on v_mfma_f32_32x32x16_bf16.
//
// Data flow per block (BM x BN outputs, K consumed 64 logical columns at a time):
//   * W operand: the compressed values / metadata (or the packed dense W) are
//     stored in MFMA operand order, so each wave loads its A fragments straight
//     from global memory into registers: every load is one contiguous 1 KiB
//     (values) or 256 B (metadata) block per wave.  No LDS is spent on W.
//   * X operand: the 64 x BN tile (row-major, N contiguous) is staged in LDS
//     with double buffering; rows are whole contiguous N-slices, so the TVW
//     gather only changes which global row each slice comes from.  B fragments
//     come out of LDS with ds_read_b64_tr_b16, which transposes 4 x 16 bf16
//     sub-tiles so each lane receives 4 consecutive k of one column.
//   * Accumulators stay in registers for the whole K loop; the epilogue rounds
//     (fp32 -> bf16 RNE) or stores fp32 with row-contiguous lane groups.
#include <cstdlib>
#include <string>

#include "p24_api_internal.hpp"
#include "p24_device.hpp"

namespace p24 {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;       // logical K per main-loop iteration
constexpr int XPAD = 32;     // bf16 elements of padding per LDS row of the X tile

template <int BM, int BN, int WGM, int WGN>
struct TileCfg {
  static constexpr int NT = WGM * WGN * 64;        // threads per block
  static constexpr int WTM = BM / WGM;             // wave tile rows
  static constexpr int WTN = BN / WGN;             // wave tile cols
  static constexpr int TM = WTM / 32;              // 32x32 MFMA tiles per wave (rows)
  static constexpr int TN = WTN / 32;              // ... (cols)
  static constexpr int LDX = BN + XPAD;            // LDS row pitch of the X tile (elements)
  static constexpr int XCH = BK * BN / 8;          // 16 B chunks per X tile
  static constexpr int XCH_PER_T = XCH / NT;
  static_assert(BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "wave tiles must be multiples of 32");
  static_assert(XCH % NT == 0, "X tile chunks must divide evenly among threads");
};

// 4 consecutive k (rows kb..kb+3 of the LDS tile) for column (c0 + lane%16)
// of a 16-lane group; see the ds_read_b64_tr_b16 lane map above.
__device__ __forceinline__ i16x4 tr_read(const uint16_t* xs, int ldx, int kb, int c0, int lane) {
  const int li = lane & 15;
  const uint16_t* p = xs + (kb + (li >> 2)) * ldx + c0 + 4 * (li & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <typename OutT> __device__ __forceinline__ void store_out(OutT* p, float v);
template <> __device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = f32_to_bf16_rne(__float_as_uint(v));
}

struct GemmArgs {
  const uint16_t* A;       // sparse: device-layout values; dense: packed W
  const uint32_t* Ameta;   // sparse: device-layout metadata
  const int32_t* kept;     // TVW: [T][Kc] gathered X rows (nullptr otherwise)
  const uint16_t* X;
  void* Y;
  int64_t ldx, ldy;
  int M, N, Kc, Kx;        // Kc: K of the W operand (compacted for TVW); Kx: rows of X
  int tile_m;              // TVW tile rows
  int nbm, nbn;            // block grid
};

template <int BM, int BN, int WGM, int WGN, bool SPARSE, bool GATHER, typename OutT>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm(const GemmArgs args) {
  using C = TileCfg<BM, BN, WGM, WGN>;
  constexpr int TM = C::TM, TN = C::TN, LDX = C::LDX;
  constexpr int ASTEPS = SPARSE ? 2 : 4;           // A fragments per K64 per row block
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BK * LDX];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- block -> output tile (XCD-aware, grouped raster) ----
  const uint32_t nblocks = (uint32_t)args.nbm * args.nbn;
  const uint32_t b = xcd_remap(blockIdx.x, nblocks);
  constexpr uint32_t GROUP = 8;
  const uint32_t group_size = GROUP * args.nbn;
  const uint32_t first_m = (b / group_size) * GROUP;
  const uint32_t gsz = min((uint32_t)args.nbm - first_m, GROUP);
  const int bm = first_m + (b % group_size) % gsz;
  const int bn = (b % group_size) / gsz;
  const int m0 = bm * BM, n0 = bn * BN;

  const int M = args.M, N = args.N, Kc = args.Kc;
  const int nk = Kc / BK;
  const int rb0 = (m0 + wm * C::WTM) / 32;
  const int nrb = (M + 31) / 32;
  const int64_t S = SPARSE ? Kc / 32 : Kc / 16;    // A blocks per row block
  const int64_t T_ = Kc / 64;

  const int32_t* kept_tile = nullptr;
  if constexpr (GATHER) kept_tile = args.kept + (int64_t)(m0 / args.tile_m) * Kc;

  // ---- register state ----
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  bf16x8 a_cur[TM][ASTEPS], a_nxt[TM][ASTEPS];
  uint32_t m_cur[TM], m_nxt[TM];
  u32x4 xr[C::XCH_PER_T];

  auto load_a = [&](int it, bf16x8 (&a)[TM][ASTEPS], uint32_t (&mt)[TM]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rb = rb0 + i;
      if (rb < nrb) {
#pragma unroll
        for (int s = 0; s < ASTEPS; ++s)
          a[i][s] = *reinterpret_cast<const bf16x8*>(args.A + (((int64_t)rb * S + (int64_t)it * ASTEPS + s) * 64 + lane) * 8);
        if constexpr (SPARSE) mt[i] = args.Ameta[((int64_t)rb * T_ + it) * 64 + lane];
      } else {
#pragma unroll
        for (int s = 0; s < ASTEPS; ++s) a[i][s] = (bf16x8){};
        mt[i] = 0x44444444u;
      }
    }
  };

  auto load_x = [&](int it) {
#pragma unroll
    for (int j = 0; j < C::XCH_PER_T; ++j) {
      const int c = tid + j * C::NT;
      const int r = c / (BN / 8), c8 = c % (BN / 8);
      int64_t gk = (int64_t)it * BK + r;
      if constexpr (GATHER) {
        int kk = kept_tile[gk];
        kk = kk < 0 ? 0 : (kk >= args.Kx ? args.Kx - 1 : kk);
        gk = kk;
      }
      const int col = n0 + c8 * 8;
      const uint16_t* src = args.X + gk * args.ldx + col;
      if (col + 8 <= N) {
        xr[j] = *reinterpret_cast<const u32x4*>(src);
      } else {
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = (col + q < N) ? (uint32_t)src[q] : 0u;
        xr[j] = (u32x4){e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
      }
    }
  };

  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::XCH_PER_T; ++j) {
      const int c = tid + j * C::NT;
      const int r = c / (BN / 8), c8 = c % (BN / 8);
      *reinterpret_cast<u32x4*>(&xs[buf][r * LDX + c8 * 8]) = xr[j];
    }
  };

  const int h = lane >> 5;                       // lane half
  const int cgrp = 16 * ((lane >> 4) & 1);       // column offset of this lane's 16-lane group
  const int wcol = wn * C::WTN;

  auto compute = [&](int buf) {
    const uint16_t* xb = xs[buf];
    if constexpr (SPARSE) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        bf16x16 bfr[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c0 = wcol + 32 * j + cgrp;
          const int kb = 32 * ss + 8 * h;
          const i16x4 q0 = tr_read(xb, LDX, kb, c0, lane);
          const i16x4 q1 = tr_read(xb, LDX, kb + 4, c0, lane);
          const i16x4 q2 = tr_read(xb, LDX, kb + 16, c0, lane);
          const i16x4 q3 = tr_read(xb, LDX, kb + 20, c0, lane);
          const i16x8 lo = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
          const i16x8 hi = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
          const i16x16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
          bfr[j] = __builtin_bit_cast(bf16x16, v);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if (ss == 0)
              acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a_cur[i][0], bfr[j], acc[i][j], (int)m_cur[i], 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a_cur[i][1], bfr[j], acc[i][j], (int)m_cur[i], 0, 1);
          }
      }
    } else {
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        bf16x8 bfr[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c0 = wcol + 32 * j + cgrp;
          const int kb = 16 * ss + 8 * h;
          const i16x4 q0 = tr_read(xb, LDX, kb, c0, lane);
          const i16x4 q1 = tr_read(xb, LDX, kb + 4, c0, lane);
          bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_cur[i][ss], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // ---- main loop: one barrier per iteration, X double-buffered in LDS ----
  load_x(0);
  load_a(0, a_cur, m_cur);
  store_x(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      load_x(it + 1);
      load_a(it + 1, a_nxt, m_nxt);
    }
    compute(cur);
    if (more) store_x(cur ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        m_cur[i] = m_nxt[i];
#pragma unroll
        for (int s = 0; s < ASTEPS; ++s) a_cur[i][s] = a_nxt[i][s];
      }
    }
  }

  // ---- epilogue ----
  OutT* Y = reinterpret_cast<OutT*>(args.Y);
  const int row_w = m0 + wm * C::WTM;
  const int col_l = n0 + wcol + (lane & 31);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = col_l + 32 * j;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row_w + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (row < M && col < N) store_out<OutT>(Y + (int64_t)row * args.ldy + col, acc[i][j][e]);
      }
    }
}

// ---------------------------------------------------------------------------
// Host-side tile configuration and dispatch
// ---------------------------------------------------------------------------
enum class Tile { T256x256, T128x256, T128x128, T64x128 };

template <int BM, int BN, int WGM, int WGN, bool SPARSE, bool GATHER>
static p24_status launch_cfg(GemmArgs a, int32_t y_dtype, hipStream_t st) {
  a.nbm = (a.M + BM - 1) / BM;
  a.nbn = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(a.nbm * a.nbn)), block(WGM * WGN * 64);
  if (y_dtype == P24_F32)
    hipLaunchKernelGGL((k_gemm<BM, BN, WGM, WGN, SPARSE, GATHER, float>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, WGM, WGN, SPARSE, GATHER, uint16_t>), grid, block, 0, st, a);
  return launch_status();
}

static int64_t nblocks_for(Tile t, int64_t M, int64_t N) {
  int bm = 256, bn = 256;
  switch (t) {
    case Tile::T256x256: bm = 256; bn = 256; break;
    case Tile::T128x256: bm = 128; bn = 256; break;
    case Tile::T128x128: bm = 128; bn = 128; break;
    case Tile::T64x128: bm = 64; bn = 128; break;
  }
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// Largest tile that still gives at least one block per CU; otherwise the one
// with the most blocks.  P24_TILE=<256x256|128x256|128x128|64x128> overrides
// (measurement aid).
static Tile choose_tile(int64_t M, int64_t N) {
  if (const char* e = getenv("P24_TILE")) {
    const std::string s(e);
    if (s == "256x256") return Tile::T256x256;
    if (s == "128x256") return Tile::T128x256;
    if (s == "128x128") return Tile::T128x128;
    if (s == "64x128") return Tile::T64x128;
  }
  const Tile order[] = {Tile::T256x256, Tile::T128x256, Tile::T128x128, Tile::T64x128};
  for (Tile t : order)
    if (nblocks_for(t, M, N) >= 256) return t;
  return Tile::T64x128;
}

template <bool SPARSE>
static p24_status dispatch(const GemmArgs& a, int32_t y_dtype, hipStream_t st) {
  switch (choose_tile(a.M, a.N)) {
    case Tile::T256x256: return launch_cfg<256, 256, 2, 2, SPARSE, false>(a, y_dtype, st);
    case Tile::T128x256: return launch_cfg<128, 256, 2, 2, SPARSE, false>(a, y_dtype, st);
    case Tile::T128x128: return launch_cfg<128, 128, 2, 2, SPARSE, false>(a, y_dtype, st);
    case Tile::T64x128: return launch_cfg<64, 128, 1, 2, SPARSE, false>(a, y_dtype, st);
  }
  return P24_ERR_UNSUPPORTED;
}

static p24_status check_xy(const void* X, int64_t ldx, int64_t N, const void* Y, int32_t y_dtype,
                           int64_t ldy) {
  if (y_dtype != P24_F32 && y_dtype != P24_BF16) return P24_ERR_DTYPE;
  if (N < 0 || ldx < N || ldy < N || N > INT32_MAX) return P24_ERR_SHAPE;
  (void)X;
  (void)Y;
  return P24_OK;
}

static p24_status check_xy_ptrs(const void* X, int64_t ldx, const void* Y, int32_t y_dtype) {
  if (!X || !Y) return P24_ERR_NULL;
  if (!aligned(X, 16) || ldx % 8) return P24_ERR_ALIGN;
  if (!aligned(Y, y_dtype == P24_F32 ? 4 : 2)) return P24_ERR_ALIGN;
  return P24_OK;
}

}  // namespace p24

using namespace p24;

extern "C" P24_API p24_status spmm24(const void* values, const void* meta, int32_t layout, int64_t M, int64_t K,
                                     const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                                     int64_t ldy, int32_t algo, void* stream) {
  if (layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (algo != P24_ALGO_AUTO && algo != P24_ALGO_SMFMAC) return P24_ERR_UNSUPPORTED;
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K < 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return P24_OK;
  if (K == 0) return P24_ERR_UNSUPPORTED;
  if (!values || !meta) return P24_ERR_NULL;
  if (!aligned(values, 16) || !aligned(meta, 16)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(X, ldx, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)values;
  a.Ameta = (const uint32_t*)meta;
  a.X = (const uint16_t*)X;
  a.Y = Y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = (int)K;
  a.Kx = (int)K;
  a.tile_m = 1;
  return dispatch<true>(a, y_dtype, (hipStream_t)stream);
}

extern "C" P24_API p24_status spmm_tvw(const int32_t* kept, const void* values, const void* meta, int32_t layout,
                                       int64_t M, int64_t K, int64_t tile_m, int64_t keep_k, const void* X,
                                       int64_t ldx, int64_t N, void* Y, int32_t y_dtype, int64_t ldy,
                                       void* stream) {
  if (layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K <= 0 || tile_m <= 0 || keep_k <= 0 || keep_k > K || M > INT32_MAX || K > INT32_MAX)
    return P24_ERR_SHAPE;
  if (tile_m % 128 || keep_k % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return P24_OK;
  if (!kept || !values || !meta) return P24_ERR_NULL;
  if (!aligned(values, 16) || !aligned(meta, 16) || !aligned(kept, 4)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(X, ldx, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)values;
  a.Ameta = (const uint32_t*)meta;
  a.kept = kept;
  a.X = (const uint16_t*)X;
  a.Y = Y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = (int)keep_k;
  a.Kx = (int)K;
  a.tile_m = (int)tile_m;
  // one block row = one 128-row slice of a TVW tile
  return launch_cfg<128, 256, 2, 2, true, true>(a, y_dtype, (hipStream_t)stream);
}

extern "C" P24_API p24_status gemm_bf16(const void* Wp, int64_t M, int64_t K, const void* X, int64_t ldx,
                                        int64_t N, void* Y, int32_t y_dtype, int64_t ldy, void* stream) {
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K < 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return P24_OK;
  if (K == 0) return P24_ERR_UNSUPPORTED;
  if (!Wp) return P24_ERR_NULL;
  if (!aligned(Wp, 16)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(X, ldx, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)Wp;
  a.X = (const uint16_t*)X;
  a.Y = Y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = (int)K;
  a.Kx = (int)K;
  a.tile_m = 1;
  return dispatch<false>(a, y_dtype, (hipStream_t)stream);
}
