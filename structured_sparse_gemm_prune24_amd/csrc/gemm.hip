// Tile loop for Y = W X on gfx950: 2:4-sparse W on the sparse MFMA
// (v_smfmac_f32_32x32x32_bf16), optionally with a TVW row gather of X, and the
// dense bf16 baseline on v_mfma_f32_32x32x16_bf16.
//
// Data flow per block (BM x BN outputs, K consumed 64 logical columns at a time):
//   * W operand: the compressed values / metadata (or the packed dense W) are
//     stored in MFMA operand order, so each wave loads its A fragments straight
//     from global memory into registers, one contiguous 1 KiB (values) or
//     256 B (metadata) block per wave and load.  No LDS is spent on W.  The
//     fragments of iteration it+1 are in flight while iteration it computes.
//   * X operand: 64 x BN tiles (row-major, N contiguous) go global -> LDS with
//     direct-to-LDS loads (global_load_lds_dwordx4: lane l writes its 16 B at
//     the wave's LDS base + 16 l), into a ring of three LDS stages, two tiles
//     ahead of the compute.  Rows are whole N-slices, so the TVW gather only
//     changes the global row a slice comes from.  Inside a row the 16 B chunks
//     are XOR-swizzled by the row's low bits so that the transposed reads below
//     spread over all LDS banks.
//   * B fragments come out of LDS with ds_read_b64_tr_b16: within a group of
//     16 lanes, lane i receives element i%4 of the 8-byte pieces addressed by
//     lanes 4e + i/4 (e = 0..3), i.e. 4 consecutive k of one column when the
//     16 lanes address a 4-row x 16-column sub-tile.  These reads are issued as
//     inline asm with explicit lgkmcnt waits tied to the fragments: the
//     compiler would otherwise stall every LDS read on all outstanding
//     direct-to-LDS loads.
//   * Tails: addresses are clamped instead of branched on.  Columns of X at or
//     beyond N only feed output columns that are never stored, and rows past M
//     only feed rows that are never stored, so the clamped (valid) data there
//     is harmless.
//   * Accumulators stay in registers for the whole K loop; the epilogue rounds
//     (fp32 -> bf16 RNE) or stores fp32 with row-contiguous lane groups.
#include <cstdlib>
#include <string>
#include <type_traits>

#include "p24_api_internal.hpp"
#include "p24_device.hpp"

namespace p24 {

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 64;       // logical K per main-loop iteration
constexpr int NSTAGE = 3;    // LDS ring depth for the X tiles

template <int BM, int BN, int WGM, int WGN>
struct TileCfg {
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int NT = NWAVES * 64;           // threads per block
  static constexpr int WTM = BM / WGM;             // wave tile rows
  static constexpr int WTN = BN / WGN;             // wave tile cols
  static constexpr int TM = WTM / 32;              // 32x32 MFMA tiles per wave (rows)
  static constexpr int TN = WTN / 32;              // ... (cols)
  static constexpr int ROWB = BN * 2;              // bytes per LDS row of an X tile
  static constexpr int CPR = BN / 8;               // 16 B chunks per row
  static constexpr int STAGE_BYTES = BK * ROWB;
  static constexpr int XCH = BK * CPR;             // 16 B chunks per X tile
  static constexpr int XCH_PER_T = XCH / NT;       // direct-to-LDS loads per thread per tile
  static_assert(BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "wave tiles must be multiples of 32");
  static_assert(XCH % NT == 0, "X tile chunks must divide evenly among threads");
  static_assert(CPR >= 16, "the chunk swizzle needs at least 16 chunks per row");
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// XOR applied to the 16 B chunk index of row r.  Rows r..r+3 of one transposed
// read land on 32 B bank groups {0,3,5,6} (x2 chunks): distinct both modulo 4
// and (pairs) modulo 8 groups.
__device__ __forceinline__ int chunk_swizzle(int r) {
  const int q = r & 3;
  return ((q << 1) | (__builtin_popcount(q) & 1)) << 1;
}

template <int OFF>
__device__ __forceinline__ i16x4 ds_read_tr(uint32_t addr) {
  i16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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
  constexpr int TM = C::TM, TN = C::TN;
  constexpr int ASTEPS = SPARSE ? 2 : 4;           // A fragments per K64 per row block
  constexpr int A_LOADS = SPARSE ? TM * (ASTEPS + 1) : TM * ASTEPS;   // vector loads per A prefetch
  __shared__ __attribute__((aligned(1024))) uint8_t xs[NSTAGE * C::STAGE_BYTES];

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
  const int nrb = (M + 31) / 32;
  const int64_t S = SPARSE ? Kc / 32 : Kc / 16;    // A blocks per row block
  const int64_t T_ = Kc / 64;
  const int n_hi = ((N + 7) & ~7) - 8;             // last 8-aligned column start inside the readable row

  const int32_t* kept_tile = nullptr;
  if constexpr (GATHER) kept_tile = args.kept + (int64_t)(m0 / args.tile_m) * Kc;

  // ---- A operand pointers (row blocks past the matrix are clamped) ----
  const uint16_t* a_ptr[TM];
  const uint32_t* m_ptr[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int rb = (m0 + wm * C::WTM) / 32 + i;
    rb = rb < nrb ? rb : nrb - 1;
    a_ptr[i] = args.A + ((int64_t)rb * S * 64 + lane) * 8;
    m_ptr[i] = SPARSE ? args.Ameta + (int64_t)rb * T_ * 64 + lane : nullptr;
  }

  // ---- X direct-to-LDS loads: this lane's chunk of each load instruction ----
  // load j of this wave covers tile chunks [(j*NWAVES + wave)*64, +64); lane -> one chunk.
  int x_row[C::XCH_PER_T], x_col[C::XCH_PER_T];
#pragma unroll
  for (int j = 0; j < C::XCH_PER_T; ++j) {
    const int p = (j * C::NWAVES + wave) * 64 + lane;
    const int r = p / C::CPR, cs = p % C::CPR;
    const int c = cs ^ chunk_swizzle(r);
    int col = n0 + 8 * c;
    col = col <= n_hi ? col : n_hi;
    x_row[j] = r;
    x_col[j] = col;
  }
  const uint32_t xs_base = (uint32_t)(uintptr_t)(lds_void*)xs;

  // TVW: the gathered X rows of tile it+1 are read one iteration ahead of their
  // direct-to-LDS loads (issued just before them), so waiting for the indices
  // never waits for the X tile still in flight.
  int k_cur[GATHER ? C::XCH_PER_T : 1], k_nxt[GATHER ? C::XCH_PER_T : 1];
  auto load_kept = [&](int it, int (&kk)[GATHER ? C::XCH_PER_T : 1]) {
    if constexpr (GATHER) {
#pragma unroll
      for (int j = 0; j < C::XCH_PER_T; ++j) kk[j] = kept_tile[(int64_t)it * BK + x_row[j]];
    }
  };

  auto issue_x = [&](int it, int stage, const int (&kk)[GATHER ? C::XCH_PER_T : 1]) {
#pragma unroll
    for (int j = 0; j < C::XCH_PER_T; ++j) {
      int64_t gk = (int64_t)it * BK + x_row[j];
      if constexpr (GATHER) {
        int k = kk[j];
        k = k < 0 ? 0 : (k >= args.Kx ? args.Kx - 1 : k);
        gk = k;
      }
      const uint16_t* src = args.X + gk * args.ldx + x_col[j];
      uint8_t* dst = xs + stage * C::STAGE_BYTES + (j * C::NWAVES + wave) * 64 * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)dst, 16, 0, 0);
    }
  };

  // ---- register state ----
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  bf16x8 a_cur[TM][ASTEPS], a_nxt[TM][ASTEPS];
  uint32_t m_cur[TM], m_nxt[TM];

  auto load_a = [&](int it, bf16x8 (&a)[TM][ASTEPS], uint32_t (&mt)[TM]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int s = 0; s < ASTEPS; ++s)
        a[i][s] = *reinterpret_cast<const bf16x8*>(a_ptr[i] + ((int64_t)it * ASTEPS + s) * 512);
      if constexpr (SPARSE) mt[i] = m_ptr[i][(int64_t)it * 64];
    }
  };

  // per-lane part of the transposed-read address of B fragment j (see the lane map above)
  const int li = lane & 15, h = lane >> 5, g16 = (lane >> 4) & 1;
  uint32_t b_off[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int c = (wn * C::WTN) / 8 + 4 * j + 2 * g16 + ((li & 3) >> 1);
    const int cs = c ^ chunk_swizzle(li >> 2);
    b_off[j] = xs_base + (8 * h + (li >> 2)) * C::ROWB + cs * 16 + (li & 1) * 8;
  }

  // B fragments of one K step: sparse 32 k (4 transposed reads per fragment),
  // dense 16 k (2 reads).  KB is the step's first tile row.
  auto read_b_sparse = [&](auto KB, uint32_t stage_off, i16x16 (&bf)[TN]) {
    constexpr int R = decltype(KB)::value * C::ROWB;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint32_t a = b_off[j] + stage_off;
      const i16x4 q0 = ds_read_tr<R>(a);
      const i16x4 q1 = ds_read_tr<R + 4 * C::ROWB>(a);
      const i16x4 q2 = ds_read_tr<R + 16 * C::ROWB>(a);
      const i16x4 q3 = ds_read_tr<R + 20 * C::ROWB>(a);
      const i16x8 lo = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
      const i16x8 hi = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
      bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
  };
  auto read_b_dense = [&](auto KB, uint32_t stage_off, i16x8 (&bf)[TN]) {
    constexpr int R = decltype(KB)::value * C::ROWB;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint32_t a = b_off[j] + stage_off;
      const i16x4 q0 = ds_read_tr<R>(a);
      const i16x4 q1 = ds_read_tr<R + 4 * C::ROWB>(a);
      bf[j] = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  // Wait for all LDS reads and tie the wait to the fragments that carry them.
  auto wait_b16 = [&](i16x16 (&bf)[TN]) {
    static_assert(TN <= 4, "wait helper covers up to 4 fragments");
    if constexpr (TN == 4)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]));
    else if constexpr (TN == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bf[0]), "+v"(bf[1]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bf[0]));
  };
  auto wait_b8 = [&](i16x8 (&bf)[TN]) {
    if constexpr (TN == 4)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]));
    else if constexpr (TN == 2)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bf[0]), "+v"(bf[1]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bf[0]));
  };

  auto compute = [&](int stage) {
    const uint32_t so = (uint32_t)(stage * C::STAGE_BYTES);
    if constexpr (SPARSE) {
      i16x16 b0[TN], b1[TN];
      read_b_sparse(std::integral_constant<int, 0>{}, so, b0);
      wait_b16(b0);
      read_b_sparse(std::integral_constant<int, 32>{}, so, b1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a_cur[i][0], __builtin_bit_cast(bf16x16, b0[j]),
                                                                acc[i][j], (int)m_cur[i], 0, 0);
      wait_b16(b1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a_cur[i][1], __builtin_bit_cast(bf16x16, b1[j]),
                                                                acc[i][j], (int)m_cur[i], 0, 1);
    } else {
      i16x8 bb[2][TN];
      read_b_dense(std::integral_constant<int, 0>{}, so, bb[0]);
      static_for<0, 4>([&](auto SS) {
        constexpr int ss = decltype(SS)::value;
        wait_b8(bb[ss & 1]);
        if constexpr (ss + 1 < 4) read_b_dense(std::integral_constant<int, 16 * (ss + 1)>{}, so, bb[(ss + 1) & 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_cur[i][ss], __builtin_bit_cast(bf16x8, bb[ss & 1][j]),
                                                                acc[i][j], 0, 0, 0);
      });
    }
  };

  // ---- main loop ----
  // Issue order per iteration it: [wait X(it); barrier; X(it+2) -> stage (it+2)%3;
  // A(it+1) -> registers; compute(it)].  Vector-memory counters retire in issue
  // order, so "X(it) has landed" is vmcnt <= (loads issued after it), which is at
  // least |X(it+1)| + |A(it)| while a next tile exists and |A(it)| at the last.
  load_kept(0, k_cur);
  issue_x(0, 0, k_cur);
  if (nk > 1) {
    load_kept(1, k_cur);
    issue_x(1, 1, k_cur);
  }
  if (nk > 2) load_kept(2, k_cur);
  load_a(0, a_cur, m_cur);
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk)
      wait_vmcnt<C::XCH_PER_T + A_LOADS>();
    else
      wait_vmcnt<A_LOADS>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + 3 < nk) load_kept(it + 3, k_nxt);
    if (it + 2 < nk) issue_x(it + 2, (it + 2) % NSTAGE, k_cur);
    if (it + 1 < nk) load_a(it + 1, a_nxt, m_nxt);
    asm volatile("" ::: "memory");
    compute(it % NSTAGE);
    if constexpr (GATHER) {
#pragma unroll
      for (int j = 0; j < C::XCH_PER_T; ++j) k_cur[j] = k_nxt[j];
    }
    if (it + 1 < nk) {
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
  const int col_l = n0 + wn * C::WTN + (lane & 31);
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
