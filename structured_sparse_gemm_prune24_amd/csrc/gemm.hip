// Tile loop for Y = W X on gfx950: 2:4-sparse W on the sparse MFMA
// (v_smfmac_f32_32x32x32_bf16), optionally with a TVW row gather of X, and the
// dense bf16 baseline on v_mfma_f32_32x32x16_bf16.
//
// Data flow per block (BM x BN outputs, K consumed 64 logical columns at a time):
//   * Both operands stream global -> LDS with direct-to-LDS buffer loads
//     (buffer_load_dwordx4 / _dword with the LDS flag: lane l writes its 16 / 4
//     bytes at the wave's LDS base + l * size) into a ring of LDS stages,
//     NSTAGE-1 K steps ahead of the compute.  No register holds data in
//     flight, so the accumulators own the register file.  The two-stage
//     gathered tiles refill each stage by 32-k halves, each half as soon as
//     every wave is done with it, which gives a load a step and a half.
//   * On the sparse tiles both the loads of a later step and the fragment
//     reads of the next half-step go out spread over the MFMAs, a few after
//     each, so that a wave stalled on a full memory or LDS queue holds back
//     one instruction rather than its MFMAs.
//   * W operand: the compressed values / metadata (or the packed dense W) are
//     stored in MFMA operand order, so one K step of one 32-row block is a
//     contiguous 1 KiB (values) or 256 B (metadata) run in memory, in LDS, and
//     in the wave's registers (lane l reads 16 B at +16 l).
//   * X operand: 64 x BN tiles, row-major (N contiguous).  Rows are whole
//     N-slices, so the TVW gather only changes the global row a slice comes
//     from.  Inside an LDS row the 16 B chunks are XOR-swizzled by the row's
//     low bits so that the transposed reads spread over all LDS banks.
//   * B fragments come out of LDS with ds_read_b64_tr_b16: within a group of
//     16 lanes, lane i receives element i%4 of the 8-byte pieces addressed by
//     lanes 4e + i/4 (e = 0..3), i.e. 4 consecutive k of one column when the
//     16 lanes address a 4-row x 16-column sub-tile.
//   * Every LDS read is inline asm followed by an explicit lgkmcnt wait tied
//     to the registers it fills: the compiler would otherwise stall each LDS
//     read on all outstanding direct-to-LDS loads.  The direct-to-LDS loads are
//     waited for explicitly (vmcnt, which retires in issue order) before the
//     block barrier that publishes a stage.
//   * Tails: addresses are clamped instead of branched on.  Columns of X at or
//     beyond N only feed output columns that are never stored, rows past M
//     only feed rows that are never stored, and K steps past the end are
//     loaded into stages that are never read, so every count is static.
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 64;                 // logical K per main-loop iteration
constexpr int LDS_LIMIT = 160 * 1024;  // gfx950 LDS per workgroup

// How the X operand arrives: K x N row-major (N contiguous, transposed on the
// LDS read), the same with a TVW row gather, or N x K row-major (X^T, K
// contiguous: the operand order of the MFMA, read with plain 16-byte loads).
enum XMode { X_KN = 0, X_KN_GATHER = 1, X_NK = 2, X_KN_GATHER_VAR = 3 };

// How the W operand arrives and is multiplied: packed dense bf16 on dense MFMA;
// compressed 2:4 values + metadata on the sparse MFMA (smfmac); or the same
// compressed operand expanded block-wide into a dense LDS tile (zeros in the
// pruned slots) that the dense MFMA loop then reads.
enum AMode { A_DENSE = 0, A_SPARSE = 1, A_DECOMP = 2 };

template <int BM, int BN, int WGM, int WGN, int AM, bool GATHER_X = false>
struct TileCfg {
  static constexpr bool SPARSE = AM != A_DENSE;    // compressed operand staged in LDS
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int NT = NWAVES * 64;           // threads per block
  static constexpr int WTM = BM / WGM;             // wave tile rows
  static constexpr int WTN = BN / WGN;             // wave tile cols
  static constexpr int TM = WTM / 32;              // 32x32 MFMA tiles per wave (rows)
  static constexpr int TN = WTN / 32;              // ... (cols)
  static constexpr int RB = BM / 32;               // 32-row blocks per block
  static constexpr int ASTEPS = SPARSE ? 2 : 4;    // 1 KiB A blocks per row block per K step
  // stage layout: [X tile | A blocks | metadata blocks | kept indices]
  static constexpr int ROWB = BN * 2;              // bytes per LDS row of an X tile
  static constexpr int CPR = BN / 8;               // 16 B chunks per X row
  static constexpr int X_BYTES = BK * ROWB;
  static constexpr int A_BYTES = RB * ASTEPS * 1024;
  // metadata: one 1 KiB load per group of four row blocks (a 64-row block
  // loads its whole group and reads its half; a 192-row block, which starts
  // at a group boundary or in the middle of a group, loads two groups)
  static constexpr int MG = SPARSE ? (RB % 4 == 0 ? RB / 4 : RB / 4 + 1) : 0;
  static constexpr int M_BYTES = MG * 1024;
  // gathered X on the sparse MFMA: the kept row indices of a later step (64 x 4 B)
  static constexpr int K_BYTES = GATHER_X && AM == A_SPARSE ? 256 : 0;
  static constexpr int STAGE = X_BYTES + A_BYTES + M_BYTES + K_BYTES;
  // A_DECOMP: one dense A tile (BM x BK bf16 in dense fragment order) after the stages
  static constexpr int D_BYTES = AM == A_DECOMP ? RB * 4 * 1024 : 0;
  static constexpr int NSTAGE = 3 * STAGE + D_BYTES <= LDS_LIMIT ? 3 : 2;
  // Waves that issue the stage loads.  With 8 waves, two per SIMD, only the
  // first four load (one per SIMD, waves taking SIMDs in turn): after each
  // stage barrier the other wave of the SIMD goes straight to its multiplies
  // while its partner issues the loads.  Measured (graph replay, A/B against
  // all eight waves loading): 8192^3 sparse 523 -> 505 us, X given N x K
  // 518 -> 492 us, dense 835 -> 792 us; BERT FFN 18.6 -> 18.1 us.  The
  // gathered products keep all eight: their loaders also fetch the kept row
  // indices, and the 4096^3 TVW product measured 60 -> 63 us with four.  It
  // needs the four loaders' counts to fit the 6-bit load counter with
  // NSTAGE - 1 steps in flight.
  static constexpr int LW_HALF = NWAVES / 2;
  static constexpr bool HALF_LOAD =
      !GATHER_X && NWAVES == 8 && (X_BYTES / 1024 / LW_HALF + A_BYTES / 1024 / LW_HALF + 1) * 3 < 64;
  static constexpr int LW = HALF_LOAD ? LW_HALF : NWAVES;
  // direct-to-LDS loads per loading wave per K step (each moves 1 KiB, or 256 B for metadata)
  static constexpr int X_DMA = X_BYTES / 1024 / LW;
  static constexpr int A_DMA = A_BYTES / 1024 / LW;
  // waves 0 .. MG-1 issue one metadata load per step on top of their share
  // of X and A, so the per-wave load counts differ by one
  static constexpr int DMA_O = X_DMA + A_DMA;
  static constexpr int DMA_M = DMA_O + 1;
  static_assert(BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "wave tiles must be multiples of 32");
  static_assert(X_BYTES % (1024 * LW) == 0 && A_BYTES % (1024 * LW) == 0, "even load split");
  static_assert(AM != A_DECOMP || RB % NWAVES == 0, "the expansion splits row blocks evenly among waves");
  static_assert(RB % 4 == 0 || RB == 2 || RB == 6, "row blocks: whole metadata groups, one half, or one and a half");
  static_assert(MG <= LW, "one metadata load per loading wave at most");
  static_assert(CPR >= 16, "the chunk swizzle needs at least 16 chunks per row");
  static_assert(2 * STAGE + D_BYTES <= LDS_LIMIT, "two stages must fit in LDS");
  static_assert(3 * DMA_M < 64, "vmcnt range");
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// XOR applied to the 16 B chunk index of X-tile row r.  The 4 rows of one
// transposed read land on 32 B bank groups {0,3,5,6} (x2 chunks): distinct
// both modulo 4 and, as pairs, modulo 8 groups.
__device__ __forceinline__ int chunk_swizzle(int r) {
  const int q = r & 3;
  return ((q << 1) | (__builtin_popcount(q) & 1)) << 1;
}

template <int OFF>
__device__ __forceinline__ i16x4 lds_read_tr(uint32_t addr) {
  i16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ i16x8 lds_read_b128(uint32_t addr) {
  i16x8 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_read_b32(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// vmcnt wait for a count that depends on whether this wave issues a metadata
// load per step (the wave index is uniform, so this is a scalar branch).
template <int N_META, int N_OTHER>
__device__ __forceinline__ void wait_vmcnt_by_wave(bool meta_wave) {
  if (meta_wave) wait_vmcnt<N_META>();
  else wait_vmcnt<N_OTHER>();
}

// lgkmcnt(0) tied to the registers that carry the LDS reads: every use of
// those registers is ordered after the wait.
template <typename T, int N>
__device__ __forceinline__ void wait_lds(T (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}


struct GemmArgs {
  const uint16_t* A;       // sparse: device-layout values; dense: packed W
  const uint32_t* Ameta;   // sparse: device-layout metadata
  const int32_t* kept;     // TVW: [T][Kc] gathered X rows (nullptr otherwise); per-tile keep: all tiles' lists
  const int64_t* offsets;  // per-tile keep: [T + 1] first kept column of each tile in the concatenated storage
  const int32_t* order;    // per-tile keep: tile of each block-row slot (heaviest first)
  const uint16_t* X;
  void* Y;
  int64_t ldx, ldy;
  int M, N, Kc, Kx;        // Kc: K of the W operand (compacted for TVW); Kx: rows of X
  int tile_m;              // TVW tile rows
  int nbm, nbn;            // block grid
  const float* bias;       // fused epilogue: one value per output row, or nullptr
  int act;                 // fused epilogue: P24_ACT_NONE / _RELU / _GELU
};

// GELU in its exact form z * Phi(z) = z/2 (1 + erf(z / sqrt 2)), fp32.  erf
// comes from Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for x >= 0, erfc(x) = (a1 t + ... + a5 t^5) exp(-x^2) + e(x),
// t = 1 / (1 + p x), |e(x)| <= 1.5e-7.  With q = erfc(|z| / sqrt 2) the result
// is z/2 (2 - q) for z >= 0 and z/2 q below, which keeps the negative side
// free of cancellation.
__device__ __forceinline__ float gelu_f32(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float q = poly * __builtin_amdgcn_exp2f(-x * x * 1.44269504088896341f);
  return 0.5f * z * (z >= 0.0f ? 2.0f - q : q);
}

// Epilogue activation in fp32.
__device__ __forceinline__ float apply_act(float v, int act) {
  if (act == P24_ACT_RELU) return v > 0.0f ? v : 0.0f;
  if (act == P24_ACT_GELU) return gelu_f32(v);
  return v;
}

// Buffer resource over [base, base + bytes): raw (untyped) loads, no swizzle.
// Loads past `bytes` return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 4, voff, soff, 0, 0);
}

template <int BM, int BN, int WGM, int WGN, int AM, int XM, typename OutT, int EPI>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm(const GemmArgs args) {
  using C = TileCfg<BM, BN, WGM, WGN, AM, XM == X_KN_GATHER || XM == X_KN_GATHER_VAR>;
  constexpr bool SPARSE = C::SPARSE, SMFMAC = AM == A_SPARSE, DECOMP = AM == A_DECOMP;
  constexpr bool VAR = XM == X_KN_GATHER_VAR;
  constexpr bool GATHER = XM == X_KN_GATHER || VAR;
  static_assert(!VAR || BM == 128, "per-tile keep: one block row per 128-row tile");
  constexpr bool XT = XM == X_NK;
  constexpr int TM = C::TM, TN = C::TN, ASTEPS = C::ASTEPS, NSTAGE = C::NSTAGE;
  static_assert(!DECOMP || XM == X_KN, "the expanded-tile path reads X as K x N");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * C::STAGE + C::D_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- block -> output tile ----
  int bm, bn;
  if constexpr (VAR) {
    // Per-tile keep counts: block-row slots in the order the host gives
    // (heaviest tile first, so the light ones fill the tail), the N blocks of
    // one slot back to back: the 8 XCDs, which take consecutive blocks in
    // turn, work through the slots together and each keeps to the same
    // eighth of the X column slices.
    const int slot = (int)(blockIdx.x / (uint32_t)args.nbn);
    bn = (int)(blockIdx.x % (uint32_t)args.nbn);
    bm = args.order[slot];
  } else {
    // XCD-aware, grouped raster
    const uint32_t nblocks = (uint32_t)args.nbm * args.nbn;
    const uint32_t b = xcd_remap(blockIdx.x, nblocks);
    constexpr uint32_t GROUP = 8;
    const uint32_t group_size = GROUP * args.nbn;
    const uint32_t first_m = (b / group_size) * GROUP;
    const uint32_t gsz = min((uint32_t)args.nbm - first_m, GROUP);
    bm = first_m + (b % group_size) % gsz;
    bn = (b % group_size) / gsz;
  }
  const int m0 = bm * BM, n0 = bn * BN;

  const int M = args.M, N = args.N;
  // The W operand of this block: with per-tile keep counts the tile's own
  // storage (128 rows, its own compacted K), else the whole matrix.
  const uint16_t* A = args.A;
  const uint32_t* Ameta = args.Ameta;
  int Kc = args.Kc, a_rows = M, a_m0 = m0;
  int64_t var_p = 0;
  if constexpr (VAR) {
    var_p = args.offsets[bm];
    Kc = (int)(args.offsets[bm + 1] - var_p);
    A += var_p * (SPARSE ? 64 : 128);   // 128 rows x Kc/2 values (sparse) or Kc values (dense) per tile
    Ameta += var_p * 4;                 // sparse: 16 B of metadata per kept column
    a_rows = M - m0 < BM ? M - m0 : BM;
    a_m0 = 0;
  }
  const int nk = Kc / BK;
  const int nrb = (a_rows + 31) / 32;
  const int rb0 = a_m0 / 32;
  const int64_t S = SPARSE ? Kc / 32 : Kc / 16;    // A blocks per row block
  const int64_t T_ = Kc / 64;
  const int n_hi = ((N + 7) & ~7) - 8;             // last 8-aligned column start inside the readable row
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
  const int64_t ldx = args.ldx;

  // ---- direct-to-LDS load plan ----
  // X: load j of this wave fills tile chunks [(j*NWAVES + wave)*64, +64), one
  // per lane.  A 64-lane load covers 64/CPR whole rows, so the chunk position
  // inside the row (hence the swizzled source column) is the same for every j
  // and the row advances by a fixed multiple of 4: one per-lane offset plus a
  // scalar stride covers every load.
  static_assert(C::CPR % 32 == 0 || 64 % C::CPR == 0, "row/chunk split of a 64-lane load");
  constexpr int X_ROWS_PER_LOAD = 64 / C::CPR > 0 ? 64 / C::CPR : 1;     // rows one 64-lane load covers
  constexpr int X_LOADS_PER_ROW = C::CPR / 64 > 0 ? C::CPR / 64 : 1;     // loads per row when CPR > 64
  static_assert(X_LOADS_PER_ROW == 1, "BN <= 512");
  const int p0 = wave * 64 + lane;                   // chunk of load j = 0
  const int x_r0 = p0 / C::CPR;                      // its tile row; load j adds j * LW * X_ROWS_PER_LOAD rows
  int x_col = n0 + 8 * ((p0 % C::CPR) ^ chunk_swizzle(x_r0));
  x_col = x_col <= n_hi ? x_col : n_hi;
  constexpr int X_ROW_STEP = C::LW * X_ROWS_PER_LOAD;   // multiple of 4: the swizzle of row x_r0 holds for all j
  static_assert(X_ROW_STEP % 4 == 0, "X row step must keep the swizzle phase");
  uint32_t x_voff = GATHER ? (uint32_t)x_col * 2 : (uint32_t)(x_r0 * ldx + x_col) * 2;
  // X^T (N x K): the stage holds BN rows (n) of 64 k = 8 chunks of 16 B.  LDS
  // slot of (n, chunk c) = (n ^ ((n >> 3) & 1)) * 8 + (c ^ (n & 7)): rows n and
  // n+8 land in opposite 128 B halves of a bank line and the chunk XOR spreads 8
  // rows over the 8 slots of a half, so 16 consecutive n at one chunk (one
  // quarter of a 16-byte-per-lane read) hit 16 distinct bank groups.  Load j of
  // this wave fills slots [(j*NWAVES + wave)*64, +64): rows 8q .. 8q+7, q = j*NWAVES + wave.
  uint32_t xt_jstride = 0;
  if constexpr (XT) {
    const int q = wave;                                     // j = 0
    const int n_loc = 8 * q + ((lane >> 3) ^ (q & 1));      // row' = 8q + lane/8, n = row' ^ (q & 1)
    const int c = (lane & 7) ^ (n_loc & 7);
    x_voff = (uint32_t)(n_loc * ldx + 8 * c) * 2;
    xt_jstride = (uint32_t)(8 * C::LW * ldx * 2);           // q advances by LW (even: parity kept)
    static_assert(C::LW % 2 == 0, "X^T loads keep the row-pair parity per wave");
  }
  // A values: load j fills the (row block, step) block q = j*NWAVES + wave of
  // the stage.  Metadata: wave w < MG loads group w (four row blocks, 1 KiB per
  // K-pair).  Only the lane part of an address is per lane; the block part is
  // wave-uniform and goes into the scalar offset.  Blocks past the matrix read
  // past the resource end and come back as zeros.
  const uint32_t a_voff = (uint32_t)lane * 16;
  auto a_block_off = [&](int j) -> uint32_t {
    const int q = j * C::LW + wave;
    return (uint32_t)(((q / ASTEPS) * S + q % ASTEPS) * 1024);
  };
  const bool meta_wave = wave < C::MG;
  // waves with one load per step beyond their share of X and A: the metadata
  // loaders and, for a gather on the sparse MFMA, the wave that brings the
  // kept indices (defined below)
  bool extra_wave = meta_wave;
  const int rb_end = nrb < rb0 + C::RB ? nrb : rb0 + C::RB;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      make_rsrc(A + (int64_t)rb0 * S * 512, (uint32_t)((rb_end - rb0) * S * 1024));
  const int ngroups = (int)(device_row_blocks(a_rows) / 4);  // metadata groups in the array
  const int g0 = rb0 / 4;
  const int g_end = ngroups < g0 + C::MG ? ngroups : g0 + C::MG;
  const __amdgpu_buffer_rsrc_t m_rsrc =
      SPARSE ? make_rsrc(Ameta + (int64_t)g0 * T_ * 256, (uint32_t)((g_end - g0) * T_ * 1024)) : a_rsrc;
  const int m_in_group = C::RB % 4 ? (rb0 & 3) : 0;        // first row block's place in its metadata group
  const int n_rows = N - n0 < BN ? N - n0 : BN;
  const __amdgpu_buffer_rsrc_t xt_rsrc =
      make_rsrc(args.X + (XT ? (int64_t)n0 * ldx : 0), (uint32_t)(XT ? (int64_t)n_rows * ldx * 2 : 0));
  // TVW: whole-X resource (the host guarantees it spans < 4 GiB)
  const __amdgpu_buffer_rsrc_t xg_rsrc = make_rsrc(args.X, (uint32_t)(GATHER ? (int64_t)args.Kx * ldx * 2 : 0));

  const int32_t* kept_tile = nullptr;
  if constexpr (VAR) kept_tile = args.kept + var_p;
  else if constexpr (GATHER) kept_tile = args.kept + (int64_t)(m0 / args.tile_m) * Kc;
  // TVW: the gathered X rows of step g are read one step before their loads
  // are issued (and are issued before them), so waiting for the indices never
  // waits for a tile in flight.
  // Only the loading waves read kept entries: their rows x_r0 + j * X_ROW_STEP
  // cover exactly the step's BK entries, while the rows the other waves would
  // compute run past the step (and, on a tile's last step, past its list).
  static_assert(!GATHER || C::X_DMA * X_ROW_STEP == BK, "a loading wave's kept rows stay inside the step");
  int k_cur[GATHER ? C::X_DMA : 1], k_nxt[GATHER ? C::X_DMA : 1];
  auto load_kept = [&](int g, int (&kk)[GATHER ? C::X_DMA : 1]) {
    if (C::LW < C::NWAVES && wave >= C::LW) return;
    if constexpr (GATHER) {
#pragma unroll
      for (int j = 0; j < C::X_DMA; ++j) kk[j] = kept_tile[(int64_t)g * BK + x_r0 + j * X_ROW_STEP];
    }
  };
  // On the sparse MFMA the indices travel through LDS instead: the loads of
  // step g also bring the 64 indices of step g + NSTAGE into the stage's last
  // 256 B (one 4-byte load per lane, by wave MG), ordered so that a lane's
  // X_DMA entries are consecutive: position x_r0 * X_DMA + j holds entry
  // x_r0 + j * X_ROW_STEP.  A wave reads them from the stage with that
  // stage's fragments, so the loads of step g + NSTAGE, issued one step
  // later, find their rows in registers and never wait on a global load.
  constexpr bool KG = C::K_BYTES > 0;
  // When one X load covers one whole row (512-wide blocks) a load's row is
  // the same for the whole wave: each lane then holds one of the wave's
  // indices (lane j those of load j) and a load takes its row offset as a
  // scalar (readlane), instead of every lane holding all of them.
  constexpr bool KU = KG && X_ROWS_PER_LOAD == 1;
  static_assert(!KG || ((KU ? C::X_DMA <= 64 : C::X_DMA % 4 == 0) && C::MG < C::LW),
                "kept indices: one per lane or whole 16-byte reads, a free loading wave");
  constexpr int KV = KU ? 1 : (KG ? C::X_DMA / 4 : 1);
  using KvT = typename std::conditional<KU, int, i32x4>::type;
  const uint32_t ldx2 = (uint32_t)(ldx * 2);   // X row pitch in bytes (< 4 GiB for a gather)
  constexpr int K_OFF = C::X_BYTES + C::A_BYTES + C::M_BYTES;
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(kept_tile, (uint32_t)(KG ? Kc * 4 : 0));
  const uint32_t k_voff = (uint32_t)((lane / C::X_DMA) + (lane % C::X_DMA) * X_ROW_STEP) * 4;
  const bool kept_wave = KG && wave == C::MG;
  extra_wave = extra_wave || kept_wave;
  KvT kv_cur[KV], kv_nxt[KV];

  // Load q of a loading wave's list for K step g into stage st: X loads
  // first (q < X_DMA), then A (q < X_DMA + A_DMA), then the metadata load of
  // the waves that take one.  The caller keeps the non-loading waves out.
  constexpr int NQ = C::X_DMA + C::A_DMA + (SPARSE ? 1 : 0);
  const bool loader = !(C::LW < C::NWAVES && wave >= C::LW);
  auto issue_one = [&](auto QC, int g, int st) {
    constexpr int q = decltype(QC)::value;
    uint8_t* stage = lds + st * C::STAGE;
    if constexpr (q < C::X_DMA) {
      constexpr int j = q;
      if constexpr (KU) {
        int k = __builtin_amdgcn_readlane(kv_cur[0], j);
        k = k < 0 ? 0 : (k >= args.Kx ? args.Kx - 1 : k);
        dma16_to_lds(xg_rsrc, stage + (j * C::LW + wave) * 1024, x_voff, (uint32_t)k * ldx2);
      } else if constexpr (GATHER) {
        int k;
        if constexpr (KG) k = kv_cur[j / 4][j % 4];
        else k = k_cur[j];
        k = k < 0 ? 0 : (k >= args.Kx ? args.Kx - 1 : k);
        dma16_to_lds(xg_rsrc, stage + (j * C::LW + wave) * 1024, (uint32_t)(k * ldx * 2) + x_voff, 0);
      } else if constexpr (XT) {
        dma16_to_lds(xt_rsrc, stage + (j * C::LW + wave) * 1024, x_voff, (uint32_t)g * BK * 2 + j * xt_jstride);
      } else {
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(args.X + (int64_t)g * BK * ldx, (uint32_t)(BK * ldx * 2));
        dma16_to_lds(xr, stage + (j * C::LW + wave) * 1024, x_voff, (uint32_t)(j * X_ROW_STEP * ldx * 2));
      }
    } else if constexpr (q < C::X_DMA + C::A_DMA) {
      constexpr int j = q - C::X_DMA;
      dma16_to_lds(a_rsrc, stage + C::X_BYTES + (j * C::LW + wave) * 1024, a_voff,
                   (uint32_t)g * ASTEPS * 1024 + a_block_off(j));
    } else if constexpr (SPARSE) {
      if (meta_wave)
        dma16_to_lds(m_rsrc, stage + C::X_BYTES + C::A_BYTES + wave * 1024, a_voff,
                     (uint32_t)g * 1024 + (uint32_t)wave * T_ * 1024);
      else if (kept_wave)
        dma4_to_lds(k_rsrc, stage + K_OFF, k_voff, (uint32_t)min(g + NSTAGE, nk - 1) * BK * 4);
    }
  };
  // loads [Q0, Q1) of K step g into stage st
  auto issue_range = [&](auto Q0, auto Q1, int g, int st) {
    if (!loader) return;
    static_for<decltype(Q0)::value, decltype(Q1)::value>([&](auto Q) { issue_one(Q, g, st); });
  };
  // all direct-to-LDS loads of K step g into stage st (loading waves only)
  auto issue_step = [&](int g, int st) {
    issue_range(std::integral_constant<int, 0>{}, std::integral_constant<int, NQ>{}, g, st);
  };
  // The loads of a step split by the 32-k half of the stage they fill, for
  // the two-stage gathered tiles (one row per X load): half 0 takes X rows
  // 0..31 (loads j < X_DMA / 2) and the metadata and kept indices (both read
  // along with half 0), half 1 X rows 32..63.  A load j of wave w fills A
  // block j * LW + w, which is row block (j * LW + w) / 2 at k half w % 2 (LW
  // even), so the even waves' A loads go with half 0 and the odd waves' with
  // half 1.  Load k of half HC; NH0 and NH1 loads per half.
  constexpr int XH = C::X_DMA / 2, NH0 = XH + C::A_DMA + 1, NH1 = XH + C::A_DMA;
  auto issue_h = [&](auto HC, auto KC, int g, int st) {
    constexpr int hf = decltype(HC)::value, k = decltype(KC)::value;
    if constexpr (k < XH) {
      issue_one(std::integral_constant<int, hf * XH + k>{}, g, st);
    } else if constexpr (k < XH + C::A_DMA) {
      if ((wave & 1) == hf) issue_one(std::integral_constant<int, C::X_DMA + k - XH>{}, g, st);
    } else {
      static_assert(hf == 0 && k == XH + C::A_DMA, "the extra load goes with half 0");
      issue_one(std::integral_constant<int, C::X_DMA + C::A_DMA>{}, g, st);
    }
  };

  // ---- LDS read addresses, one set per stage ----
  const int li = lane & 15, h = lane >> 5, g16 = (lane >> 4) & 1;
  uint32_t b_off[NSTAGE][TN], a_off[NSTAGE], m_off[NSTAGE];
#pragma unroll
  for (int st = 0; st < NSTAGE; ++st) {
    const uint32_t base = lds_base + st * C::STAGE;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c = (wn * C::WTN) / 8 + 4 * j + 2 * g16 + ((li & 3) >> 1);
      const int cs = c ^ chunk_swizzle(li >> 2);
      b_off[st][j] = base + (8 * h + (li >> 2)) * C::ROWB + cs * 16 + (li & 1) * 8;
    }
    a_off[st] = DECOMP ? lds_base + NSTAGE * C::STAGE + wm * TM * 4 * 1024 + lane * 16
                       : base + C::X_BYTES + wm * TM * ASTEPS * 1024 + lane * 16;
    m_off[st] = base + C::X_BYTES + C::A_BYTES + (m_in_group + wm * TM) * 256 + lane * 4;
  }
  // X^T fragments: lane (column n = wave cols + 32 j + lane % 32, half h) reads
  // 16 B chunks of k; the fragment j offset (32 rows = 4 KiB) is an immediate.
  uint32_t xt_off[XT ? NSTAGE : 1][4];
  if constexpr (XT) {
    const int nl = lane & 31;
    const uint32_t row = (uint32_t)(wn * C::WTN + (nl ^ ((nl >> 3) & 1))) * 128;
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // sparse: q = 2*ss + e reads chunk 4ss + 2e + h; dense: q = ss reads chunk 2ss + h
        const int c = SMFMAC ? (4 * (q >> 1) + 2 * (q & 1) + h) : (2 * q + h);
        xt_off[st][q] = lds_base + st * C::STAGE + row + (uint32_t)((c ^ (nl & 7)) * 16);
      }
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

  // A_DECOMP: expand the compressed W of stage ST into the dense tile.  Thread
  // (row block q, lane L) takes lane L of the two 32-k value blocks of q and its
  // metadata word: value block s' holds row L % 32, k 32 s' + 16 (L / 32) + [0, 16)
  // as 4 groups of (2 values, one nibble: position of the first value in bits
  // 0-1, of the second in bits 2-3).  Those 16 dense k are the first 8 k of
  // dense lane L % 32 and the last 8 of dense lane L % 32 + 32 in the dense
  // 16-k block 2 s' + L / 32.
  auto expand = [&](auto ST) {
    constexpr int st = decltype(ST)::value;
    const uint32_t cbase = lds_base + st * C::STAGE + C::X_BYTES;
    const uint32_t dbase = lds_base + NSTAGE * C::STAGE;
    static_for<0, C::RB / C::NWAVES>([&](auto J) {
      const int q = decltype(J)::value * C::NWAVES + wave;
      const uint32_t va = cbase + q * ASTEPS * 1024 + lane * 16;
      uint32_t mw[1] = {lds_read_b32<0>(cbase + C::A_BYTES + (m_in_group + q) * 256 + lane * 4)};
      i16x8 v[2] = {lds_read_b128<0>(va), lds_read_b128<1024>(va)};
      wait_lds(mw);
      wait_lds(v);
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const u32x4 w = __builtin_bit_cast(u32x4, v[sp]);
        uint32_t d[8];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t nib = mw[0] >> (16 * sp + 4 * g);
          const uint64_t e = ((uint64_t)(w[g] & 0xFFFFu) << (16 * (nib & 3))) |
                             ((uint64_t)(w[g] >> 16) << (16 * ((nib >> 2) & 3)));
          d[2 * g] = (uint32_t)e;
          d[2 * g + 1] = (uint32_t)(e >> 32);
        }
        const uint32_t dst = dbase + (q * 4 + 2 * sp + (lane >> 5)) * 1024 + (lane & 31) * 16;
        const u32x4 lo = {d[0], d[1], d[2], d[3]}, hi = {d[4], d[5], d[6], d[7]};
        asm volatile("ds_write_b128 %0, %1" ::"v"(dst), "v"(lo) : "memory");
        asm volatile("ds_write_b128 %0, %1 offset:512" ::"v"(dst), "v"(hi) : "memory");
      }
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // Sparse-MFMA fragments of stage ST, 32-k half SS (k 0..31 or 32..63 of the step).
  auto rd_meta = [&](auto ST, uint32_t (&meta)[TM]) {
    constexpr int st = decltype(ST)::value;
    static_for<0, TM>([&](auto I) { meta[decltype(I)::value] = lds_read_b32<decltype(I)::value * 256>(m_off[st]); });
  };
  // this lane's kept indices from stage ST (those of the step NSTAGE after the stage's own)
  auto rd_kept = [&](auto ST, KvT (&kv)[KV]) {
    if constexpr (KU) {
      constexpr int st = decltype(ST)::value;
      kv[0] = (int)lds_read_b32<0>(lds_base + st * C::STAGE + K_OFF + (uint32_t)(x_r0 * C::X_DMA + lane % C::X_DMA) * 4);
    } else if constexpr (KG) {
      constexpr int st = decltype(ST)::value;
      const uint32_t ad = lds_base + st * C::STAGE + K_OFF + (uint32_t)x_r0 * C::X_DMA * 4;
      static_for<0, KV>([&](auto V) {
        kv[decltype(V)::value] = __builtin_bit_cast(i32x4, lds_read_b128<decltype(V)::value * 16>(ad));
      });
    }
  };
  auto rd_a = [&](auto ST, auto SS, i16x8 (&a)[TM]) {
    constexpr int st = decltype(ST)::value;
    static_for<0, TM>([&](auto I) {
      a[decltype(I)::value] =
          lds_read_b128<(decltype(I)::value * ASTEPS + decltype(SS)::value) * 1024>(a_off[st]);
    });
  };
  auto rd_b = [&](auto ST, auto SS, i16x16 (&bf)[TN]) {
    constexpr int st = decltype(ST)::value;
    constexpr int ss = decltype(SS)::value;
    if constexpr (XT) {
      static_for<0, TN>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const i16x8 lo = lds_read_b128<j * 32 * 128>(xt_off[st][2 * ss]);
        const i16x8 hi = lds_read_b128<j * 32 * 128>(xt_off[st][2 * ss + 1]);
        bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      });
    } else {
      constexpr int R = 32 * ss * C::ROWB;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t ad = b_off[st][j];
        const i16x4 q0 = lds_read_tr<R>(ad);
        const i16x4 q1 = lds_read_tr<R + 4 * C::ROWB>(ad);
        const i16x4 q2 = lds_read_tr<R + 16 * C::ROWB>(ad);
        const i16x4 q3 = lds_read_tr<R + 20 * C::ROWB>(ad);
        const i16x8 lo = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
        const i16x8 hi = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
        bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
    }
  };
  auto mma_sparse = [&](auto SS, const i16x8 (&a)[TM], const i16x16 (&bf)[TN], const uint32_t (&meta)[TM]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                              __builtin_bit_cast(bf16x16, bf[j]), acc[i][j],
                                                              (int)meta[i], 0, decltype(SS)::value);
  };
  // The same multiplies with loads Q0 .. Q1-1 of step g (into stage st)
  // issued one after each MFMA, the rest after the last: spread out this way
  // a loading wave's vector-memory issue waits sit in the shadow of its
  // MFMAs instead of holding them back in one burst.
  // Fragment reads one at a time: read r of a half's list (the metadata
  // words, the A blocks, then the four 8-byte transposing pieces of each B
  // fragment) from stage ST, half SS.
  auto rd_one = [&](auto ST, auto SS, auto R, uint32_t (&meta)[TM], i16x8 (&a)[TM], i16x4 (&bq)[TN][4]) {
    constexpr int st = decltype(ST)::value, ss = decltype(SS)::value;
    constexpr int r = decltype(R)::value;
    if constexpr (r < TM) {
      meta[r] = lds_read_b32<r * 256>(m_off[st]);
    } else if constexpr (r < 2 * TM) {
      constexpr int i = r - TM;
      a[i] = lds_read_b128<(i * ASTEPS + ss) * 1024>(a_off[st]);
    } else {
      constexpr int q = r - 2 * TM, j = q / 4, piece = q % 4;
      constexpr int OFFS[4] = {0, 4 * C::ROWB, 16 * C::ROWB, 20 * C::ROWB};
      bq[j][piece] = lds_read_tr<32 * ss * C::ROWB + OFFS[piece]>(b_off[st][j]);
    }
  };
  auto assemble_b = [&](const i16x4 (&bq)[TN][4], i16x16 (&bf)[TN]) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const i16x8 lo = __builtin_shufflevector(bq[j][0], bq[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
      const i16x8 hi = __builtin_shufflevector(bq[j][2], bq[j][3], 0, 1, 2, 3, 4, 5, 6, 7);
      bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
  };
  // The MFMAs of half SS with this wave's loads [Q0, Q1) (loading waves only)
  // and the reads [R0, R1) of stage RST, half RSS, spread over them: after
  // MFMA k go load Q0 + k and the k-th share of the reads, all of them within
  // the first three quarters of the MFMAs so that the last ones still cover
  // the reads' latency.
  // HL: the loads are those of the step's list (HL < 0) or of its half HL
  // (issue_h).
  auto mma_io = [&](auto LD, auto HL, auto SS, const i16x8 (&a)[TM], const i16x16 (&bf)[TN],
                    const uint32_t (&meta)[TM], auto Q0, auto Q1, int g, int stl, auto RST, auto RSS, auto R0,
                    auto R1, uint32_t (&rmeta)[TM], i16x8 (&ra)[TM], i16x4 (&rbq)[TN][4]) {
    constexpr int q0 = decltype(Q0)::value, q1 = decltype(Q1)::value, hl = decltype(HL)::value;
    constexpr int r0 = decltype(R0)::value, r1 = decltype(R1)::value, NR = r1 - r0;
    constexpr int SPREAD = TM * TN * 3 / 4 > 0 ? TM * TN * 3 / 4 : 1;
    auto issue_q = [&](auto Q) {
      if constexpr (hl < 0) issue_one(Q, g, stl);
      else issue_h(std::integral_constant<int, hl>{}, Q, g, stl);
    };
    static_for<0, TM * TN>([&](auto KC) {
      constexpr int k = decltype(KC)::value, i = k / TN, j = k % TN;
      acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                            __builtin_bit_cast(bf16x16, bf[j]), acc[i][j],
                                                            (int)meta[i], 0, decltype(SS)::value);
      if constexpr (decltype(LD)::value && q0 + k < q1) issue_q(std::integral_constant<int, q0 + k>{});
      constexpr int lo = k < SPREAD ? r0 + (NR * k) / SPREAD : r1;
      constexpr int hi = k < SPREAD ? r0 + (NR * (k + 1)) / SPREAD : r1;
      static_for<lo, hi>([&](auto R) { rd_one(RST, RSS, R, rmeta, ra, rbq); });
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (decltype(LD)::value)
      static_for<q0 + TM * TN < q1 ? q0 + TM * TN : q1, q1>([&](auto Q) { issue_q(Q); });
  };
  // LD (compile time) says whether this wave loads: a branch on it here,
  // between fragment reads and their wait, would let the compiler copy the
  // read registers at the join before they have arrived.
  auto mma_sparse_loads = [&](auto LD, auto SS, const i16x8 (&a)[TM], const i16x16 (&bf)[TN],
                              const uint32_t (&meta)[TM], auto Q0, auto Q1, int g, int st) {
    constexpr int q0 = decltype(Q0)::value, q1 = decltype(Q1)::value;
    if constexpr (!decltype(LD)::value) {
      mma_sparse(SS, a, bf, meta);
      return;
    }
    static_for<0, TM * TN>([&](auto KC) {
      constexpr int k = decltype(KC)::value, i = k / TN, j = k % TN;
      acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                            __builtin_bit_cast(bf16x16, bf[j]), acc[i][j],
                                                            (int)meta[i], 0, decltype(SS)::value);
      if constexpr (q0 + k < q1) issue_one(std::integral_constant<int, q0 + k>{}, g, st);
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<q0 + TM * TN < q1 ? q0 + TM * TN : q1, q1>([&](auto Q) { issue_one(Q, g, st); });
  };

  // One K step on stage ST (dense MFMA on packed W or on the expanded tile).
  // A loading wave (LD) issues its loads for step g into stage stl spread over
  // the step's MFMAs, one after every (TM * TN * 4) / NQ of them, instead of
  // in one burst ahead of them.
  auto compute = [&](auto ST, auto LD, int g, int stl) {
    constexpr int st = decltype(ST)::value;
    if constexpr (!SMFMAC) {
      i16x8 a[2][TM], bb[2][TN];
      constexpr int DSTEPS = 4;    // dense 16-k blocks per row block per K step (packed W or expanded tile)
      auto read_step = [&](auto SS) {
        constexpr int ss = decltype(SS)::value;
        static_for<0, TM>([&](auto I) {
          a[ss & 1][decltype(I)::value] = lds_read_b128<(decltype(I)::value * DSTEPS + ss) * 1024>(a_off[st]);
        });
        if constexpr (XT) {
          static_for<0, TN>([&](auto J) {
            constexpr int j = decltype(J)::value;
            bb[ss & 1][j] = lds_read_b128<j * 32 * 128>(xt_off[st][ss]);
          });
        } else {
          constexpr int R = 16 * ss * C::ROWB;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const uint32_t ad = b_off[st][j];
            const i16x4 q0 = lds_read_tr<R>(ad);
            const i16x4 q1 = lds_read_tr<R + 4 * C::ROWB>(ad);
            bb[ss & 1][j] = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      };
      // one read of sub-step SS: A block r (r < TM), then the B pieces (two
      // transposing reads per fragment of X given K x N, one 16-byte read of X
      // given N x K)
      constexpr int DBP = XT ? 1 : 2;
      i16x4 bq[2][TN][2];
      auto read_one = [&](auto SS, auto R) {
        constexpr int ss = decltype(SS)::value, r = decltype(R)::value;
        if constexpr (r < TM) {
          a[ss & 1][r] = lds_read_b128<(r * DSTEPS + ss) * 1024>(a_off[st]);
        } else if constexpr (XT) {
          bb[ss & 1][r - TM] = lds_read_b128<(r - TM) * 32 * 128>(xt_off[st][ss]);
        } else {
          constexpr int j = (r - TM) / 2, piece = (r - TM) % 2;
          bq[ss & 1][j][piece] = lds_read_tr<16 * ss * C::ROWB + piece * 4 * C::ROWB>(b_off[st][j]);
        }
      };
      auto finish_b = [&](auto SS) {
        constexpr int ss = decltype(SS)::value;
        if constexpr (!XT) {
#pragma unroll
          for (int j = 0; j < TN; ++j)
            bb[ss & 1][j] = __builtin_shufflevector(bq[ss & 1][j][0], bq[ss & 1][j][1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      // the plain dense tiles spread the next sub-step's reads over the
      // current one's MFMAs (the first three quarters of them), as the sparse
      // loop does
      constexpr bool DIOL = !DECOMP && TM * TN >= 4;
      constexpr int NRD = TM + DBP * TN;
      read_step(std::integral_constant<int, 0>{});
      static_for<0, 4>([&](auto SS) {
        constexpr int ss = decltype(SS)::value;
        wait_lds(a[ss & 1]);
        if constexpr (DIOL && !XT && ss > 0) {
          static_for<0, TN>([&](auto J) { wait_lds(bq[ss & 1][decltype(J)::value]); });
          finish_b(SS);
        } else {
          wait_lds(bb[ss & 1]);
        }
        if constexpr (!DIOL && ss + 1 < 4) read_step(std::integral_constant<int, ss + 1>{});
        constexpr int NMF = TM * TN * 4, STRIDE = NMF / NQ > 0 ? NMF / NQ : 1;
        constexpr int SPREAD = TM * TN * 3 / 4 > 0 ? TM * TN * 3 / 4 : 1;
        static_for<0, TM * TN>([&](auto KC) {
          constexpr int k = decltype(KC)::value, i = k / TN, j = k % TN, kk = ss * TM * TN + k;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[ss & 1][i]),
                                                              __builtin_bit_cast(bf16x8, bb[ss & 1][j]),
                                                              acc[i][j], 0, 0, 0);
          if constexpr (decltype(LD)::value && kk % STRIDE == 0 && kk / STRIDE < NQ)
            issue_one(std::integral_constant<int, kk / STRIDE>{}, g, stl);
          if constexpr (DIOL && ss + 1 < 4) {
            constexpr int lo = k < SPREAD ? (NRD * k) / SPREAD : NRD;
            constexpr int hi = k < SPREAD ? (NRD * (k + 1)) / SPREAD : NRD;
            static_for<lo, hi>([&](auto R) { read_one(std::integral_constant<int, ss + 1>{}, R); });
          }
          if constexpr ((decltype(LD)::value && kk % STRIDE == 0 && kk / STRIDE < NQ) || DIOL)
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (decltype(LD)::value && ss == 3)
          static_for<(NMF + STRIDE - 1) / STRIDE < NQ ? (NMF + STRIDE - 1) / STRIDE : NQ, NQ>(
              [&](auto Q) { issue_one(Q, g, stl); });
      });
    }
  };

  // ---- main loop ----
  if constexpr (SMFMAC) {
    // Step g is loaded into stage g % NSTAGE.  The stage barrier sits between
    // the two 32-k halves of a step: after it every wave is done with stage
    // it (its reads were waited for) and sees stage it+1, so a wave refills
    // stage it with step it+NSTAGE and reads the first half of step it+1 while
    // its MFMAs on the second half of step it run.  Waves on one SIMD never
    // meet an LDS wait with an empty MFMA queue except at the block's start.
    // At the barrier of step it the loads of steps it+2 .. it+NSTAGE-1 may
    // still be in flight (vmcnt retires in issue order).  Steps past the end
    // reload the last step into a stage that is never read and the reads of
    // "step nk" go to a stage that is never used, so every count is static.
    // The loop is unrolled by NSTAGE so every stage address is a constant.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // With three stages the loads of step it+NSTAGE are split: the first P0
    // go out with the multiplies after the barrier of step it, the rest with
    // the first-half multiplies of step it+1, ahead of its barrier (so the
    // count waited for there is unchanged).  The prologue issues that first
    // part only for its last step.  With two stages every load of a step goes
    // out after the barrier, as the stage is needed one half-step later.  The
    // gathered products keep all loads after the barrier too: their X loads
    // take the kept indices that are replaced at the end of the step.  So do
    // the 4-wave tiles, where every wave loads a batch of five or six: there
    // is no burst to spread, and the ResNet-50 3x3 shape (64 x 128 tiles)
    // measured 3 % slower split.
    constexpr bool SPLIT = !GATHER && NSTAGE >= 3 && C::HALF_LOAD;
    constexpr int P0 = SPLIT ? (C::X_DMA + C::A_DMA) / 4 : NQ;
    // Scheduling fences that keep each half's fragment reads ahead of the
    // multiplies that overlap them (and those multiplies on their side of the
    // stage barrier).  Without them the scheduler sinks the reads below most
    // of the multiplies to save registers, so their latency shows at the
    // wait.  They need all four fragment sets live at once, which fits the
    // 256 registers without spilling only in the plain bf16-output variant of
    // the widest tile; measured there 1-1.5 % faster.
    constexpr bool PIN = !(BM == 256 && BN == 256) || (XM == X_KN && EPI == 0 && sizeof(OutT) == 2);
    using QP0 = std::integral_constant<int, P0>;
    using QNQ = std::integral_constant<int, NQ>;
    // Where the reads fit between the MFMAs (X given K x N, spread loads, at
    // least four MFMAs per half, and on the widest tile a bf16 output: with
    // fp32 output it would spill), each half's fragment reads for the next
    // half go out spread over its MFMAs too, a few after each, instead of all
    // ahead of them: a wave that finds the LDS queue full then holds back one
    // read, not its whole half of MFMAs.  8192^3: 461 -> 445 us and
    // 497 -> 478 us in interleaved runs on two boxes; with bias + GELU
    // 519 -> 499 us.
    // The gathered products take the same schedule with every load of a step
    // after a barrier (their stage count or kept indices rule out the split).
    constexpr bool IOL = (SPLIT || KG) && !XT && TM * TN >= 4 && (!(BM == 256 && BN == 256) || sizeof(OutT) == 2);
    // Half-stage refill (HS), for the two-stage gathered tiles: a second
    // barrier at the end of each step, after which every wave is done with
    // the first half of stage it (read during the previous step) and the
    // metadata and kept indices read with it.  The loads of step it+2 for that
    // half go out with the first-half multiplies of step it, those for the
    // second half after the middle barrier as before, so each has a step and
    // a half to land instead of one: half 0 of step it+2 is read after the
    // middle barrier of step it+1, half 1 after its end barrier.  Each barrier
    // waits for the half issued one and a half steps earlier, with the next
    // two halves (one step's loads) still in flight.
    constexpr bool HS = KG && NSTAGE == 2 && IOL;
    static_assert(!HS || (C::LW % 2 == 0 && ASTEPS == 2 && X_ROWS_PER_LOAD == 1 && XH * X_ROW_STEP == BK / 2),
                  "half-stage refill: A halves by wave parity, X loads j < X_DMA / 2 cover k 0..31");
#pragma unroll
    for (int g = 0; g < NSTAGE; ++g) {
      if constexpr (KG) {
        // the prologue's own steps take their indices straight from the list
        if (loader) {
          if constexpr (KU) {
            kv_cur[0] = kept_tile[(int64_t)min(g, nk - 1) * BK + x_r0 + (lane % C::X_DMA) * X_ROW_STEP];
          } else {
#pragma unroll
            for (int j = 0; j < C::X_DMA; ++j)
              kv_cur[j / 4][j % 4] = kept_tile[(int64_t)min(g, nk - 1) * BK + x_r0 + j * X_ROW_STEP];
          }
        }
      } else {
        load_kept(min(g, nk - 1), k_cur);
      }
      if (SPLIT && g == NSTAGE - 1) {
        issue_range(I0{}, QP0{}, min(g, nk - 1), g);
      } else if constexpr (HS) {
        // half 0 then half 1, the order the loop's counts assume
        if (loader) {
          static_for<0, NH0>([&](auto Q) { issue_h(I0{}, Q, min(g, nk - 1), g); });
          static_for<0, NH1>([&](auto Q) { issue_h(I1{}, Q, min(g, nk - 1), g); });
        }
      } else {
        issue_step(min(g, nk - 1), g);
      }
    }
    if constexpr (!KG) load_kept(min(NSTAGE, nk - 1), k_cur);
    constexpr int PRO_M = SPLIT ? (NSTAGE - 2) * C::DMA_M + P0 : (NSTAGE - 1) * C::DMA_M;
    constexpr int PRO_O = SPLIT ? (NSTAGE - 2) * C::DMA_O + P0 : (NSTAGE - 1) * C::DMA_O;
    wait_vmcnt_by_wave<PRO_M, PRO_O>(extra_wave);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The fragment reads are asynchronous (results land at the lgkmcnt wait)
    // but the compiler treats them as complete at issue, so no read result may
    // be copied before its wait: the metadata words get one register set per
    // stage (no copy between steps), and each step ends with the wait for the
    // next step's first-half reads, ahead of any copy at the loop edge.
    uint32_t meta[NSTAGE][TM];
    i16x8 a0[TM], a1[TM];
    i16x16 b0[TN], b1[TN];
    i16x4 b0q[TN][4], b1q[TN][4];
    uint32_t meta_none[TM];
    rd_meta(I0{}, meta[0]);
    rd_a(I0{}, I0{}, a0);
    rd_b(I0{}, I0{}, b0);
    wait_lds(meta[0]);
    wait_lds(a0);
    wait_lds(b0);
    // only the loading waves read kept indices (theirs are the stage's 64)
    if constexpr (KG) {
      if (loader) {
        rd_kept(I0{}, kv_cur);
        wait_lds(kv_cur);
      }
    }
    if constexpr (HS) {
      // the end barrier of "step -1": every wave is done with half 0 of stage 0
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // wait at a barrier: with HS one step's loads stay in flight, else NSTAGE - 2 steps'
    constexpr int BW_M = HS ? C::DMA_M : (NSTAGE - 2) * C::DMA_M;
    constexpr int BW_O = HS ? C::DMA_O : (NSTAGE - 2) * C::DMA_O;
    using HL0 = std::integral_constant<int, HS ? 0 : -1>;
    using HL1 = std::integral_constant<int, HS ? 1 : -1>;
    auto body_spread = [&](auto ST, auto LD, int it) {
      constexpr int st = decltype(ST)::value;
      constexpr int nx = (st + 1) % NSTAGE;
      using NR = std::integral_constant<int, 2 * TM + 4 * TN>;   // reads of a half: metadata, A, B pieces
      // first half on (a0, b0); this stage's second-half A and B reads spread
      // over it, and with HS the loads of half 0 of step it+2 into this stage
      if constexpr (HS)
        mma_io(LD, HL0{}, I0{}, a0, b0, meta[st], I0{}, std::integral_constant<int, NH0>{},
               min(it + NSTAGE, nk - 1), st, ST, I1{}, std::integral_constant<int, TM>{}, NR{}, meta_none, a1, b1q);
      else
        mma_io(LD, HL0{}, I0{}, a0, b0, meta[st], QP0{}, QNQ{}, min(it + NSTAGE - 1, nk - 1),
               (st + NSTAGE - 1) % NSTAGE, ST, I1{}, std::integral_constant<int, TM>{}, NR{}, meta_none, a1, b1q);
      wait_lds(a1);
      static_for<0, TN>([&](auto J) { wait_lds(b1q[decltype(J)::value]); });
      assemble_b(b1q, b1);
      wait_vmcnt_by_wave<BW_M, BW_O>(extra_wave);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // second half on (a1, b1); the next stage's first-half reads spread over it
      if constexpr (decltype(LD)::value) rd_kept(std::integral_constant<int, nx>{}, kv_nxt);
      if constexpr (HS)
        mma_io(LD, HL1{}, I1{}, a1, b1, meta[st], I0{}, std::integral_constant<int, NH1>{},
               min(it + NSTAGE, nk - 1), st, std::integral_constant<int, nx>{}, I0{}, I0{}, NR{}, meta[nx], a0, b0q);
      else
        mma_io(LD, HL1{}, I1{}, a1, b1, meta[st], I0{}, QP0{}, min(it + NSTAGE, nk - 1), st,
               std::integral_constant<int, nx>{}, I0{}, I0{}, NR{}, meta[nx], a0, b0q);
      __builtin_amdgcn_sched_barrier(0);
      wait_lds(meta[nx]);
      wait_lds(a0);
      static_for<0, TN>([&](auto J) { wait_lds(b0q[decltype(J)::value]); });
      assemble_b(b0q, b0);
      if constexpr (KG && decltype(LD)::value) {
        wait_lds(kv_nxt);
#pragma unroll
        for (int v = 0; v < KV; ++v) kv_cur[v] = kv_nxt[v];
      }
      if constexpr (HS) {
        wait_vmcnt_by_wave<BW_M, BW_O>(extra_wave);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    };
    auto body = [&](auto ST, auto LD, int it) {
      constexpr int st = decltype(ST)::value;
      constexpr int nx = (st + 1) % NSTAGE;
      if constexpr (IOL) {
        body_spread(ST, LD, it);
        return;
      }
      rd_a(ST, I1{}, a1);
      rd_b(ST, I1{}, b1);
      if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
      if constexpr (SPLIT)
        mma_sparse_loads(LD, I0{}, a0, b0, meta[st], QP0{}, QNQ{}, min(it + NSTAGE - 1, nk - 1),
                         (st + NSTAGE - 1) % NSTAGE);
      else
        mma_sparse(I0{}, a0, b0, meta[st]);
      if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
      wait_lds(a1);
      wait_lds(b1);
      wait_vmcnt_by_wave<(NSTAGE - 2) * C::DMA_M, (NSTAGE - 2) * C::DMA_O>(extra_wave);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
      if constexpr (!KG) load_kept(min(it + NSTAGE + 1, nk - 1), k_nxt);
      if constexpr (!SPLIT) {
        if constexpr (decltype(LD)::value) issue_step(min(it + NSTAGE, nk - 1), st);
        asm volatile("" ::: "memory");
      }
      rd_meta(std::integral_constant<int, nx>{}, meta[nx]);
      rd_a(std::integral_constant<int, nx>{}, I0{}, a0);
      rd_b(std::integral_constant<int, nx>{}, I0{}, b0);
      if constexpr (decltype(LD)::value) rd_kept(std::integral_constant<int, nx>{}, kv_nxt);
      if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
      if constexpr (SPLIT)
        mma_sparse_loads(LD, I1{}, a1, b1, meta[st], I0{}, QP0{}, min(it + NSTAGE, nk - 1), st);
      else
        mma_sparse(I1{}, a1, b1, meta[st]);
      __builtin_amdgcn_sched_barrier(0);
      wait_lds(meta[nx]);
      wait_lds(a0);
      wait_lds(b0);
      if constexpr (KG && decltype(LD)::value) {
        wait_lds(kv_nxt);
#pragma unroll
        for (int v = 0; v < KV; ++v) kv_cur[v] = kv_nxt[v];
      }
    };
    // loading and non-loading waves run separate copies of the loop (the
    // branch is taken here, with no fragment read in flight)
    auto main_loop = [&](auto LD) {
      for (int it = 0; it < nk; it += NSTAGE) {
        static_for<0, NSTAGE>([&](auto ST) {
          if (it + decltype(ST)::value < nk) body(ST, LD, it + decltype(ST)::value);
        });
      }
    };
    if (loader) main_loop(std::true_type{});
    else main_loop(std::false_type{});
  } else {
    // Step g is loaded into stage g % NSTAGE by the loads issued NSTAGE-1 steps
    // earlier.  At the top of step it the loads of steps it+1 .. it+NSTAGE-2 may
    // still be in flight (vmcnt retires in issue order), then the barrier makes
    // every wave's part of stage it visible and guarantees that no wave still
    // reads the stage about to be refilled.  Steps past the end reload the last
    // step into a stage that is never read, so the counts stay static.  The loop
    // is unrolled by NSTAGE so every stage address is fixed at compile time.
    load_kept(0, k_cur);
    issue_step(0, 0);
#pragma unroll
    for (int g = 1; g < NSTAGE - 1; ++g) {
      load_kept(min(g, nk - 1), k_cur);
      issue_step(min(g, nk - 1), g);
    }
    load_kept(min(NSTAGE - 1, nk - 1), k_cur);
    // The expanded-tile path keeps its loads ahead of the expansion.
    constexpr bool SPREAD = !DECOMP;
    auto body = [&](auto ST, auto LD, int it) {
      constexpr int st = decltype(ST)::value;
      wait_vmcnt_by_wave<(NSTAGE - 2) * C::DMA_M, (NSTAGE - 2) * C::DMA_O>(meta_wave);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int gn = min(it + NSTAGE - 1, nk - 1), sn = (st + NSTAGE - 1) % NSTAGE;
      load_kept(min(it + NSTAGE, nk - 1), k_nxt);
      if constexpr (!SPREAD) {
        issue_step(gn, sn);
        asm volatile("" ::: "memory");
      }
      if constexpr (DECOMP) {
        // the dense tile is rewritten after the barrier above (every wave is past
        // its reads of the previous step) and read after this one
        expand(ST);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      compute(ST, std::integral_constant<bool, SPREAD && decltype(LD)::value>{}, gn, sn);
      if constexpr (GATHER) {
#pragma unroll
        for (int j = 0; j < C::X_DMA; ++j) k_cur[j] = k_nxt[j];
      }
    };
    // loading and non-loading waves run separate copies of the loop (no branch
    // between a fragment read and its wait)
    auto main_loop = [&](auto LD) {
      for (int it = 0; it < nk; it += NSTAGE) {
        static_for<0, NSTAGE>([&](auto ST) {
          if (it + decltype(ST)::value < nk) body(ST, LD, it + decltype(ST)::value);
        });
      }
    };
    if (loader) main_loop(std::true_type{});
    else main_loop(std::false_type{});
  }

  // The last NSTAGE-1 steps issued loads into stages that are never read; they
  // must land before the block ends and its LDS is handed to another block.
  wait_vmcnt<0>();

  // ---- epilogue ----
  // Each wave passes its tile through LDS one 32-row slice at a time: the
  // MFMA result holds one column per lane, the store wants rows.  Slice i is
  // written as [32 rows][WTN cols] with a 16 B pad per row (the two row
  // halves a write instruction touches land on disjoint banks), read back as
  // 16 B row pieces and stored whole when Y allows it, element by element at
  // ragged edges or for an unaligned Y.  The fused variants (EPI = 1: bias,
  // ReLU; EPI = 2: bias, GELU) stage acc + bias in fp32 and apply the
  // activation and the output rounding on the way out.  Whole pieces go out
  // as non-temporal stores: Y is written once and not read here, and
  // allocating it in L2 would evict the X and W lines that the blocks still
  // running on the same XCD share (4-5 % on the 8192^3 product).
  __builtin_amdgcn_s_barrier();   // every wave's loads have landed and its reads are done
  asm volatile("" ::: "memory");
  constexpr bool FUSED = EPI != 0;
  using StageT = typename std::conditional<FUSED, float, OutT>::type;
  constexpr int ES = (int)sizeof(OutT);
  constexpr int SES = (int)sizeof(StageT);
  constexpr int PITCH = C::WTN * SES + 16;          // bytes per staged row
  constexpr int VEC = 16 / SES;                     // staged elements per 16 B piece
  constexpr int PPR = C::WTN / VEC;                 // pieces per row
  constexpr int PPL = 32 * PPR / 64;                // pieces per lane per slice
  static_assert(C::NWAVES * 32 * PITCH <= NSTAGE * C::STAGE + C::D_BYTES, "epilogue staging fits in LDS");
  static_assert((32 * PPR) % 64 == 0, "whole pieces per lane");
  OutT* Y = reinterpret_cast<OutT*>(args.Y);
  uint8_t* region = lds + wave * 32 * PITCH;
  const int row_w = m0 + wm * C::WTM;
  const int col_w = n0 + wn * C::WTN;
  const bool vec_ok = ((uintptr_t)Y % 16 == 0) && ((args.ldy * ES) % 16 == 0);   // 16 B row stores
  // fused: the bias of every row this lane stages, loaded once (16 rows per slice)
  float bz[FUSED ? TM : 1][16];
  if constexpr (FUSED) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row_w + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        bz[i][e] = args.bias ? args.bias[row < M ? row : M - 1] : 0.0f;
      }
  }
  // The staged slice is written as StageT and read back as 16 B words: the
  // compiler barriers keep those differently typed accesses in program order
  // (the wave's LDS operations then execute in that order).
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (!FUSED && ES == 2) {
        // bf16 output: elements e and e + 1 are rows r and r + 1 of the lane's
        // column; one packed conversion (v_cvt_pk_bf16_f32, round to nearest
        // even) makes both, then each half goes to its row.
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int r = 8 * (e >> 2) + 4 * h + (e & 3);
          const uint32_t w = __builtin_bit_cast(
              uint32_t, __builtin_convertvector((f32x2){acc[i][j][e], acc[i][j][e + 1]}, bf16x2));
          uint8_t* p = region + r * PITCH + (32 * j + (lane & 31)) * 2;
          *reinterpret_cast<uint16_t*>(p) = (uint16_t)w;
          *reinterpret_cast<uint16_t*>(p + PITCH) = (uint16_t)(w >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 8 * (e >> 2) + 4 * h + (e & 3);
          StageT v;
          if constexpr (FUSED) v = acc[i][j][e] + bz[i][e];
          else v = acc[i][j][e];
          *reinterpret_cast<StageT*>(region + r * PITCH + (32 * j + (lane & 31)) * SES) = v;
        }
      }
    }
    asm volatile("" ::: "memory");
    if constexpr (FUSED) {
      // VO outputs per 16 B store, read as VO staged fp32 values (32 B for a
      // bf16 output, 16 B for fp32)
      constexpr int VO = 16 / ES;
      constexpr int PRO = C::WTN / VO;              // stores per row
      constexpr int PLO = 32 * PRO / 64;            // stores per lane per slice
      static_assert((32 * PRO) % 64 == 0, "whole stores per lane");
      // the GELU variant keeps this loop rolled: unrolling it measured no
      // faster and quadruples the code
#pragma unroll(EPI == 2 ? 1 : PLO)
      for (int t = 0; t < PLO; ++t) {
        const int q = t * 64 + lane;
        const int r = q / PRO, cc = (q % PRO) * VO;
        const int row = row_w + 32 * i + r, col = col_w + cc;
        float zf[VO];
#pragma unroll
        for (int w = 0; w < VO / 4; ++w) {
          const u32x4 piece = *reinterpret_cast<const u32x4*>(region + r * PITCH + (cc + 4 * w) * 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) zf[4 * w + u] = __uint_as_float(piece[u]);
        }
        if (row >= M) continue;
        OutT o[VO];
        float f[VO];
#pragma unroll
        for (int u = 0; u < VO; ++u) {
          const float z = zf[u];
          f[u] = EPI == 2 ? apply_act(z, P24_ACT_GELU) : (args.act == P24_ACT_RELU ? (z > 0.0f ? z : 0.0f) : z);
        }
#pragma unroll
        for (int u = 0; u < VO; u += 2) {
          if constexpr (ES == 2) {
            // packed conversion, round to nearest even (v_cvt_pk_bf16_f32)
            const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[u], f[u + 1]}, bf16x2));
            o[u] = (uint16_t)w;
            o[u + 1] = (uint16_t)(w >> 16);
          } else {
            o[u] = f[u];
            o[u + 1] = f[u + 1];
          }
        }
        OutT* dst = Y + (int64_t)row * args.ldy + col;
        if (vec_ok && col + VO <= N) {
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), reinterpret_cast<u32x4*>(dst));
        } else {
#pragma unroll
          for (int u = 0; u < VO; ++u)
            if (col + u < N) dst[u] = o[u];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < PPL; ++t) {
        const int q = t * 64 + lane;
        const int r = q / PPR, cc = (q % PPR) * VEC;
        const u32x4 piece = *reinterpret_cast<const u32x4*>(region + r * PITCH + cc * SES);
        const int row = row_w + 32 * i + r, col = col_w + cc;
        if (row >= M) continue;
        OutT* dst = Y + (int64_t)row * args.ldy + col;
        if (vec_ok && col + VEC <= N) {
          __builtin_nontemporal_store(piece, reinterpret_cast<u32x4*>(dst));
        } else {
          const OutT* pv = reinterpret_cast<const OutT*>(&piece);
#pragma unroll
          for (int u = 0; u < VEC; ++u)
            if (col + u < N) dst[u] = pv[u];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side tile configuration and dispatch
// ---------------------------------------------------------------------------
enum class Tile { T256x256, T192x256, T128x256, T128x128, T64x128 };

template <int BM, int BN, int WGM, int WGN, int AM, int XM, int EPI = 0>
static p24_status launch_cfg(GemmArgs a, int32_t y_dtype, hipStream_t st) {
  a.nbm = (a.M + BM - 1) / BM;
  a.nbn = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(a.nbm * a.nbn)), block(WGM * WGN * 64);
  if (y_dtype == P24_F32)
    hipLaunchKernelGGL((k_gemm<BM, BN, WGM, WGN, AM, XM, float, EPI>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, WGM, WGN, AM, XM, uint16_t, EPI>), grid, block, 0, st, a);
  return launch_status();
}

static int64_t nblocks_for(Tile t, int64_t M, int64_t N) {
  int bm = 256, bn = 256;
  switch (t) {
    case Tile::T256x256: bm = 256; bn = 256; break;
    case Tile::T192x256: bm = 192; bn = 256; break;
    case Tile::T128x256: bm = 128; bn = 256; break;
    case Tile::T128x128: bm = 128; bn = 128; break;
    case Tile::T64x128: bm = 64; bn = 128; break;
  }
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// The first of 256x256, 128x256, 128x128 and 64x128 that still gives at
// least 160 blocks (five eighths of the CUs), else the one with the most
// blocks.  The big tiles move the fewest bytes per MFMA, so they win even with
// a quarter of the CUs idle; below that the smaller tiles, which also fit two
// blocks per CU, win on parallelism.  Measured: 256x256 on the 8192^3 and
// BERT FFN shapes, 128x256 on one GPU's share of 8192^3 split 8 ways (256
// blocks; 7 % over 128x128), 128x128 and 64x128 on the ResNet-50 shapes.
// When 256x256 leaves part of a single round of CUs idle and 192x256 fills
// more of that round (the BERT FFN shape: 192 blocks become 256), the
// sparse products take 192x256.
// P24_TILE=<256x256|192x256|128x256|128x128|64x128> overrides (measurement aid).
static Tile choose_tile(int64_t M, int64_t N, bool tall_ok) {
  if (const char* e = getenv("P24_TILE")) {
    const std::string s(e);
    if (s == "256x256") return Tile::T256x256;
    if (s == "192x256" && tall_ok) return Tile::T192x256;
    if (s == "128x256") return Tile::T128x256;
    if (s == "128x128") return Tile::T128x128;
    if (s == "64x128") return Tile::T64x128;
  }
  constexpr int64_t CUS = 256;
  const Tile order[] = {Tile::T256x256, Tile::T128x256, Tile::T128x128, Tile::T64x128};
  for (Tile t : order)
    if (nblocks_for(t, M, N) >= 160) {
      const int64_t n256 = nblocks_for(Tile::T256x256, M, N), n192 = nblocks_for(Tile::T192x256, M, N);
      if (t == Tile::T256x256 && tall_ok && n256 < CUS && n192 <= CUS && n192 > n256) return Tile::T192x256;
      return t;
    }
  return Tile::T64x128;
}

template <int AM, int XM, int EPI = 0>
static p24_status dispatch(const GemmArgs& a, int32_t y_dtype, hipStream_t st) {
  switch (choose_tile(a.M, a.N, AM == A_SPARSE)) {
    // The 256 x 256 tile runs 8 waves (2 x 4, each 128 x 64), two per SIMD:
    // while one wave waits on LDS reads or the stage barrier the other issues
    // MFMAs.  The 128 x 256 smfmac tile does the same with 64 x 64 per wave,
    // the 192 x 256 one with 96 x 64.
    case Tile::T256x256: return launch_cfg<256, 256, 2, 4, AM, XM, EPI>(a, y_dtype, st);
    case Tile::T192x256:
      if constexpr (AM == A_SPARSE) return launch_cfg<192, 256, 2, 4, AM, XM, EPI>(a, y_dtype, st);
      else return launch_cfg<256, 256, 2, 4, AM, XM, EPI>(a, y_dtype, st);
    case Tile::T128x256:
      if constexpr (AM == A_SPARSE) return launch_cfg<128, 256, 2, 4, AM, XM, EPI>(a, y_dtype, st);
      else return launch_cfg<128, 256, 2, 2, AM, XM, EPI>(a, y_dtype, st);
    // The smaller tiles take as many waves as their shape allows (2 x 4 of
    // 64 x 32, and 2 x 2 of 32 x 64): the skinny shapes that use them are
    // latency-bound, and the extra waves hide LDS and load waits (measured
    // 9-20 % faster on the ResNet-50 1x1 and 3x3 shapes, sparse and dense).
    // The expanded-tile path keeps its 4 and 2 waves (its expansion splits row
    // blocks over waves).
    case Tile::T128x128:
      if constexpr (AM != A_DECOMP) return launch_cfg<128, 128, 2, 4, AM, XM, EPI>(a, y_dtype, st);
      else return launch_cfg<128, 128, 2, 2, AM, XM, EPI>(a, y_dtype, st);
    case Tile::T64x128:
      if constexpr (AM != A_DECOMP) return launch_cfg<64, 128, 2, 2, AM, XM, EPI>(a, y_dtype, st);
      else return launch_cfg<64, 128, 1, 2, AM, XM, EPI>(a, y_dtype, st);
  }
  return P24_ERR_UNSUPPORTED;
}

static p24_status check_xy(const void* X, int64_t ldx, int64_t N, const void* Y, int32_t y_dtype,
                           int64_t ldy) {
  if (y_dtype != P24_F32 && y_dtype != P24_BF16) return P24_ERR_DTYPE;
  if (N < 0 || ldx < N || ldy < N || N > INT32_MAX) return P24_ERR_SHAPE;
  if (N > 0 && (uint64_t)ldx * 2 * 64 >= (1ull << 32)) return P24_ERR_UNSUPPORTED;   // one K step's rows in a 32-bit range
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
  if (algo != P24_ALGO_AUTO && algo != P24_ALGO_SMFMAC && algo != P24_ALGO_DECOMP_MFMA) return P24_ERR_UNSUPPORTED;
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
  // AUTO takes the sparse MFMA: on every measured shape it beats expanding the
  // operand for the dense MFMA, which issues twice the MFMA work.
  if (algo == P24_ALGO_DECOMP_MFMA) return dispatch<A_DECOMP, X_KN>(a, y_dtype, (hipStream_t)stream);
  return dispatch<A_SPARSE, X_KN>(a, y_dtype, (hipStream_t)stream);
}

// Gathered products (TVW on the sparse MFMA, TW alone on the dense MFMA): one
// block row = one 128-row slice of a tile, 8 waves; the fused variants add
// the bias + activation epilogue.
//
// Block width.  With one keep count for every tile the block is 128 x 512 when
// that grid still gives at least 160 blocks (five eighths of the CUs), else
// 128 x 256.  The wide block moves fewer X bytes per multiply-add and halves
// the number of blocks: on the 4096^3 TVW product (keep 2048) that is one
// round of 256 blocks instead of two rounds of 512, measured 10 % faster, in
// spite of holding only two 73 KiB stages.  Per-tile keep counts stay at
// 128 x 256: their heaviest-first order needs more blocks than CUs to even out
// the tiles (one round of 128 x 512 blocks measured 24 % slower).
// P24_GATHER_TILE=<128x256|128x512> overrides the width of the fixed-keep
// products (measurement and test aid).
static bool wide_gather(int64_t M, int64_t N) {
  if (const char* e = getenv("P24_GATHER_TILE")) {
    const std::string s(e);
    if (s == "128x512") return true;
    if (s == "128x256") return false;
  }
  return ((M + 127) / 128) * ((N + 511) / 512) >= 160;
}

// Wave layout: the sparse blocks take 1 x 8 waves of 128 x (BN / 8).  At 512
// wide that is the 8192^3 product's wave tile, with a fifth fewer LDS
// fragment bytes per MFMA than 2 x 4 waves of 64 x 128 (4096^3 TVW keep 2048:
// 46.1 -> 45.2 us); at 256 wide the bytes are equal but half of the B reads
// become A reads, which do not transpose (per-tile keep: 55.6 -> 54.4 us).
// The dense (TW) blocks take 1 x 8 at 512 wide (TW keep 2048 63.2 -> 62.5 us,
// keep 1024 37.8 -> 36.1 us) and keep 2 x 4 at 256 wide (per-tile keep TW
// measured 2-3 % slower with 1 x 8).
template <int AM, int XM, int BN>
static p24_status launch_gather_bn(const GemmArgs& a, int32_t y_dtype, bool fused, int32_t act, hipStream_t st) {
  constexpr int WM = AM == A_SPARSE || BN == 512 ? 1 : 2, WN = 8 / WM;
  if (!fused) return launch_cfg<128, BN, WM, WN, AM, XM, 0>(a, y_dtype, st);
  if (act == P24_ACT_GELU) return launch_cfg<128, BN, WM, WN, AM, XM, 2>(a, y_dtype, st);
  return launch_cfg<128, BN, WM, WN, AM, XM, 1>(a, y_dtype, st);
}

template <int AM, int XM>
static p24_status launch_gather(const GemmArgs& a, int32_t y_dtype, bool fused, int32_t act, hipStream_t st) {
  if constexpr (XM == X_KN_GATHER) {
    if (wide_gather(a.M, a.N)) return launch_gather_bn<AM, XM, 512>(a, y_dtype, fused, act, st);
  }
  return launch_gather_bn<AM, XM, 256>(a, y_dtype, fused, act, st);
}

template <int XM>
static p24_status launch_tvw(const GemmArgs& a, int32_t y_dtype, bool fused, int32_t act, hipStream_t st) {
  return launch_gather<A_SPARSE, XM>(a, y_dtype, fused, act, st);
}

static p24_status check_epilogue(const float* bias, int32_t act) {
  if (act != P24_ACT_NONE && act != P24_ACT_RELU && act != P24_ACT_GELU) return P24_ERR_UNSUPPORTED;
  if (bias && !aligned(bias, 4)) return P24_ERR_ALIGN;
  return P24_OK;
}

// dry_run: validate only (nothing is launched); the status is the one the call would return.
static p24_status tvw_fixed(const int32_t* kept, const void* values, const void* meta, int32_t layout, int64_t M,
                            int64_t K, int64_t tile_m, int64_t keep_k, const void* X, int64_t ldx, int64_t N,
                            void* Y, int32_t y_dtype, int64_t ldy, bool fused, const float* bias, int32_t act,
                            void* stream, bool dry_run = false) {
  if (layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K <= 0 || tile_m <= 0 || keep_k <= 0 || keep_k > K || M > INT32_MAX || K > INT32_MAX)
    return P24_ERR_SHAPE;
  if (tile_m % 128 || keep_k % 64) return P24_ERR_UNSUPPORTED;
  if (fused && (s = check_epilogue(bias, act)) != P24_OK) return s;
  if (M == 0 || N == 0) return P24_OK;
  if ((uint64_t)K * ldx * 2 >= (1ull << 32)) return P24_ERR_UNSUPPORTED;   // gathered rows: all of X in a 32-bit range
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
  a.bias = bias;
  a.act = act;
  if (dry_run) return P24_OK;
  return launch_tvw<X_KN_GATHER>(a, y_dtype, fused, act, (hipStream_t)stream);
}

static p24_status tvw_var(const int64_t* offsets, const int32_t* order, const int32_t* kept, const void* values,
                          const void* meta, int64_t M, int64_t K, const void* X, int64_t ldx, int64_t N, void* Y,
                          int32_t y_dtype, int64_t ldy, bool fused, const float* bias, int32_t act, void* stream) {
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K <= 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (fused && (s = check_epilogue(bias, act)) != P24_OK) return s;
  if (M == 0 || N == 0) return P24_OK;
  if ((uint64_t)K * ldx * 2 >= (1ull << 32)) return P24_ERR_UNSUPPORTED;   // gathered rows: all of X in a 32-bit range
  if (!offsets || !order || !kept || !values || !meta) return P24_ERR_NULL;
  if (!aligned(values, 16) || !aligned(meta, 16) || !aligned(kept, 4) || !aligned(offsets, 8) ||
      !aligned(order, 4))
    return P24_ERR_ALIGN;
  s = check_xy_ptrs(X, ldx, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)values;
  a.Ameta = (const uint32_t*)meta;
  a.kept = kept;
  a.offsets = offsets;
  a.order = order;
  a.X = (const uint16_t*)X;
  a.Y = Y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = 0;            // per tile, from the offsets
  a.Kx = (int)K;
  a.tile_m = 128;
  a.bias = bias;
  a.act = act;
  return launch_tvw<X_KN_GATHER_VAR>(a, y_dtype, fused, act, (hipStream_t)stream);
}

extern "C" P24_API p24_status spmm_tvw(const int32_t* kept, const void* values, const void* meta, int32_t layout,
                                       int64_t M, int64_t K, int64_t tile_m, int64_t keep_k, const void* X,
                                       int64_t ldx, int64_t N, void* Y, int32_t y_dtype, int64_t ldy,
                                       void* stream) {
  return tvw_fixed(kept, values, meta, layout, M, K, tile_m, keep_k, X, ldx, N, Y, y_dtype, ldy, false, nullptr,
                   P24_ACT_NONE, stream);
}

extern "C" P24_API p24_status spmm_tvw_fused(const int32_t* kept, const void* values, const void* meta,
                                             int32_t layout, int64_t M, int64_t K, int64_t tile_m, int64_t keep_k,
                                             const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                                             int64_t ldy, const float* bias, int32_t act, void* stream) {
  return tvw_fixed(kept, values, meta, layout, M, K, tile_m, keep_k, X, ldx, N, Y, y_dtype, ldy, true, bias, act,
                   stream);
}

extern "C" P24_API p24_status spmm_tvw_var(const int64_t* offsets, const int32_t* order, const int32_t* kept,
                                           const void* values, const void* meta, int64_t M, int64_t K,
                                           const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                                           int64_t ldy, void* stream) {
  return tvw_var(offsets, order, kept, values, meta, M, K, X, ldx, N, Y, y_dtype, ldy, false, nullptr,
                 P24_ACT_NONE, stream);
}

extern "C" P24_API p24_status spmm_tvw_var_fused(const int64_t* offsets, const int32_t* order,
                                                 const int32_t* kept, const void* values, const void* meta,
                                                 int64_t M, int64_t K, const void* X, int64_t ldx, int64_t N,
                                                 void* Y, int32_t y_dtype, int64_t ldy, const float* bias,
                                                 int32_t act, void* stream) {
  return tvw_var(offsets, order, kept, values, meta, M, K, X, ldx, N, Y, y_dtype, ldy, true, bias, act, stream);
}

// TW alone: the dense MFMA on each tile's packed kept columns, X rows gathered
// by the tile's kept list (block shapes as for TVW above).
template <int XM>
static p24_status launch_tw(const GemmArgs& a, int32_t y_dtype, bool fused, int32_t act, hipStream_t st) {
  return launch_gather<A_DENSE, XM>(a, y_dtype, fused, act, st);
}

static p24_status tw_fixed(const int32_t* kept, const void* Wp, int64_t M, int64_t K, int64_t tile_m,
                           int64_t keep_k, const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                           int64_t ldy, bool fused, const float* bias, int32_t act, void* stream) {
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K <= 0 || tile_m <= 0 || keep_k <= 0 || keep_k > K || M > INT32_MAX || K > INT32_MAX)
    return P24_ERR_SHAPE;
  if (tile_m % 128 || keep_k % 64) return P24_ERR_UNSUPPORTED;
  if (fused && (s = check_epilogue(bias, act)) != P24_OK) return s;
  if (M == 0 || N == 0) return P24_OK;
  if ((uint64_t)K * ldx * 2 >= (1ull << 32)) return P24_ERR_UNSUPPORTED;   // gathered rows: all of X in a 32-bit range
  if (!kept || !Wp) return P24_ERR_NULL;
  if (!aligned(Wp, 16) || !aligned(kept, 4)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(X, ldx, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)Wp;
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
  a.bias = bias;
  a.act = act;
  return launch_tw<X_KN_GATHER>(a, y_dtype, fused, act, (hipStream_t)stream);
}

static p24_status tw_var(const int64_t* offsets, const int32_t* order, const int32_t* kept, const void* Wp,
                         int64_t M, int64_t K, const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                         int64_t ldy, bool fused, const float* bias, int32_t act, void* stream) {
  p24_status s = check_xy(X, ldx, N, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (M < 0 || K <= 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (fused && (s = check_epilogue(bias, act)) != P24_OK) return s;
  if (M == 0 || N == 0) return P24_OK;
  if ((uint64_t)K * ldx * 2 >= (1ull << 32)) return P24_ERR_UNSUPPORTED;
  if (!offsets || !order || !kept || !Wp) return P24_ERR_NULL;
  if (!aligned(Wp, 16) || !aligned(kept, 4) || !aligned(offsets, 8) || !aligned(order, 4)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(X, ldx, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)Wp;
  a.kept = kept;
  a.offsets = offsets;
  a.order = order;
  a.X = (const uint16_t*)X;
  a.Y = Y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = 0;            // per tile, from the offsets
  a.Kx = (int)K;
  a.tile_m = 128;
  a.bias = bias;
  a.act = act;
  return launch_tw<X_KN_GATHER_VAR>(a, y_dtype, fused, act, (hipStream_t)stream);
}

extern "C" P24_API p24_status spmm_tw(const int32_t* kept, const void* Wp, int64_t M, int64_t K, int64_t tile_m,
                                      int64_t keep_k, const void* X, int64_t ldx, int64_t N, void* Y,
                                      int32_t y_dtype, int64_t ldy, void* stream) {
  return tw_fixed(kept, Wp, M, K, tile_m, keep_k, X, ldx, N, Y, y_dtype, ldy, false, nullptr, P24_ACT_NONE, stream);
}

extern "C" P24_API p24_status spmm_tw_fused(const int32_t* kept, const void* Wp, int64_t M, int64_t K,
                                            int64_t tile_m, int64_t keep_k, const void* X, int64_t ldx, int64_t N,
                                            void* Y, int32_t y_dtype, int64_t ldy, const float* bias, int32_t act,
                                            void* stream) {
  return tw_fixed(kept, Wp, M, K, tile_m, keep_k, X, ldx, N, Y, y_dtype, ldy, true, bias, act, stream);
}

extern "C" P24_API p24_status spmm_tw_var(const int64_t* offsets, const int32_t* order, const int32_t* kept,
                                          const void* Wp, int64_t M, int64_t K, const void* X, int64_t ldx,
                                          int64_t N, void* Y, int32_t y_dtype, int64_t ldy, void* stream) {
  return tw_var(offsets, order, kept, Wp, M, K, X, ldx, N, Y, y_dtype, ldy, false, nullptr, P24_ACT_NONE, stream);
}

extern "C" P24_API p24_status spmm_tw_var_fused(const int64_t* offsets, const int32_t* order, const int32_t* kept,
                                                const void* Wp, int64_t M, int64_t K, const void* X, int64_t ldx,
                                                int64_t N, void* Y, int32_t y_dtype, int64_t ldy, const float* bias,
                                                int32_t act, void* stream) {
  return tw_var(offsets, order, kept, Wp, M, K, X, ldx, N, Y, y_dtype, ldy, true, bias, act, stream);
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
  return dispatch<A_DENSE, X_KN>(a, y_dtype, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// X given as X^T (N x K row-major, K contiguous)
// ---------------------------------------------------------------------------
static p24_status check_xt(const void* XT, int64_t ldxt, int64_t N, int64_t K, const void* Y, int32_t y_dtype,
                           int64_t ldy) {
  if (y_dtype != P24_F32 && y_dtype != P24_BF16) return P24_ERR_DTYPE;
  if (N < 0 || ldxt < K || ldy < N || N > INT32_MAX) return P24_ERR_SHAPE;
  if (N > 0 && (uint64_t)ldxt * 2 * 256 >= (1ull << 32)) return P24_ERR_UNSUPPORTED;   // one tile's rows in a 32-bit range
  (void)XT;
  (void)Y;
  return P24_OK;
}

extern "C" P24_API p24_status spmm24_xt(const void* values, const void* meta, int32_t layout, int64_t M, int64_t K,
                                        const void* XT, int64_t ldxt, int64_t N, void* Y, int32_t y_dtype,
                                        int64_t ldy, void* stream) {
  if (layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (M < 0 || K < 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  p24_status s = check_xt(XT, ldxt, N, K, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return P24_OK;
  if (K == 0) return P24_ERR_UNSUPPORTED;
  if (!values || !meta) return P24_ERR_NULL;
  if (!aligned(values, 16) || !aligned(meta, 16)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(XT, ldxt, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)values;
  a.Ameta = (const uint32_t*)meta;
  a.X = (const uint16_t*)XT;
  a.Y = Y;
  a.ldx = ldxt;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = (int)K;
  a.Kx = (int)K;
  a.tile_m = 1;
  return dispatch<A_SPARSE, X_NK>(a, y_dtype, (hipStream_t)stream);
}

// Fused epilogue: Y = act(W X + b), b one fp32 per output row.  X as K x N
// (P24_X_KN, rules of spmm24) or as N x K (P24_X_NK, rules of spmm24_xt).
// dry_run: validate only (nothing is launched); the status is the one the call would return.
static p24_status fused24(const void* values, const void* meta, int32_t layout, int64_t M, int64_t K, const void* X,
                          int64_t ldx, int32_t x_order, int64_t N, void* Y, int32_t y_dtype, int64_t ldy,
                          const float* bias, int32_t act, void* stream, bool dry_run) {
  if (layout != P24_LAYOUT_DEVICE) return P24_ERR_LAYOUT;
  if (x_order != P24_X_KN && x_order != P24_X_NK) return P24_ERR_UNSUPPORTED;
  if (act != P24_ACT_NONE && act != P24_ACT_RELU && act != P24_ACT_GELU) return P24_ERR_UNSUPPORTED;
  if (M < 0 || K < 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  p24_status s = x_order == P24_X_KN ? check_xy(X, ldx, N, Y, y_dtype, ldy) : check_xt(X, ldx, N, K, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return P24_OK;
  if (K == 0) return P24_ERR_UNSUPPORTED;
  if (!values || !meta) return P24_ERR_NULL;
  if (!aligned(values, 16) || !aligned(meta, 16) || (bias && !aligned(bias, 4))) return P24_ERR_ALIGN;
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
  a.bias = bias;
  a.act = act;
  if (dry_run) return P24_OK;
  if (act == P24_ACT_GELU) {
    if (x_order == P24_X_NK) return dispatch<A_SPARSE, X_NK, 2>(a, y_dtype, (hipStream_t)stream);
    return dispatch<A_SPARSE, X_KN, 2>(a, y_dtype, (hipStream_t)stream);
  }
  if (x_order == P24_X_NK) return dispatch<A_SPARSE, X_NK, 1>(a, y_dtype, (hipStream_t)stream);
  return dispatch<A_SPARSE, X_KN, 1>(a, y_dtype, (hipStream_t)stream);
}

extern "C" P24_API p24_status spmm24_fused(const void* values, const void* meta, int32_t layout, int64_t M,
                                           int64_t K, const void* X, int64_t ldx, int32_t x_order, int64_t N,
                                           void* Y, int32_t y_dtype, int64_t ldy, const float* bias, int32_t act,
                                           void* stream) {
  return fused24(values, meta, layout, M, K, X, ldx, x_order, N, Y, y_dtype, ldy, bias, act, stream, false);
}

// Two-layer chain Y2 = act2(W2 act1(W1 X + b1) + b2), layer 1 plain 2:4, layer 2
// TVW.  Layer 1's epilogue applies its bias and activation, rounds to bf16 and
// writes H = act1(W1 X + b1) row-major (features x tokens): the layout whose
// whole rows layer 2's TVW gather loads, so H is written once and read once per
// gathering tile, with no pass in between (no separate bias, activation, cast
// or re-layout).  Both calls are validated before either is enqueued.
extern "C" P24_API p24_status spmm24_tvw_chain(const void* values1, const void* meta1, int64_t M1, int64_t K1,
                                               const float* bias1, int32_t act1, const int32_t* kept2,
                                               const void* values2, const void* meta2, int64_t M2, int64_t tile_m2,
                                               int64_t keep_k2, const void* X, int64_t ldx, int64_t N, void* H,
                                               int64_t ldh, void* Y2, int32_t y2_dtype, int64_t ldy2,
                                               const float* bias2, int32_t act2, void* stream) {
  p24_status s = fused24(values1, meta1, P24_LAYOUT_DEVICE, M1, K1, X, ldx, P24_X_KN, N, H, P24_BF16, ldh, bias1,
                         act1, stream, true);
  if (s != P24_OK) return s;
  const bool fused2 = bias2 != nullptr || act2 != P24_ACT_NONE;
  s = tvw_fixed(kept2, values2, meta2, P24_LAYOUT_DEVICE, M2, M1, tile_m2, keep_k2, H, ldh, N, Y2, y2_dtype, ldy2,
                fused2, bias2, act2, stream, true);
  if (s != P24_OK) return s;
  if (M1 == 0 || M2 == 0 || N == 0) return P24_OK;
  if (H == X || H == Y2) return P24_ERR_UNSUPPORTED;     // the intermediate must be its own buffer
  s = fused24(values1, meta1, P24_LAYOUT_DEVICE, M1, K1, X, ldx, P24_X_KN, N, H, P24_BF16, ldh, bias1, act1, stream,
              false);
  if (s != P24_OK) return s;
  return tvw_fixed(kept2, values2, meta2, P24_LAYOUT_DEVICE, M2, M1, tile_m2, keep_k2, H, ldh, N, Y2, y2_dtype, ldy2,
                   fused2, bias2, act2, stream, false);
}

extern "C" P24_API p24_status gemm_bf16_xt(const void* Wp, int64_t M, int64_t K, const void* XT, int64_t ldxt,
                                           int64_t N, void* Y, int32_t y_dtype, int64_t ldy, void* stream) {
  if (M < 0 || K < 0 || M > INT32_MAX || K > INT32_MAX) return P24_ERR_SHAPE;
  p24_status s = check_xt(XT, ldxt, N, K, Y, y_dtype, ldy);
  if (s != P24_OK) return s;
  if (K % 64) return P24_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return P24_OK;
  if (K == 0) return P24_ERR_UNSUPPORTED;
  if (!Wp) return P24_ERR_NULL;
  if (!aligned(Wp, 16)) return P24_ERR_ALIGN;
  s = check_xy_ptrs(XT, ldxt, Y, y_dtype);
  if (s != P24_OK) return s;
  GemmArgs a{};
  a.A = (const uint16_t*)Wp;
  a.X = (const uint16_t*)XT;
  a.Y = Y;
  a.ldx = ldxt;
  a.ldy = ldy;
  a.M = (int)M;
  a.N = (int)N;
  a.Kc = (int)K;
  a.Kx = (int)K;
  a.tile_m = 1;
  return dispatch<A_DENSE, X_NK>(a, y_dtype, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// bf16 transpose: dst (C x R) = src (R x C)^T, through a 64 x 64 LDS tile.
// ---------------------------------------------------------------------------
namespace p24 {
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src, int64_t R, int64_t Cc,
                                                       int64_t lds_src, uint16_t* __restrict__ dst, int64_t ldd) {
  __shared__ uint16_t tile[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;          // 32 x 8 threads, 2 columns each
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = ty + 8 * i;
    const int64_t gr = r0 + r, gc = c0 + 2 * tx;
    uint32_t v = 0;
    if (gr < R) {
      if (gc + 1 < Cc && ((gc & 1) == 0) && (lds_src % 2 == 0)) {
        v = *reinterpret_cast<const uint32_t*>(src + gr * lds_src + gc);
      } else {
        const uint32_t lo = gc < Cc ? src[gr * lds_src + gc] : 0;
        const uint32_t hi = gc + 1 < Cc ? src[gr * lds_src + gc + 1] : 0;
        v = lo | (hi << 16);
      }
    }
    tile[r][2 * tx] = (uint16_t)(v & 0xFFFFu);
    tile[r][2 * tx + 1] = (uint16_t)(v >> 16);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = ty + 8 * i;                                      // output row (source column)
    const int64_t gc = c0 + c, gr = r0 + 2 * tx;
    if (gc < Cc) {
      const uint32_t lo = tile[2 * tx][c], hi = tile[2 * tx + 1][c];
      if (gr + 1 < R && (gr & 1) == 0 && (ldd % 2 == 0)) {
        *reinterpret_cast<uint32_t*>(dst + gc * ldd + gr) = lo | (hi << 16);
      } else {
        if (gr < R) dst[gc * ldd + gr] = (uint16_t)lo;
        if (gr + 1 < R) dst[gc * ldd + gr + 1] = (uint16_t)hi;
      }
    }
  }
}
}  // namespace p24

extern "C" P24_API p24_status transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t ld_src, void* dst,
                                             int64_t ld_dst, void* stream) {
  if (rows < 0 || cols < 0 || ld_src < cols || ld_dst < rows) return P24_ERR_SHAPE;
  if (rows == 0 || cols == 0) return P24_OK;
  if (!src || !dst) return P24_ERR_NULL;
  if (!aligned(src, 4) || !aligned(dst, 4)) return P24_ERR_ALIGN;
  if ((cols + 63) / 64 > INT32_MAX || (rows + 63) / 64 > 65535) return P24_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, (hipStream_t)stream, (const uint16_t*)src, rows, cols,
                     ld_src, (uint16_t*)dst, ld_dst);
  return launch_status();
}
