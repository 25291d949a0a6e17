/*
 * prune24.h -- C ABI of libprune24.so: 2:4 structured-sparse GEMM and
 * tile-vector-wise (TVW) sparsity on AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 *   - 2:4 pattern: in every run of four consecutive weights along the
 *     reduction axis K, two are zero, so half the weights and half the math
 *     remain (NVIDIA A100 sparsity blog page, body text; "Accelerating Sparse
 *     Deep Neural Networks", Abstract).
 *   - Compressed representation: the kept values plus a small per-value
 *     position code (same blog page, Figure 1 -- its drawing is not on the
 *     page, so the bit layout below is this library's own).
 *   - TVW: per GEMM tile of output rows, whole K columns are dropped at the
 *     global-memory level and 2:4 is applied to the columns that remain
 *     ("Accelerating Sparse DNNs Based on Tiled GEMM", Abstract and Figure 3).
 *
 * Conventions (all entry points)
 *   - W is M x K (output features x input features), X is K x N (input
 *     features x tokens), Y = W X is M x N.  All matrices are row-major with a
 *     leading dimension (ld*) counted in elements.  2:4 groups run along K,
 *     aligned at k = 0.
 *   - Every pointer argument is a DEVICE pointer, except where stated.  The
 *     caller allocates and owns every buffer; the library allocates nothing and
 *     keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on that stream and never synchronises; the caller keeps
 *     the buffers alive until the stream has passed the work.
 *   - Arguments are validated first; on any error the status is returned and
 *     nothing is enqueued.  P24_ERR_HIP means a launch failed.  M == 0 or
 *     N == 0 is a valid no-op.
 *   - The library is stateless and thread-safe.
 *   - It links the HIP runtime by soname (libamdhip64.so.7) and uses the copy
 *     the process has already loaded.  A process holds one copy: when another
 *     component opens its own copy by path (PyTorch does), load that component
 *     first.
 *   - The products pick their block tile from the shape.  Two environment
 *     variables, read at each call, force a tile instead (measurement and
 *     test aids; results stay within the same bounds):
 *     P24_TILE=256x256|128x256|128x128|64x128 for spmm24, spmm24_xt, the
 *     fused product and gemm_bf16; P24_GATHER_TILE=128x256|128x512 for the
 *     fixed-keep gathered products (spmm_tvw, spmm_tw and their fused forms).
 *
 * Layouts of a compressed matrix (values are bf16, metadata uint32)
 *   P24_LAYOUT_CANONICAL
 *     values: M x K/2 row-major bf16; values[m][2g+j] is the j-th kept entry
 *       (in ascending position order) of group g = k/4.
 *     meta: M x ceil(K/32) row-major uint32; value s of row m (s = 0..K/2-1)
 *       stores its position inside its group (0..3) at bits [2s, 2s+2) of the
 *       row's little-endian bit stream.  Unused high bits are 0.
 *   P24_LAYOUT_DEVICE (operand order of the gfx950 sparse MFMA
 *     v_smfmac_f32_32x32x32_bf16; needs K % 64 == 0; Mp = M rounded up to 32)
 *     values: (Mp/32) x (K/32) blocks of 64 x 8 bf16 (1 KiB), block (rb, s)
 *       at element offset (rb*(K/32) + s)*512; lane L's 8 values are
 *       canonical values[32*rb + L%32][16*s + 8*(L/32) .. +8].
 *     meta: (Mp/32) x (K/64) blocks of 64 uint32, block (rb, t) at word offset
 *       (rb*(K/64) + t)*64; lane L's word holds, for row 32*rb + L%32, the
 *       positions of compressed columns 32*t + 8*(L/32) .. +8 in bits [0,16)
 *       and of 32*t + 16 + 8*(L/32) .. +8 in bits [16,32), 2 bits per value
 *       in value order.  Rows M..Mp-1 hold zero values and positions 0,1.
 *
 * Readings the pages leave open (magnitude criterion, tie order, rounding)
 *   - Selection keeps the two entries of each group with the largest
 *     magnitude key = the IEEE bit pattern with the sign cleared, read as an
 *     unsigned integer; ties go to the lower index (so -0 ties +0, NaN ranks
 *     above +Inf).
 *   - fp32 inputs are selected on their fp32 bits, then the kept values are
 *     rounded to bf16 to nearest-even (NaN -> 0x7FC0 with the input's sign).
 */
#ifndef PRUNE24_H
#define PRUNE24_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define P24_API __attribute__((visibility("default")))
#define PRUNE24_ABI_VERSION 1

typedef int32_t p24_status;

enum {
  P24_OK = 0,
  P24_ERR_NULL = -1,         /* a required pointer is NULL */
  P24_ERR_SHAPE = -2,        /* negative size, ld too small, K % 4 != 0, bad tile/keep */
  P24_ERR_ALIGN = -3,        /* pointer or leading dimension not aligned as required */
  P24_ERR_DTYPE = -4,        /* unknown dtype code */
  P24_ERR_UNSUPPORTED = -5,  /* valid request the library does not implement (e.g. K % 64) */
  P24_ERR_HIP = -6,          /* the HIP runtime reported an error at launch */
  P24_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than required */
  P24_ERR_LAYOUT = -8,       /* unknown layout code, or layout not accepted here */
  P24_ERR_SCRATCH = -9       /* larger than the fixed scratch of a no-allocation entry point */
};

enum { P24_F32 = 0, P24_BF16 = 1 };                         /* element dtypes */
enum { P24_LAYOUT_CANONICAL = 0, P24_LAYOUT_DEVICE = 1 };    /* compressed layouts */
enum { P24_ALGO_AUTO = 0, P24_ALGO_SMFMAC = 1, P24_ALGO_DECOMP_MFMA = 2 };   /* spmm24 algorithms */
enum { P24_X_KN = 0, P24_X_NK = 1 };                            /* spmm24_fused: X orientation */
enum { P24_ACT_NONE = 0, P24_ACT_RELU = 1, P24_ACT_GELU = 2 };  /* fused epilogues: activation */

/* ABI version of the loaded library (PRUNE24_ABI_VERSION). */
P24_API int32_t prune24_abi_version(void);

/* Human-readable text for a status code (static storage; never NULL). */
P24_API const char* prune24_strerror(p24_status s);

/* Bytes of the values / metadata buffers for an M x K matrix in `layout`
 * (0 for an invalid request).  Host-only helpers; they touch no device. */
P24_API size_t prune24_values_bytes(int64_t M, int64_t K, int32_t layout);
P24_API size_t prune24_meta_bytes(int64_t M, int64_t K, int32_t layout);

/*
 * prune24_compress -- magnitude 2:4 selection + compression of W.
 *   W        M x K, dtype w_dtype (P24_F32 or P24_BF16), leading dim ldw >= K.
 *            Alignment: W 16 B aligned and ldw % 4 == 0 (fp32); 8 B and
 *            ldw % 4 == 0 (bf16).
 *   values   output, prune24_values_bytes(M, K, layout) bytes, 16 B aligned.
 *   meta     output, prune24_meta_bytes(M, K, layout) bytes, 16 B aligned.
 *   layout   P24_LAYOUT_CANONICAL (K % 4 == 0) or P24_LAYOUT_DEVICE (K % 64 == 0).
 * Result is bit-exact and deterministic.
 */
P24_API p24_status prune24_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K,
                                    int64_t ldw, void* values, void* meta, int32_t layout,
                                    void* stream);

/*
 * prune24_decompress -- expand a compressed matrix back to dense bf16:
 *   W_out[m][k] = the kept value at k, +0 elsewhere.  W_out is M x K bf16 with
 *   leading dim ldo >= K, 2 B aligned.  Same layout rules as prune24_compress.
 */
P24_API p24_status prune24_decompress(const void* values, const void* meta, int32_t layout,
                                      int64_t M, int64_t K, void* W_out, int64_t ldo,
                                      void* stream);

/*
 * spmm24 -- Y = W X with W given compressed (2:4) and X dense bf16.
 *   values, meta  compressed W in P24_LAYOUT_DEVICE (the layout the sparse MFMA
 *                 reads directly; other layouts return P24_ERR_LAYOUT).
 *   M, K          logical shape of W; K % 64 == 0 (else P24_ERR_UNSUPPORTED).
 *   X             K x N bf16, leading dim ldx >= N, ldx % 8 == 0, 16 B aligned;
 *                 128 * ldx < 2^32 (one K step of rows is addressed with 32 bits),
 *                 else P24_ERR_UNSUPPORTED.
 *                 The kernel reads X in 16 B pieces: when N % 8 != 0 the last
 *                 row must stay readable up to column roundup(N, 8) - 1 (any
 *                 values there are ignored).
 *   Y             M x N, y_dtype P24_F32 or P24_BF16 (round to nearest even),
 *                 leading dim ldy >= N, naturally aligned.
 *   algo          P24_ALGO_SMFMAC: the sparse MFMA consumes the compressed
 *                 operand and its metadata directly (the 2:4 pattern the
 *                 matrix units exploit, "Accelerating Sparse Deep Neural
 *                 Networks", Abstract).
 *                 P24_ALGO_DECOMP_MFMA: each block expands the compressed
 *                 operand into a dense tile in LDS (zeros in the pruned slots)
 *                 and runs the dense MFMA on it: the same result up to fp32
 *                 summation order, twice the MFMA work.  Kept as the measured
 *                 alternative.
 *                 P24_ALGO_AUTO: P24_ALGO_SMFMAC.  Other codes return
 *                 P24_ERR_UNSUPPORTED.
 * Products are exact in fp32 and accumulate in fp32.  The result is
 * deterministic run to run (no atomics, fixed reduction order).  With finite X
 * both algorithms agree with the exact product of the pruned W within the same
 * bound; a non-finite X element meets the explicit zeros of
 * P24_ALGO_DECOMP_MFMA (0 * inf = NaN) but is skipped by P24_ALGO_SMFMAC.
 */
P24_API p24_status spmm24(const void* values, const void* meta, int32_t layout, int64_t M,
                          int64_t K, const void* X, int64_t ldx, int64_t N, void* Y,
                          int32_t y_dtype, int64_t ldy, int32_t algo, void* stream);

/*
 * spmm24_xt -- spmm24 with X supplied transposed.
 *   XT            N x K bf16 row-major (K contiguous: the layout of activations
 *                 stored tokens x features), leading dim ldxt >= K, ldxt % 8 == 0,
 *                 16 B aligned, 512 * ldxt < 2^32 (else P24_ERR_UNSUPPORTED).
 *                 Rows of XT at or past N are never read.
 * Everything else (layout, K % 64, Y, determinism) as for spmm24.  The MFMA
 * operands want K-contiguous fragments, so this form reads X with plain 16 B
 * LDS loads instead of transposing LDS loads; for the same inputs it returns
 * bit-identical results to spmm24.
 */
P24_API p24_status spmm24_xt(const void* values, const void* meta, int32_t layout, int64_t M,
                             int64_t K, const void* XT, int64_t ldxt, int64_t N, void* Y,
                             int32_t y_dtype, int64_t ldy, void* stream);

/*
 * spmm24_fused -- Y = act(W X + b) in one pass: the sparse-MFMA product with a
 * bias add and an activation applied to the fp32 accumulator before the
 * output rounding (kernel fusion, "Accelerating Sparse DNNs Based on Tiled
 * GEMM", TL;DR).
 *   x_order   P24_X_KN: X is K x N with the rules of spmm24 (ldx, alignment,
 *             readable tail); P24_X_NK: X is given as N x K with the rules of
 *             spmm24_xt (ldx is then its leading dimension, >= K).
 *   bias      M fp32 values, one per output row (added to every column), 4 B
 *             aligned; NULL adds nothing.
 *   act       P24_ACT_NONE; P24_ACT_RELU: z > 0 ? z : 0 (NaN -> 0);
 *             P24_ACT_GELU: z * Phi(z) = z/2 (1 + erf(z / sqrt 2)), evaluated
 *             in fp32 with erf from Abramowitz & Stegun 7.1.26 (absolute error
 *             <= 1.5e-7).  Other codes: P24_ERR_UNSUPPORTED.
 * Everything else (layout, K % 64, Y, determinism) as for spmm24.  With
 * bias == NULL and P24_ACT_NONE the result equals spmm24's (or spmm24_xt's)
 * bit for bit.
 */
P24_API p24_status spmm24_fused(const void* values, const void* meta, int32_t layout, int64_t M,
                                int64_t K, const void* X, int64_t ldx, int32_t x_order, int64_t N,
                                void* Y, int32_t y_dtype, int64_t ldy, const float* bias,
                                int32_t act, void* stream);

/*
 * Masked fine-tuning ("Accelerating Sparse Deep Neural Networks", Abstract:
 * prune the trained network to 2:4, then retrain it with that pattern).
 * prune24_refresh -- prune24_compress of W and, in the same pass, every
 *   dropped entry of W set to +0 in place (kept entries are left bit for
 *   bit), so W equals its pruned self afterwards.  Arguments and rules as for
 *   prune24_compress; W is read and written.  The re-prune a fine-tuning loop
 *   runs every few steps.
 * prune24_mask_apply -- W[m][k] := +0 for every k the stored metadata `meta`
 *   (in `layout`, as written for an M x K matrix) does not select; selected
 *   entries are left bit for bit.  W fp32 (16 B aligned) or bf16 (8 B
 *   aligned), ldw >= K, ldw % 4 == 0; meta 4 B aligned; K % 4 == 0 (% 64 for
 *   the device layout).  The per-step masking between re-prunes.
 */
P24_API p24_status prune24_refresh(void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                   void* values, void* meta, int32_t layout, void* stream);
P24_API p24_status prune24_mask_apply(void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                      const void* meta, int32_t layout, void* stream);

/*
 * transpose_bf16 -- dst = src^T for 16-bit elements (a bit copy).
 *   src   rows x cols, leading dim ld_src >= cols;  dst  cols x rows, ld_dst >= rows.
 *   Both 4 B aligned; rows <= 65535 * 64.  Turns X (K x N) into XT for spmm24_xt.
 */
P24_API p24_status transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                                  void* dst, int64_t ld_dst, void* stream);

/*
 * tvw_compress -- TVW selection and compression of fp32 W.
 *   Tile t covers output rows [t*tile_m, min(M, (t+1)*tile_m)).  Its column
 *   score is the fp64 sum over those rows, in ascending row order, of |W[m][k]|;
 *   the keep_k columns with the largest score (ties -> lower k; a NaN score
 *   ranks above +Inf and NaN scores tie, whatever their payload) are kept, listed ascending
 *   in kept[t][0..keep_k).  The tile's rows restricted to those columns are then
 *   compressed 2:4 exactly as prune24_compress does, along the compacted axis.
 *   W         M x K fp32 (w_dtype must be P24_F32), ldw % 4 == 0, 16 B aligned;
 *             M, K <= 2^31 - 1.
 *   tile_m    > 0 and a multiple of 32.  keep_k: 0 < keep_k <= K, keep_k % 4 == 0
 *             (% 64 for the device layout).
 *   kept      output int32 [ceil(M/tile_m)][keep_k].
 *   values, meta   output, sized as for an M x keep_k matrix in `layout`.
 *   workspace device scratch of at least tvw_workspace_bytes(...) bytes,
 *             8 B aligned; its contents on entry do not matter.
 */
P24_API size_t tvw_workspace_bytes(int64_t M, int64_t K, int64_t tile_m, int64_t keep_k);
P24_API p24_status tvw_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K,
                                int64_t ldw, int64_t tile_m, int64_t keep_k, int32_t* kept,
                                void* values, void* meta, int32_t layout, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * tvw_compress_noalloc -- tvw_compress for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc): no workspace argument, and the call allocates and frees
 *   nothing.  The column scores go to a fixed scratch array in device memory
 *   that the library holds on every GPU it runs on until the process ends,
 *   tvw_noalloc_scratch_bytes() bytes (8 MiB) per GPU.
 *   Same arguments, outputs and errors as tvw_compress without workspace and
 *   ws_bytes, plus:
 *     P24_ERR_SCRATCH      tvw_workspace_bytes(M, K, tile_m, keep_k) exceeds
 *                          the scratch (nothing is enqueued);
 *     P24_ERR_UNSUPPORTED  `stream` belongs to another device than the current
 *                          one (the current device's scratch is used);
 *     P24_ERR_HIP          the scratch address could not be looked up.
 *   The first call on a device looks up that device's scratch address
 *   (thread-safe); later calls reuse it.  Every call on one GPU shares that
 *   GPU's scratch: calls that overlap on one GPU (two streams, two host
 *   threads) race and give undefined results; calls in one stream are
 *   ordered and safe.  Nothing in the scratch needs to start at zero.
 */
P24_API size_t tvw_noalloc_scratch_bytes(void);
P24_API p24_status tvw_compress_noalloc(const void* W, int32_t w_dtype, int64_t M, int64_t K,
                                        int64_t ldw, int64_t tile_m, int64_t keep_k, int32_t* kept,
                                        void* values, void* meta, int32_t layout, void* stream);

/*
 * spmm_tvw -- Y = W X for a TVW-compressed W: for output rows of tile t,
 *   Y[m][n] = sum_j Wc[m][j] * X[kept[t][j]][n], with Wc the 2:4-compressed
 *   M x keep_k matrix (P24_LAYOUT_DEVICE).  X rows are gathered by `kept`
 *   (whole, contiguous N-slices).  Needs tile_m % 128 == 0 and keep_k % 64 == 0.
 *   kept entries must lie in [0, K); the kernel clamps out-of-range entries
 *   into that range (the result is then meaningless but no access leaves X).
 *   Gathered rows are addressed with 32 bits from X: 2 * K * ldx < 2^32, else
 *   P24_ERR_UNSUPPORTED.  Other arguments as for spmm24.
 */
P24_API p24_status spmm_tvw(const int32_t* kept, const void* values, const void* meta,
                            int32_t layout, int64_t M, int64_t K, int64_t tile_m,
                            int64_t keep_k, const void* X, int64_t ldx, int64_t N, void* Y,
                            int32_t y_dtype, int64_t ldy, void* stream);

/*
 * spmm_tvw_fused -- spmm_tvw with the epilogue of spmm24_fused:
 *   Y = act(W X + bias), bias fp32 [M] (one value per output row, nullptr for
 *   none, 4 B aligned), act P24_ACT_NONE / _RELU / _GELU (else
 *   P24_ERR_UNSUPPORTED); other arguments and rules as for spmm_tvw.
 */
P24_API p24_status spmm_tvw_fused(const int32_t* kept, const void* values, const void* meta,
                                  int32_t layout, int64_t M, int64_t K, int64_t tile_m,
                                  int64_t keep_k, const void* X, int64_t ldx, int64_t N, void* Y,
                                  int32_t y_dtype, int64_t ldy, const float* bias, int32_t act,
                                  void* stream);

/*
 * spmm24_tvw_chain -- two layers, the second TVW ("Accelerating Sparse DNNs Based on
 *   Tiled GEMM", TL;DR: kernel fusion):
 *     H  = bf16(act1(W1 X + bias1))          W1: M1 x K1, 2:4 (P24_LAYOUT_DEVICE)
 *     Y2 = act2(W2 H + bias2)                W2: M2 x M1, TVW (kept2, tile_m2, keep_k2)
 *   Layer 1's epilogue applies bias1 and act1, rounds to bf16 and writes H
 *   row-major (M1 features x N tokens, leading dim ldh): the layout whose whole
 *   rows layer 2 gathers by kept2, so no pass runs between the two products.
 *   H is a caller-owned device buffer of M1 x N bf16 (ldh >= N, ldh % 8 == 0,
 *   16 B aligned), distinct from X and Y2; on return it holds layer 1's output.
 *   X (K1 x N bf16), bias1 / act1 as for spmm24_fused; kept2, values2, meta2,
 *   tile_m2, keep_k2 as for spmm_tvw with K = M1; Y2, y2_dtype, ldy2, bias2 /
 *   act2 as for spmm_tvw_fused (bias2 NULL and act2 P24_ACT_NONE: no epilogue).
 *   Both products are validated before either is enqueued (any error of
 *   spmm24_fused or spmm_tvw_fused; P24_ERR_SHAPE for M1 == 0;
 *   P24_ERR_UNSUPPORTED if H is X or Y2).  M2 == 0 or N == 0: no-op.
 */
P24_API p24_status spmm24_tvw_chain(const void* values1, const void* meta1, int64_t M1, int64_t K1,
                                    const float* bias1, int32_t act1, const int32_t* kept2,
                                    const void* values2, const void* meta2, int64_t M2,
                                    int64_t tile_m2, int64_t keep_k2, const void* X, int64_t ldx,
                                    int64_t N, void* H, int64_t ldh, void* Y2, int32_t y2_dtype,
                                    int64_t ldy2, const float* bias2, int32_t act2, void* stream);

/*
 * TVW with a keep count per tile ("Accelerating Sparse DNNs Based on Tiled
 * GEMM", Abstract: regular structure inside a tile, irregular pruning across
 * the matrix; TL;DR: load balancing through batching).  Tiles are 128 rows:
 * T = ceil(M/128).
 * tvw_var_compress -- scores as for tvw_compress (tile_m = 128).  All T*K
 *   (tile, column) scores are ranked (score descending, then t*K + k
 *   ascending) and the top total_keep taken; tile t keeps c_t columns, its
 *   number of those rounded to the nearest multiple of 64 (halves up) and
 *   clamped to [64, K].  Tile t's c_t highest-scored columns (ties -> lower k),
 *   ascending, are compressed 2:4 along the compacted axis.
 *   W            M x K fp32 (P24_F32), ldw % 4 == 0, 16 B aligned; K % 64 == 0;
 *                M, K <= 2^31 - 1 and T*K <= 2^31 - 1.  0 < total_keep <= T*K.
 *   offsets      output int64 [T + 1], 8 B aligned: offsets[t] = c_0 + ... + c_{t-1};
 *                offsets[T] is the total of kept columns (at most T*K).
 *   order        output int32 [T]: the tiles by c_t descending, then tile
 *                ascending (the GEMM's block-row order: heavy tiles first).
 *   kept         output int32, capacity T*K: tile t's columns at
 *                [offsets[t], offsets[t+1]).
 *   values       output, capacity T*K*128 bytes, 16 B aligned: tile t's 128 x c_t
 *                compressed rows in P24_LAYOUT_DEVICE from byte 128*offsets[t].
 *   meta         output, capacity T*K*16 bytes, 16 B aligned: the tile's device
 *                metadata from byte 16*offsets[t].  Rows past M are padding
 *                (zero values, positions 0 and 1).
 *   workspace    device scratch, tvw_var_workspace_bytes(M, K) bytes, 256 B
 *                aligned; contents on entry do not matter.
 * spmm_tvw_var -- Y = W X for that storage: rows of tile t take
 *   sum_j Wc_t[m][j] X[kept[offsets[t] + j]][n].  Block rows run in `order`.
 *   offsets / order / kept as written by tvw_var_compress (out-of-range kept
 *   entries are clamped into [0, K)); X, Y as for spmm_tvw (2 * K * ldx < 2^32).
 *   offsets and order are device data the call cannot check without a
 *   synchronization: offsets must be non-decreasing multiples of 64 with steps
 *   of at most K, and order a permutation of 0 .. T-1; anything else is
 *   undefined behaviour (the kernels address W through them).
 */
P24_API size_t tvw_var_workspace_bytes(int64_t M, int64_t K);
P24_API p24_status tvw_var_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                    int64_t total_keep, int64_t* offsets, int32_t* order, int32_t* kept,
                                    void* values, void* meta, void* workspace, size_t ws_bytes,
                                    void* stream);
P24_API p24_status spmm_tvw_var(const int64_t* offsets, const int32_t* order, const int32_t* kept,
                                const void* values, const void* meta, int64_t M, int64_t K,
                                const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                                int64_t ldy, void* stream);
/* spmm_tvw_var_fused -- spmm_tvw_var with bias + activation, as spmm_tvw_fused. */
P24_API p24_status spmm_tvw_var_fused(const int64_t* offsets, const int32_t* order,
                                      const int32_t* kept, const void* values, const void* meta,
                                      int64_t M, int64_t K, const void* X, int64_t ldx, int64_t N,
                                      void* Y, int32_t y_dtype, int64_t ldy, const float* bias,
                                      int32_t act, void* stream);

/*
 * TW alone -- the tile column drop without the 2:4 step ("Accelerating Sparse
 * DNNs Based on Tiled GEMM", Abstract, Figure 3); the kept columns are
 * multiplied with the dense MFMA.
 * tw_compress -- the kept lists exactly as tvw_compress chooses them
 *   (tile_m % 32 == 0, keep_k % 64 == 0, W fp32 as there, workspace
 *   tvw_workspace_bytes(...)), and Wp: the M x keep_k matrix of tile rows on
 *   their kept columns, bf16 (round to nearest even), in the dense operand
 *   order of gemm_bf16_pack (gemm_bf16_packed_bytes(M, keep_k) bytes, 16 B aligned).
 * spmm_tw -- Y = W X with Y[m][n] = sum_j Wc[m][j] X[kept[t][j]][n];
 *   tile_m % 128 == 0; other rules of spmm_tvw.
 * tw_var_compress -- per-tile keep counts, offsets, order and kept lists
 *   exactly as tvw_var_compress; Wp (capacity T*K*256 bytes, 16 B aligned)
 *   holds tile t's 128 x c_t dense operand (rows past M zero) from element
 *   128*offsets[t].  Workspace tvw_var_workspace_bytes(M, K).
 * spmm_tw_var -- Y = W X for that storage; block rows run in `order`
 *   (same requirements on offsets and order as spmm_tvw_var).
 */
P24_API p24_status tw_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                               int64_t tile_m, int64_t keep_k, int32_t* kept, void* Wp, void* workspace,
                               size_t ws_bytes, void* stream);
P24_API p24_status spmm_tw(const int32_t* kept, const void* Wp, int64_t M, int64_t K, int64_t tile_m,
                           int64_t keep_k, const void* X, int64_t ldx, int64_t N, void* Y,
                           int32_t y_dtype, int64_t ldy, void* stream);
P24_API p24_status tw_var_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                                   int64_t total_keep, int64_t* offsets, int32_t* order, int32_t* kept,
                                   void* Wp, void* workspace, size_t ws_bytes, void* stream);
P24_API p24_status spmm_tw_var(const int64_t* offsets, const int32_t* order, const int32_t* kept,
                               const void* Wp, int64_t M, int64_t K, const void* X, int64_t ldx,
                               int64_t N, void* Y, int32_t y_dtype, int64_t ldy, void* stream);

/*
 * spmm_tw_fused / spmm_tw_var_fused -- spmm_tw / spmm_tw_var with the epilogue
 *   of spmm24_fused: Y = act(W X + bias), bias fp32 [M] (one value per output
 *   row, nullptr for none, 4 B aligned), act P24_ACT_NONE / _RELU / _GELU
 *   (else P24_ERR_UNSUPPORTED); other arguments and rules as for the plain
 *   calls (kernel fusion, "Accelerating Sparse DNNs Based on Tiled GEMM",
 *   TL;DR).
 */
P24_API p24_status spmm_tw_fused(const int32_t* kept, const void* Wp, int64_t M, int64_t K, int64_t tile_m,
                                 int64_t keep_k, const void* X, int64_t ldx, int64_t N, void* Y,
                                 int32_t y_dtype, int64_t ldy, const float* bias, int32_t act,
                                 void* stream);
P24_API p24_status spmm_tw_var_fused(const int64_t* offsets, const int32_t* order, const int32_t* kept,
                                     const void* Wp, int64_t M, int64_t K, const void* X, int64_t ldx,
                                     int64_t N, void* Y, int32_t y_dtype, int64_t ldy, const float* bias,
                                     int32_t act, void* stream);

/*
 * Comparison patterns ("Accelerating Sparse DNNs Based on Tiled GEMM",
 * Abstract: TVW against block and unstructured sparsity; Figure 5 names the
 * element-wise and block-wise patterns).
 * bw_compress -- block-wise: blocks of 128 rows (T = ceil(M/128) tiles) x 64
 *   columns.  A block's score is the fp64 sum, in ascending column order, of
 *   the tile column scores of tvw_compress (tile_m = 128); each tile keeps its
 *   keep_blocks highest-scored blocks (ties -> lower block).  kept: int32
 *   [T][keep_blocks*64], the kept blocks' columns ascending; Wp as for
 *   tw_compress with keep_k = keep_blocks*64 (gemm_bf16_packed_bytes(M,
 *   keep_k) bytes).  W fp32 as for tvw_compress, K % 64 == 0,
 *   0 < keep_blocks <= K/64; workspace bw_workspace_bytes(M, K), 8 B aligned.
 *   The product is spmm_tw(kept, Wp, M, K, 128, keep_blocks*64, ...).
 * ew_compress -- unstructured: every weight ranked by magnitude (the fp32
 *   bit pattern with the sign cleared) over the whole matrix, ties -> lower
 *   m*K + k; the top keep_total (0 < keep_total <= M*K <= 2^32 - 1) are kept
 *   in CSR form: row_ptr int64 [M+1] (8 B aligned), cols int32 [keep_total]
 *   ascending within a row, vals bf16 [keep_total] (round to nearest even).
 *   W fp32, 4 B aligned, ldw >= K; workspace ew_workspace_bytes(M, K), 256 B
 *   aligned.
 * spmm_ew -- Y = W X for that CSR form on the fp32 vector ALUs (row m:
 *   sum over its entries in column order).  X bf16 K x N, 16 B aligned,
 *   ldx >= N, ldx % 8 == 0; Y as for spmm24.  row_ptr must be non-decreasing
 *   from 0 (device data, not checked; the kernel reads cols and vals through
 *   it); columns must ascend within a row and lie in [0, K) -- others add
 *   unspecified terms but no access leaves X or the kernel's LDS tile.
 */
P24_API size_t bw_workspace_bytes(int64_t M, int64_t K);
P24_API p24_status bw_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                               int64_t keep_blocks, int32_t* kept, void* Wp, void* workspace,
                               size_t ws_bytes, void* stream);
P24_API size_t ew_workspace_bytes(int64_t M, int64_t K);
P24_API p24_status ew_compress(const void* W, int32_t w_dtype, int64_t M, int64_t K, int64_t ldw,
                               int64_t keep_total, int64_t* row_ptr, int32_t* cols, void* vals,
                               void* workspace, size_t ws_bytes, void* stream);
P24_API p24_status spmm_ew(const int64_t* row_ptr, const int32_t* cols, const void* vals, int64_t M,
                           int64_t K, const void* X, int64_t ldx, int64_t N, void* Y, int32_t y_dtype,
                           int64_t ldy, void* stream);

/*
 * Dense bf16 GEMM, the denominator of every speedup (the pages measure their
 * speedups against the dense model: "Accelerating Sparse DNNs Based on Tiled
 * GEMM", Abstract).  It runs the same
 * tile loop as spmm24 with the dense MFMA v_mfma_f32_32x32x16_bf16.
 *   gemm_bf16_pack: W (M x K bf16, ldw >= K, ldw % 8 == 0, 16 B aligned) ->
 *     Wp in MFMA operand order: (Mp/32) x (K/16) blocks of 64 x 8 bf16, block
 *     (rb, s) at element offset (rb*(K/16) + s)*512, lane L's 8 values are
 *     W[32*rb + L%32][16*s + 8*(L/32) .. +8]; rows >= M are zero.  K % 64 == 0.
 *   gemm_bf16: Y = W X from the packed Wp; X, Y as for spmm24.
 */
P24_API size_t gemm_bf16_packed_bytes(int64_t M, int64_t K);
P24_API p24_status gemm_bf16_pack(const void* W, int64_t M, int64_t K, int64_t ldw, void* Wp,
                                  void* stream);
P24_API p24_status gemm_bf16(const void* Wp, int64_t M, int64_t K, const void* X, int64_t ldx,
                             int64_t N, void* Y, int32_t y_dtype, int64_t ldy, void* stream);
/* gemm_bf16_xt -- the dense baseline with X supplied transposed (rules of spmm24_xt). */
P24_API p24_status gemm_bf16_xt(const void* Wp, int64_t M, int64_t K, const void* XT, int64_t ldxt,
                                int64_t N, void* Y, int32_t y_dtype, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PRUNE24_H */
