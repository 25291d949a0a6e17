"""CPU oracle for 2:4 structured-sparse GEMM, tile-wise (TW) and tile-vector-wise
(TVW) sparsity, masked fine-tuning and the block-wise / unstructured comparisons.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It is plain, slow, numpy-only code
written from the definitions below; it shares no code, table or helper with the
HIP library, and it imports neither torch nor the package.

Sources (the method's definition):
  * "Accelerating Sparse Deep Neural Networks" (Mishra et al.), Abstract: a 2:4
    pattern keeps 50% of the weights and the sparse matrix unit does twice the
    dense math rate.
  * NVIDIA A100 sparsity blog page, body text and its
    (missing) Figure 1: in every run of four consecutive weights at least two
    are zero; the survivors are stored in a compressed form with a small amount
    of position metadata.
  * "Accelerating Sparse DNNs Based on Tiled GEMM", Abstract, TL;DR and
    Figure 3: tile-wise (TW) sparsity removes whole reduction-axis rows per GEMM
    tile in global memory, and TVW applies 2:4 on top of it inside the tile.

Readings where the pages are silent:
  * criterion: magnitude; order: key descending, index ascending (ties go to
    the lower index); key = IEEE bit pattern with the sign bit cleared, read as
    an unsigned integer (monotone in |w|, -0 == +0, NaN above +Inf).
  * groups of four run along K (the reduction axis), aligned at k = 0.
  * fp32 masters are pruned first, then the kept values are rounded to bf16
    with round-to-nearest-even (NaN -> quiet NaN 0x7FC0 with the input's sign).
  * canonical metadata: row-major bit stream per row, value s (s = 0..K/2-1)
    stores the 2-bit in-group position of that value at bits [2s, 2s+2);
    32-bit words, little endian, ceil(K/32) words per row, unused bits zero.
  * device metadata/value layout: the operand order of the gfx950 sparse MFMA
    32x32x32 bf16 instruction (defined in ``to_device_layout``).
  * TVW: tile t = output rows [t*tile_m, (t+1)*tile_m); column score = fp64
    sum of |W| over the tile's rows in ascending row order; keep the keep_k
    columns with the largest score (ties -> lower k), listed ascending; then
    2:4 along the compacted axis.  A computed score that is NaN ranks above
    +Inf, and NaN scores tie with each other (``score_key``): IEEE 754 leaves
    the payload of an arithmetic NaN open, so no order may depend on it.
  * GEMM tolerance: |y - y_ref| <= 1e-3 * (|W|.|X|)_ij on the fp32 result; a
    bf16 result also gets the half-ulp of its final rounding,
    2^-8 * (|y_ref| + 1e-3 * (|W|.|X|)).
  * fused epilogue: y = act(W X + b), b per output row, act none / ReLU / exact
    GELU (see ``fused_ref``).
  * per-tile keep counts: one global ranking of every (tile, column) score,
    a tile's share of the top total_keep rounded to a multiple of 64 and
    clamped to [64, K] (see ``tvw_var_counts``); TW alone keeps the same
    columns without the 2:4 step.
  * masked fine-tuning: unselected weights become +0, selected ones keep
    their bits (see ``mask_apply``).
  * block-wise: 128 x 64 blocks, a fixed count per tile; unstructured: one
    global magnitude cut, CSR (see ``bw_select``, ``ew_compress``).

Parity pins for every function here live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import numpy as np

BF16_QNAN = 0x7FC0
TOL_REL = 1e-3          # elementwise bound factor on (|W|.|X|)
BF16_HALF_ULP = 2.0 ** -8


# ----------------------------------------------------------------------------
# bf16 helpers (bf16 values are carried as uint16 bit patterns)
# ----------------------------------------------------------------------------
def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even.

    Written from the rounding definition: add half of the dropped range minus
    one plus the lowest kept bit, then drop the low 16 bits.  NaN maps to the
    quiet NaN 0x7FC0 carrying the input's sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    sign = ((u >> 31) & 1).astype(np.uint32) << 15
    r = np.where(nan, sign | BF16_QNAN, r)
    return r.astype(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# 2:4 magnitude selection (blog page body text; criterion and tie rule above)
# ----------------------------------------------------------------------------
def _as_bits(W: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(W, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if dtype == "bf16":
        return np.ascontiguousarray(W, dtype=np.uint16).astype(np.uint64)
    raise ValueError(f"unknown dtype {dtype!r}")


def magnitude_key(W: np.ndarray, dtype: str) -> np.ndarray:
    """Unsigned magnitude key: the bit pattern with the sign bit cleared."""
    bits = _as_bits(W, dtype)
    mask = 0x7FFFFFFF if dtype == "f32" else 0x7FFF
    return bits & mask


def select_24(W: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """Kept in-group positions, shape (M, K/4, 2), ascending within each group.

    Each group of four along K is ordered by (key descending, index ascending)
    with a stable sort, and the first two positions are kept.
    """
    W = np.asarray(W)
    if W.ndim != 2:
        raise ValueError("W must be 2-D (M x K)")
    M, K = W.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    key = magnitude_key(W, dtype).reshape(M, K // 4, 4).astype(np.int64)
    order = np.argsort(-key, axis=-1, kind="stable")
    kept = np.sort(order[..., :2], axis=-1)
    return kept.astype(np.int64)


def prune_24(W: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """Dense pruned copy: dropped entries become +0 (bit pattern 0), kept entries are unchanged."""
    W = np.asarray(W)
    M, K = W.shape
    kept = select_24(W, dtype)
    mask = np.zeros((M, K // 4, 4), dtype=bool)
    np.put_along_axis(mask, kept, True, axis=-1)
    mask = mask.reshape(M, K)
    if dtype == "f32":
        out = np.where(mask, np.asarray(W, dtype=np.float32), np.float32(0.0))
        return out.astype(np.float32)
    return np.where(mask, np.asarray(W, dtype=np.uint16), np.uint16(0)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Compressed representation (blog page, Figure 1 reference; layout reading above)
# ----------------------------------------------------------------------------
def meta_words_per_row(K: int) -> int:
    return (K + 31) // 32


def compress_24(W: np.ndarray, dtype: str = "f32"):
    """Returns (values uint16 [M, K/2] bf16 bits, meta uint32 [M, ceil(K/32)]).

    values[m, 2g+j] = bf16(W[m, 4g + pos_j]) with pos_0 < pos_1 the kept
    positions of group g; meta holds pos of value s at bits [2s, 2s+2) of row
    m's bit stream.
    """
    W = np.asarray(W)
    M, K = W.shape
    kept = select_24(W, dtype)                      # (M, G, 2)
    G = K // 4
    grp = W.reshape(M, G, 4)
    vals = np.take_along_axis(grp, kept, axis=-1).reshape(M, K // 2)
    if dtype == "f32":
        values = bf16_rne(vals.astype(np.float32))
    else:
        values = vals.astype(np.uint16)
    pos = kept.reshape(M, K // 2).astype(np.uint64)  # position of value s
    nw = meta_words_per_row(K)
    meta = np.zeros((M, nw), dtype=np.uint64)
    for s in range(K // 2):
        bit = 2 * s
        meta[:, bit // 32] |= pos[:, s] << np.uint64(bit % 32)
    return values.astype(np.uint16), meta.astype(np.uint32)


def meta_positions(meta: np.ndarray, K: int) -> np.ndarray:
    """Decode canonical metadata into in-group positions, shape (M, K/2)."""
    meta = np.asarray(meta, dtype=np.uint32).astype(np.uint64)
    M = meta.shape[0]
    pos = np.zeros((M, K // 2), dtype=np.int64)
    for s in range(K // 2):
        bit = 2 * s
        pos[:, s] = ((meta[:, bit // 32] >> np.uint64(bit % 32)) & np.uint64(3)).astype(np.int64)
    return pos


def decompress_24(values: np.ndarray, meta: np.ndarray, K: int) -> np.ndarray:
    """Dense bf16 bits [M, K]: each value goes back to 4g + pos; zeros elsewhere."""
    values = np.asarray(values, dtype=np.uint16)
    M = values.shape[0]
    pos = meta_positions(meta, K)
    out = np.zeros((M, K), dtype=np.uint16)
    s = np.arange(K // 2)
    cols = 4 * (s // 2)[None, :] + pos
    rows = np.repeat(np.arange(M)[:, None], K // 2, axis=1)
    out[rows, cols] = values
    return out


# ----------------------------------------------------------------------------
# Device layout: operand order of the gfx950 sparse MFMA (32x32x32, bf16)
# ----------------------------------------------------------------------------
# The instruction multiplies a 32-row x 32-column (logical) sparse A by a dense
# 32 x 32 B.  Lane L (0..63) holds, for row r = L mod 32, the 8 compressed
# values whose logical columns are 16*(L div 32) .. +16, and a 16-bit index
# with 4 bits per group (position of the group's first kept value in bits
# [0,2), second in [2,4)); the instruction's abid operand picks the low (0) or
# high (1) 16 bits of the 32-bit index register.
#
# Device values: blocks of 32 rows (rows >= M are zero), K-steps of 32 logical
# columns.  Block (rb, s) is 64 lanes x 8 bf16 = 1 KiB; lane L's 8 values are
# values[32*rb + L%32, 16*s + 8*(L//32) .. +8].  Block order: rb-major, s-minor.
# Device metadata: per 32-row block rb and K-pair t (64 logical columns), 64
# uint32; lane L's word is (positions of row 32*rb + L%32, logical columns
# 64t + 16*(L//32) .. +16) in bits [0,16) and the same for columns
# 64t + 32 + 16*(L//32) .. +16 in bits [16,32).  Within 16 bits, the position
# of the i-th compressed value sits at bits [2i, 2i+2) -- the same bit-stream
# order as the canonical layout.  Padded rows get position pattern 0x4444.
def device_rows(M: int) -> int:
    """Rows of the device layout: M rounded up to whole groups of four 32-row blocks."""
    return ((M + 127) // 128) * 128


def to_device_layout(values: np.ndarray, meta: np.ndarray, K: int):
    """Canonical (values [M, K/2], meta [M, K/32]) -> device (values flat u16, meta flat u32).

    Requires K % 64 == 0.  Index names: rb row block, r row in block, s K-step
    of 32 logical columns, t K-pair (64 logical columns), h lane half (L // 32),
    half = which K-step of the pair (abid), i compressed value within a lane.
    Rows are padded to a multiple of 128.  Values are stored [rb, s, L, i];
    metadata words [rb // 4, t, rb % 4, L] (the four row blocks of a group sit
    side by side for each K-pair, 1 KiB together).
    """
    if K % 64:
        raise ValueError("device layout needs K % 64 == 0")
    values = np.asarray(values, dtype=np.uint16)
    M = values.shape[0]
    Mp = device_rows(M)
    RB, S, T = Mp // 32, K // 32, K // 64
    vpad = np.zeros((Mp, K // 2), dtype=np.uint16)
    vpad[:M] = values
    pos = np.tile(np.array([0, 1], dtype=np.uint64), (Mp, K // 4))   # padded rows: 0x4 per group
    pos[:M] = meta_positions(meta, K).astype(np.uint64)
    # values: row = 32*rb + r, compressed column = 16*s + 8*h + i  ->  [rb, s, L = 32*h + r, i]
    dv = vpad.reshape(RB, 32, S, 2, 8).transpose(0, 2, 3, 1, 4).reshape(RB, S, 64, 8)
    # meta: compressed column = 32*t + 16*half + 8*h + i  ->  word[rb, t, L] bit 16*half + 2*i
    p6 = pos.reshape(RB, 32, T, 2, 2, 8).transpose(0, 2, 4, 1, 3, 5)   # rb, t, h, r, half, i
    shifts = (16 * np.arange(2)[:, None] + 2 * np.arange(8)[None, :]).astype(np.uint64)
    words = (p6 << shifts).sum(axis=(-2, -1), dtype=np.uint64)           # disjoint bits: sum == or
    grouped = words.reshape(RB // 4, 4, T, 64).transpose(0, 2, 1, 3)     # rbg, t, rq, L
    return dv.reshape(-1).copy(), grouped.astype(np.uint32).reshape(-1)


def from_device_layout(dvals: np.ndarray, dmeta: np.ndarray, M: int, K: int):
    """Inverse of ``to_device_layout`` (drops padded rows)."""
    Mp = device_rows(M)
    RB, S, T = Mp // 32, K // 32, K // 64
    dv = np.asarray(dvals, dtype=np.uint16).reshape(RB, S, 2, 32, 8)          # rb, s, h, r, i
    values = dv.transpose(0, 3, 1, 2, 4).reshape(Mp, K // 2)
    w = (np.asarray(dmeta, dtype=np.uint32).reshape(RB // 4, T, 4, 64).transpose(0, 2, 1, 3)
         .reshape(RB, T, 2, 32).astype(np.uint64))                               # rb, t, h, r
    shifts = (16 * np.arange(2)[:, None] + 2 * np.arange(8)[None, :]).astype(np.uint64)
    p6 = (w[..., None, None] >> shifts) & np.uint64(3)                             # rb, t, h, r, half, i
    pos = p6.transpose(0, 3, 1, 4, 2, 5).reshape(Mp, K // 2)                       # rb, r, t, half, h, i
    meta = np.zeros((Mp, meta_words_per_row(K)), dtype=np.uint64)
    for s in range(K // 2):
        meta[:, (2 * s) // 32] |= pos[:, s] << np.uint64((2 * s) % 32)
    return values[:M].copy(), meta[:M].astype(np.uint32)


# ----------------------------------------------------------------------------
# Masked fine-tuning ("Accelerating Sparse Deep Neural Networks", Abstract: the
# trained network is pruned to the 2:4 pattern and then retrained with it).
# Between re-prunes the master weights keep the stored pattern: every entry
# the metadata does not select is set to +0 after each update, kept entries
# are left bit for bit.  A re-prune is selection + compression of the current
# weights with the same zeroing, i.e. (prune_24(W), compress_24(W)).
# ----------------------------------------------------------------------------
def mask_from_meta(meta: np.ndarray, K: int) -> np.ndarray:
    """bool [M, K]: True at the two stored positions of every group of four."""
    pos = meta_positions(meta, K)                     # [M, K/2], positions in group order
    M = pos.shape[0]
    mask = np.zeros((M, K // 4, 4), dtype=bool)
    np.put_along_axis(mask, pos.reshape(M, K // 4, 2), True, axis=-1)
    return mask.reshape(M, K)


def mask_apply(W: np.ndarray, meta: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """W (fp32, or bf16 bits) with every entry outside the stored positions set to +0."""
    W = np.asarray(W)
    bits = W.view(np.uint32) if dtype == "f32" else np.asarray(W, dtype=np.uint16)
    out = np.where(mask_from_meta(meta, W.shape[1]), bits, bits.dtype.type(0)).astype(bits.dtype)
    return out.view(np.float32) if dtype == "f32" else out


def refresh(W: np.ndarray, dtype: str = "f32"):
    """Re-prune: (W with its dropped entries set to +0, values, canonical meta)."""
    values, meta = compress_24(W, dtype)
    return prune_24(W, dtype), values, meta


# ----------------------------------------------------------------------------
# Tile-vector-wise sparsity ("Accelerating Sparse DNNs Based on Tiled GEMM",
# Abstract and Figure 3: TW drop at the tile level, then 2:4 inside the tile)
# ----------------------------------------------------------------------------
def tvw_num_tiles(M: int, tile_m: int) -> int:
    return (M + tile_m - 1) // tile_m


def tvw_scores(W: np.ndarray, tile_m: int) -> np.ndarray:
    """fp64 column L1 score per tile, [T, K]; rows summed one at a time in ascending order."""
    W = np.asarray(W, dtype=np.float32)
    M, K = W.shape
    T = tvw_num_tiles(M, tile_m)
    out = np.zeros((T, K), dtype=np.float64)
    for t in range(T):
        acc = np.zeros(K, dtype=np.float64)
        for m in range(t * tile_m, min(M, (t + 1) * tile_m)):
            acc = acc + np.abs(W[m].astype(np.float64))
        out[t] = acc
    return out


SCORE_NAN_KEY = 0x7FF8000000000000


def score_key(sc: np.ndarray) -> np.ndarray:
    """Ranking key of computed fp64 scores (column, block and per-tile scores).

    A score is a sum of magnitudes, so it is +0, positive, +Inf or NaN, and
    for all but NaN its bit pattern read as an unsigned integer orders like
    its value.  The payload of a NaN that arithmetic produces is not fixed by
    IEEE 754, so every NaN score gets the one key 0x7FF8000000000000: above
    +Inf (0x7FF0000000000000), and NaN scores tie with each other, the tie
    going to the lower index like every other tie.
    """
    sc = np.asarray(sc, dtype=np.float64)
    key = sc.view(np.uint64).copy()
    key[np.isnan(sc)] = SCORE_NAN_KEY
    return key


def tvw_select(W: np.ndarray, tile_m: int, keep_k: int) -> np.ndarray:
    """Kept column indices per tile, int32 [T, keep_k], ascending.

    Order: score key descending (``score_key``: the value order, every NaN
    above +Inf), then column ascending (stable sort).
    """
    M, K = np.asarray(W).shape
    if not (0 < keep_k <= K) or keep_k % 4:
        raise ValueError("keep_k must be in (0, K] and a multiple of 4")
    sc = tvw_scores(W, tile_m)
    key = score_key(sc)
    order = np.argsort(np.iinfo(np.uint64).max - key, axis=1, kind="stable")
    kept = np.sort(order[:, :keep_k], axis=1)
    return kept.astype(np.int32)


def tvw_compress(W: np.ndarray, tile_m: int, keep_k: int):
    """Returns (kept int32 [T, keep_k], values u16 [M, keep_k/2], meta u32 [M, ceil(keep_k/32)])."""
    W = np.asarray(W, dtype=np.float32)
    M, K = W.shape
    kept = tvw_select(W, tile_m, keep_k)
    Wc = np.zeros((M, keep_k), dtype=np.float32)
    for t in range(kept.shape[0]):
        r0, r1 = t * tile_m, min(M, (t + 1) * tile_m)
        Wc[r0:r1] = W[r0:r1][:, kept[t]]
    values, meta = compress_24(Wc, "f32")
    return kept, values, meta


def tvw_decompress(kept: np.ndarray, values: np.ndarray, meta: np.ndarray, M: int, K: int,
                   tile_m: int) -> np.ndarray:
    """Dense bf16 bits [M, K] with the compacted columns scattered back."""
    keep_k = kept.shape[1]
    comp = decompress_24(values, meta, keep_k)          # [M, keep_k]
    out = np.zeros((M, K), dtype=np.uint16)
    for t in range(kept.shape[0]):
        r0, r1 = t * tile_m, min(M, (t + 1) * tile_m)
        out[r0:r1, kept[t]] = comp[r0:r1]
    return out


# ----------------------------------------------------------------------------
# TVW with per-tile keep counts ("Accelerating Sparse DNNs Based on Tiled GEMM",
# Abstract: a structured pattern inside each tile, irregular pruning across
# tiles; TL;DR: load balancing through batching).  Reading, for tile_m = 128:
#   * plan: rank every (tile, column) score of tvw_scores over the whole matrix
#     (score descending, then flat index t*K + k ascending); tile t's raw count
#     c_t is the number of its columns among the top total_keep; its keep count
#     is c_t rounded to the nearest multiple of 64 (halves up), clamped to
#     [64, K] -- 64 columns are one K step of the kernels, and every tile keeps
#     at least one;
#   * tile t keeps its count highest-scored columns (tvw_select's order),
#     listed ascending, then 2:4 over its compacted axis;
#   * storage: the tiles' device-layout blocks one after another in tile order;
#   * batching order: tiles by keep count descending, then tile ascending.
# ----------------------------------------------------------------------------
VAR_STEP = 64


def tvw_var_counts(W: np.ndarray, tile_m: int, total_keep: int) -> np.ndarray:
    """Per-tile keep counts, int32 [T]."""
    sc = tvw_scores(W, tile_m)
    T, K = sc.shape
    if K % VAR_STEP or not (0 < total_keep <= T * K):
        raise ValueError("K must be a multiple of 64 and 0 < total_keep <= T*K")
    key = score_key(sc).reshape(-1)
    ranked = np.argsort(np.iinfo(np.uint64).max - key, kind="stable")
    raw = np.bincount(ranked[:total_keep] // K, minlength=T)
    counts = VAR_STEP * ((raw + VAR_STEP // 2) // VAR_STEP)
    return np.clip(counts, VAR_STEP, K).astype(np.int32)


def tvw_var_compress(W: np.ndarray, tile_m: int, counts):
    """Per tile: (kept int32 [c_t] ascending, values u16 [rows_t, c_t/2], meta u32 [rows_t, c_t/32])."""
    W = np.asarray(W, dtype=np.float32)
    M, K = W.shape
    key = score_key(tvw_scores(W, tile_m))
    out = []
    for t, c in enumerate(np.asarray(counts)):
        order = np.argsort(np.iinfo(np.uint64).max - key[t], kind="stable")
        kept = np.sort(order[:int(c)]).astype(np.int32)
        r0, r1 = t * tile_m, min(M, (t + 1) * tile_m)
        values, meta = compress_24(W[r0:r1][:, kept], "f32")
        out.append((kept, values, meta))
    return out


def tvw_var_device(tiles, counts):
    """(kept flat int32, device values flat u16, device meta flat u32, offsets int32 [T+1]):
    each tile's device layout (128 rows) appended in tile order."""
    kept = np.concatenate([k for k, _, _ in tiles]).astype(np.int32)
    dv, dm = [], []
    for (k, v, m), c in zip(tiles, counts):
        a, b = to_device_layout(v, m, int(c))
        dv.append(a)
        dm.append(b)
    offsets = np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]).astype(np.int32)
    return kept, np.concatenate(dv), np.concatenate(dm), offsets


def tvw_var_order(counts) -> np.ndarray:
    """Batching order: keep count descending, then tile ascending."""
    counts = np.asarray(counts)
    return np.lexsort((np.arange(len(counts)), -counts)).astype(np.int32)


def tvw_var_decompress(tiles, M: int, K: int, tile_m: int) -> np.ndarray:
    """Dense bf16 bits [M, K] with every tile's compacted columns scattered back."""
    out = np.zeros((M, K), dtype=np.uint16)
    for t, (kept, values, meta) in enumerate(tiles):
        r0, r1 = t * tile_m, min(M, (t + 1) * tile_m)
        out[r0:r1][:, kept] = decompress_24(values, meta, len(kept))
    return out


# ----------------------------------------------------------------------------
# TW alone ("Accelerating Sparse DNNs Based on Tiled GEMM", Abstract and
# Figure 3: the tile-level column drop without the 2:4 step inside the tile).
# The kept columns are chosen exactly as for TVW (fixed keep_k per tile, or the
# per-tile counts of tvw_var_counts) and multiplied densely: each tile's rows
# restricted to its kept columns, rounded to bf16 (nearest even).
# Dense device layout (the dense MFMA's A operand order): blocks of 32 rows
# (padding rows zero) and 16 columns; block (rb, s) is 64 lanes x 8 bf16, lane
# L's 8 values are W[32 rb + L % 32][16 s + 8 (L // 32) .. +8]; rb-major.
# ----------------------------------------------------------------------------
def dense_device_layout(Wbits: np.ndarray, rows: int) -> np.ndarray:
    """bf16 bits [R, K] (R <= rows, rows % 32 == 0, K % 16 == 0) -> flat u16 in the dense device layout."""
    Wbits = np.asarray(Wbits, dtype=np.uint16)
    R, K = Wbits.shape
    if rows % 32 or K % 16 or R > rows:
        raise ValueError("rows must be a multiple of 32 covering W, K a multiple of 16")
    pad = np.zeros((rows, K), dtype=np.uint16)
    pad[:R] = Wbits
    # row = 32 rb + r, column = 16 s + 8 h + i  ->  [rb, s, L = 32 h + r, i]
    return pad.reshape(rows // 32, 32, K // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1).copy()


def tw_compress(W: np.ndarray, tile_m: int, keep_k: int):
    """(kept int32 [T, keep_k], Wc bf16 bits [M, keep_k]): tile t's rows on its kept columns."""
    W = np.asarray(W, dtype=np.float32)
    kept = tvw_select(W, tile_m, keep_k)
    Wc = np.zeros((W.shape[0], keep_k), dtype=np.uint16)
    for t in range(kept.shape[0]):
        r0, r1 = t * tile_m, min(W.shape[0], (t + 1) * tile_m)
        Wc[r0:r1] = bf16_rne(W[r0:r1][:, kept[t]])
    return kept, Wc


def tw_var_compress(W: np.ndarray, tile_m: int, counts):
    """Per tile (kept int32 [c_t] ascending, Wc bf16 bits [rows_t, c_t])."""
    W = np.asarray(W, dtype=np.float32)
    out = []
    for t, (kept, _, _) in enumerate(tvw_var_compress(W, tile_m, counts)):
        r0, r1 = t * tile_m, min(W.shape[0], (t + 1) * tile_m)
        out.append((kept, bf16_rne(W[r0:r1][:, kept])))
    return out


def tw_var_device(tiles, counts):
    """(kept flat int32, dense device values flat u16): each tile's 128-row dense layout in tile order."""
    kept = np.concatenate([k for k, _ in tiles]).astype(np.int32)
    dv = np.concatenate([dense_device_layout(w, 128) for _, w in tiles])
    return kept, dv


def tw_decompress(kept_list, Wc_list, M: int, K: int, tile_m: int) -> np.ndarray:
    """Dense bf16 bits [M, K] with every tile's columns scattered back (dropped columns zero)."""
    out = np.zeros((M, K), dtype=np.uint16)
    for t, (kept, Wc) in enumerate(zip(kept_list, Wc_list)):
        r0, r1 = t * tile_m, min(M, (t + 1) * tile_m)
        out[r0:r1][:, kept] = Wc[: r1 - r0]
    return out


# ----------------------------------------------------------------------------
# Comparison patterns ("Accelerating Sparse DNNs Based on Tiled GEMM",
# Abstract: TVW against block sparsity and unstructured sparsity; Figure 5
# names the element-wise (EW) and block-wise (BW) patterns, caption only).
# BW: blocks of 128 rows (a tile) x 64 columns (a K step); a block's score is
#   the fp64 sum of its 64 tile column scores (tvw_scores) in ascending column
#   order; each tile keeps its keep_blocks highest-scored blocks (ties -> lower
#   block), and their columns, ascending, are multiplied densely as in TW.
# EW: every weight ranked by magnitude (sign-cleared bit pattern, as for 2:4)
#   over the whole matrix, ties -> lower flat index m*K + k; the top
#   keep_total are kept, in CSR form (row pointers, ascending columns, bf16
#   values rounded to nearest even).
# ----------------------------------------------------------------------------
BW_COLS = 64


def bw_block_scores(W: np.ndarray) -> np.ndarray:
    """fp64 [T, K/64]: per 128-row tile and 64-column block, the sum of the tile column scores."""
    sc = tvw_scores(W, 128)
    T, K = sc.shape
    if K % BW_COLS:
        raise ValueError("K must be a multiple of 64")
    out = np.zeros((T, K // BW_COLS), dtype=np.float64)
    for j in range(K // BW_COLS):
        acc = np.zeros(T, dtype=np.float64)
        for c in range(BW_COLS):
            acc = acc + sc[:, BW_COLS * j + c]
        out[:, j] = acc
    return out


def bw_select(W: np.ndarray, keep_blocks: int) -> np.ndarray:
    """Kept columns per tile, int32 [T, keep_blocks * 64], ascending."""
    bs = bw_block_scores(W)
    if not (0 < keep_blocks <= bs.shape[1]):
        raise ValueError("keep_blocks must be in (0, K/64]")
    order = np.argsort(np.iinfo(np.uint64).max - score_key(bs), axis=1, kind="stable")
    blocks = np.sort(order[:, :keep_blocks], axis=1)
    cols = (blocks[:, :, None] * BW_COLS + np.arange(BW_COLS)[None, None, :]).reshape(bs.shape[0], -1)
    return cols.astype(np.int32)


def bw_compress(W: np.ndarray, keep_blocks: int):
    """(kept int32 [T, keep_blocks*64], Wc bf16 bits [M, keep_blocks*64]) as for TW."""
    W = np.asarray(W, dtype=np.float32)
    kept = bw_select(W, keep_blocks)
    Wc = np.zeros((W.shape[0], kept.shape[1]), dtype=np.uint16)
    for t in range(kept.shape[0]):
        r0, r1 = 128 * t, min(W.shape[0], 128 * t + 128)
        Wc[r0:r1] = bf16_rne(W[r0:r1][:, kept[t]])
    return kept, Wc


def ew_compress(W: np.ndarray, keep_total: int):
    """(row_ptr int64 [M+1], cols int32 [keep_total], vals bf16 bits [keep_total])."""
    W = np.asarray(W, dtype=np.float32)
    M, K = W.shape
    if not (0 < keep_total <= M * K):
        raise ValueError("keep_total must be in (0, M*K]")
    key = magnitude_key(W, "f32").reshape(-1)
    ranked = np.argsort(np.iinfo(np.uint64).max - key.astype(np.uint64), kind="stable")
    chosen = np.sort(ranked[:keep_total])                  # flat indices, row-major = CSR order
    rows, cols = chosen // K, chosen % K
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=M))]).astype(np.int64)
    return row_ptr, cols.astype(np.int32), bf16_rne(W.reshape(-1)[chosen])


def ew_decompress(row_ptr, cols, vals, M: int, K: int) -> np.ndarray:
    """Dense bf16 bits [M, K] from the CSR form."""
    out = np.zeros((M, K), dtype=np.uint16)
    for m in range(M):
        out[m, cols[row_ptr[m]:row_ptr[m + 1]]] = vals[row_ptr[m]:row_ptr[m + 1]]
    return out


# ----------------------------------------------------------------------------
# GEMM reference and bound (fp64; every bf16 x bf16 product is exact in fp64)
# ----------------------------------------------------------------------------
def gemm_ref(Wd: np.ndarray, X: np.ndarray, rows=None):
    """(y_ref, bound) for Y = W X; Wd, X are bf16 bits; rows optionally selects output rows."""
    Wf = bf16_to_f64(Wd if rows is None else np.asarray(Wd)[rows])
    Xf = bf16_to_f64(X)
    return Wf @ Xf, np.abs(Wf) @ np.abs(Xf)


def spmm_ref_sparse(values: np.ndarray, meta: np.ndarray, K: int, X: np.ndarray, rows=None):
    """Sparse route: y[m, :] = sum_s values[m, s] * X[4*(s//2) + pos[m, s], :] in fp64."""
    values = np.asarray(values, dtype=np.uint16)
    if rows is None:
        rows = np.arange(values.shape[0])
    rows = np.asarray(rows)
    pos = meta_positions(np.asarray(meta)[rows], K)
    Xf = bf16_to_f64(X)
    s = np.arange(K // 2)
    y = np.zeros((len(rows), Xf.shape[1]), dtype=np.float64)
    for i, m in enumerate(rows):
        ks = 4 * (s // 2) + pos[i]
        y[i] = bf16_to_f64(values[m]) @ Xf[ks]
    return y


# ----------------------------------------------------------------------------
# Fused epilogue: y = act(W X + b).  "Accelerating Sparse DNNs Based on Tiled
# GEMM" (TL;DR) names kernel fusion among its techniques without details; the
# reading here: b holds one fp32 value per output row (feature), added to the
# product before the activation; act is none, ReLU (z > 0 ? z : 0, so NaN -> 0)
# or GELU in its exact form z * Phi(z) = z/2 (1 + erf(z / sqrt 2)), the one
# BERT uses.
# ----------------------------------------------------------------------------
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
GELU_LIPSCHITZ = 1.13            # max |d/dz z Phi(z)| = 1.1289... (pinned in the tests)
ACT_REL_ERR = 2.0 ** -20         # allowance for the kernel's fp32 evaluation of the activation


def act_ref(z: np.ndarray, act: int) -> np.ndarray:
    """Activation in fp64."""
    z = np.asarray(z, dtype=np.float64)
    if act == ACT_NONE:
        return z.copy()
    if act == ACT_RELU:
        return np.where(z > 0, z, 0.0)
    if act == ACT_GELU:
        from scipy.special import erf
        return 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))
    raise ValueError(act)


def fused_ref(Wd: np.ndarray, X: np.ndarray, bias, act: int, rows=None):
    """(y_ref, z_ref, bound): y = act(W X + b) in fp64, the pre-activation z and the GEMM bound."""
    y, bnd = gemm_ref(Wd, X, rows=rows)
    M = np.asarray(Wd).shape[0]
    b = np.zeros(M) if bias is None else np.asarray(bias, dtype=np.float32).astype(np.float64)
    if rows is not None:
        b = b[np.asarray(rows)]
    z = y + b[:, None]
    return act_ref(z, act), z, bnd


def fused_tolerance(y_ref: np.ndarray, z_ref: np.ndarray, bound: np.ndarray, act: int,
                    out_dtype: str) -> np.ndarray:
    """Bound on |y - y_ref| for the fused result: the GEMM bound plus one fp32
    rounding of the bias add, carried through the activation's Lipschitz
    constant, plus the activation's own evaluation error, then the output
    rounding (bf16: half an ulp of the result)."""
    lip = {ACT_NONE: 1.0, ACT_RELU: 1.0, ACT_GELU: GELU_LIPSCHITZ}[act]
    pre = TOL_REL * bound + 2.0 ** -23 * np.abs(z_ref)
    tol = lip * pre + (ACT_REL_ERR * np.abs(y_ref) if act == ACT_GELU else 0.0)
    if out_dtype == "f32":
        return tol
    if out_dtype == "bf16":
        return tol + BF16_HALF_ULP * (np.abs(y_ref) + tol)
    raise ValueError(out_dtype)


def check_fused(y, y_ref, z_ref, bound, act: int, out_dtype: str):
    """(ok, worst err/tol ratio) for a fused result.  Non-finite outputs fail."""
    y = np.asarray(y, dtype=np.float64)
    tol = fused_tolerance(y_ref, z_ref, bound, act, out_dtype)
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.isfinite(y).all() and worst <= 1.0), worst


def tolerance(y_ref: np.ndarray, bound: np.ndarray, out_dtype: str) -> np.ndarray:
    if out_dtype == "f32":
        return TOL_REL * bound
    if out_dtype == "bf16":
        return TOL_REL * bound + BF16_HALF_ULP * (np.abs(y_ref) + TOL_REL * bound)
    raise ValueError(out_dtype)


def check(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, out_dtype: str):
    """(ok, worst err/tol ratio).  Non-finite outputs always fail."""
    y = np.asarray(y, dtype=np.float64)
    tol = tolerance(y_ref, bound, out_dtype)
    err = np.abs(y - y_ref)
    finite = np.isfinite(y).all()
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(finite and worst <= 1.0), worst


# ----------------------------------------------------------------------------
# Two-layer chain ("Accelerating Sparse DNNs Based on Tiled GEMM", TL;DR:
# kernel fusion).  Reading: layer 1 (2:4) computes h = act1(W1 X + b1) and
# stores it as bf16 H, features x tokens; layer 2 (TVW) computes
# y2 = act2(W2 H + b2).  The reference uses the exact h; the tolerance carries
# layer 1's elementwise bound on |H - h| (its fused bound with the bf16
# rounding of H) through |W2| into layer 2, whose own GEMM bound is taken on
# |W2| (|h| + that bound).
# ----------------------------------------------------------------------------
def chain_ref(W1d: np.ndarray, X: np.ndarray, bias1, act1: int, W2d: np.ndarray, bias2, act2: int):
    """(y2_ref, z2_ref, bound2, carried): y2 = act2(W2 h + b2) with h = act1(W1 X + b1)
    exact in fp64; bound2 = |W2| (|h| + tol_h); carried = |W2| tol_h, where tol_h is
    layer 1's bf16-output tolerance."""
    h, z1, bnd1 = fused_ref(W1d, X, bias1, act1)
    tol_h = fused_tolerance(h, z1, bnd1, act1, "bf16")
    W2f = bf16_to_f64(W2d)
    M2 = W2f.shape[0]
    b2 = np.zeros(M2) if bias2 is None else np.asarray(bias2, dtype=np.float32).astype(np.float64)
    z2 = W2f @ h + b2[:, None]
    aW2 = np.abs(W2f)
    return act_ref(z2, act2), z2, aW2 @ (np.abs(h) + tol_h), aW2 @ tol_h


def chain_tolerance(y2_ref, z2_ref, bound2, carried, act2: int, out_dtype: str) -> np.ndarray:
    """Bound on |y2 - y2_ref|: layer 2's fused bound on bound2 plus the carried
    difference of H, both through act2's Lipschitz constant, then the output rounding."""
    lip = {ACT_NONE: 1.0, ACT_RELU: 1.0, ACT_GELU: GELU_LIPSCHITZ}[act2]
    tol = fused_tolerance(y2_ref, z2_ref, bound2, act2, "f32") + lip * carried
    if out_dtype == "f32":
        return tol
    if out_dtype == "bf16":
        return tol + BF16_HALF_ULP * (np.abs(y2_ref) + tol)
    raise ValueError(out_dtype)


def check_chain(y2, y2_ref, z2_ref, bound2, carried, act2: int, out_dtype: str):
    """(ok, worst err/tol ratio) for the chain's output.  Non-finite outputs fail."""
    y2 = np.asarray(y2, dtype=np.float64)
    tol = chain_tolerance(y2_ref, z2_ref, bound2, carried, act2, out_dtype)
    err = np.abs(y2 - y2_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.isfinite(y2).all() and worst <= 1.0), worst
