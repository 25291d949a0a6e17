"""GPU parity of the column, tile and block selections when weights hold NaN
(with different payloads) and +-Inf: tvw_compress, tw_compress,
tvw_var_compress and bw_compress against the oracle, bit for bit.

Reading ("Accelerating Sparse DNNs Based on Tiled GEMM", Abstract and Figure 3
rank columns by importance and are silent on non-finite weights): a NaN score
ranks above +Inf and all NaN scores tie (lower index first), whatever payload
the sums carry.  The fixtures put the cut among tied NaN columns, among tied
+Inf columns and between the two, in several tiles at once."""
import numpy as np
import pytest

from oracle import prune24 as O
from gpu_util import f32_dev, need_gpu, torch, u16_host, u32_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _nan_bits(rng, n):
    """Quiet NaNs with random payloads and signs (fp32 bit patterns)."""
    sign = rng.integers(0, 2, n).astype(np.uint32) << 31
    return (sign | 0x7FC00000 | rng.integers(0, 1 << 22, n).astype(np.uint32)).astype(np.uint32)


def _weights(M, K, seed):
    """Tiles of 128 rows: tile 0 has more NaN columns than any keep count, tile 1 a
    few NaN and some +-Inf columns, tile 2 more +Inf columns than any keep count,
    tile 3 a NaN and +Inf in the same column, the rest finite."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    U = W.view(np.uint32)
    T = -(-M // 128)
    for t in range(T):
        r0, r1 = 128 * t, min(M, 128 * t + 128)
        kind = t % 5
        if kind == 0:
            cols = rng.choice(K, size=(3 * K) // 4, replace=False)
        elif kind == 1:
            cols = rng.choice(K, size=K // 8, replace=False)
        elif kind == 2:
            cols = rng.choice(K, size=(3 * K) // 4, replace=False)
        elif kind == 3:
            cols = rng.choice(K, size=K // 16, replace=False)
        else:
            continue
        rows = rng.integers(r0, r1, cols.size)
        if kind in (0, 1):
            U[rows, cols] = _nan_bits(rng, cols.size)
        if kind in (1, 2):
            icols = rng.choice(K, size=K // 4 if kind == 1 else (3 * K) // 4, replace=False)
            irows = rng.integers(r0, r1, icols.size)
            U[irows, icols] = np.where(rng.integers(0, 2, icols.size) == 1, 0xFF800000, 0x7F800000).astype(np.uint32)
        if kind == 3:
            U[rows, cols] = _nan_bits(rng, cols.size)
            U[np.minimum(rows + 1, r1 - 1), cols] = 0x7F800000
    return W


@pytest.mark.parametrize("M,K,keep,layout", [
    (640, 256, 128, "device"),
    (640, 512, 192, "canonical"),
    (600, 1536, 512, "device"),        # partial last tile, two scan chunks
])
def test_tvw_compress_nonfinite(M, K, keep, layout):
    need_gpu()
    W = _weights(M, K, seed=M + K)
    print(f"[nonfinite] tvw_compress {M}x{K} keep {keep} {layout}", flush=True)
    t = p24.tvw_compress(f32_dev(W), tile_m=128, keep_k=keep, layout=layout)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        kept, values, meta = O.tvw_compress(W, 128, keep)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    if layout == "device":
        values, meta = O.to_device_layout(values, meta, keep)
    ov, om = values.reshape(-1), meta.reshape(-1)
    assert np.array_equal(u16_host(t.values)[:ov.size], ov)
    assert np.array_equal(u32_host(t.meta)[:om.size], om)


def test_tw_compress_nonfinite():
    need_gpu()
    M, K, keep = 640, 512, 256
    W = _weights(M, K, seed=21)
    print(f"[nonfinite] tw_compress {M}x{K} keep {keep}", flush=True)
    t = p24.tw_compress(f32_dev(W), 128, keep)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        kept, Wc = O.tw_compress(W, 128, keep)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    dv = O.dense_device_layout(Wc, -(-M // 32) * 32)
    assert np.array_equal(u16_host(t.Wp)[:dv.size], dv)


@pytest.mark.parametrize("frac", [0.1, 0.4, 0.75])
def test_tvw_var_compress_nonfinite(frac):
    need_gpu()
    M, K = 1280, 256
    W = _weights(M, K, seed=31)
    T = M // 128
    total = int(frac * T * K)
    print(f"[nonfinite] tvw_var_compress {M}x{K} total {total}", flush=True)
    t = p24.tvw_var_compress(f32_dev(W), total_keep=total)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        counts = O.tvw_var_counts(W, 128, total)
        tiles = O.tvw_var_compress(W, 128, counts)
    kept, dv, dm, off = O.tvw_var_device(tiles, counts)
    assert np.array_equal(t.offsets.cpu().numpy(), off.astype(np.int64))
    assert np.array_equal(t.order.cpu().numpy(), O.tvw_var_order(counts))
    n = int(off[-1])
    assert np.array_equal(t.kept.cpu().numpy()[:n], kept)
    assert np.array_equal(u16_host(t.values)[:dv.size], dv)
    assert np.array_equal(u32_host(t.meta)[:dm.size], dm)


@pytest.mark.parametrize("keep_blocks", [1, 3, 6])
def test_bw_compress_nonfinite(keep_blocks):
    need_gpu()
    M, K = 640, 512
    W = _weights(M, K, seed=41)
    print(f"[nonfinite] bw_compress {M}x{K} keep {keep_blocks} blocks", flush=True)
    t = p24.bw_compress(f32_dev(W), keep_blocks)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        kept, Wc = O.bw_compress(W, keep_blocks)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    dv = O.dense_device_layout(Wc, -(-M // 32) * 32)
    assert np.array_equal(u16_host(t.Wp)[:dv.size], dv)


def test_fixture_has_nan_ties_at_the_cut():
    """The fixture exercises what it claims: NaN scores with several bit patterns,
    and a tile whose NaN columns outnumber the keep count (CPU-side check)."""
    W = _weights(640, 256, seed=896)
    with np.errstate(invalid="ignore", over="ignore"):
        sc = O.tvw_scores(W, 128)
    assert np.isnan(sc[0]).sum() > 128
    assert len({int(b) for b in sc.view(np.uint64)[np.isnan(sc)]}) > 3
    assert np.isposinf(sc[2]).sum() > 128
