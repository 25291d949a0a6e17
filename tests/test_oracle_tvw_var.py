"""Pins for the variable-keep TVW oracle (per-tile keep counts from a global ranking).

Counts are re-derived by brute force over every (tile, column) pair; equal
counts reduce to the fixed-keep TVW oracle (pinned separately) exactly; ties
fall to the lower flat index; the device storage is each tile's device layout
at the offsets the counts give; decompression scatters every kept value back.
"""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O


def _brute_counts(W, tile_m, total_keep):
    sc = O.tvw_scores(W, tile_m)
    T, K = sc.shape
    items = [(sc[t, k], t * K + k) for t in range(T) for k in range(K)]
    items.sort(key=lambda x: (-x[0], x[1]))
    raw = [0] * T
    for _, f in items[:total_keep]:
        raw[f // K] += 1
    out = []
    for c in raw:
        r = 64 * ((c + 32) // 64)
        out.append(min(max(r, 64), K))
    return np.array(out)


@pytest.mark.parametrize("total_frac", [0.1, 0.3, 0.5, 0.77, 1.0])
def test_counts_brute_force(total_frac):
    W = workloads.random_matrix((384, 256), seed=3, sigma=0.02)
    # give the tiles different importance so counts differ
    W[:128] *= 3.0
    W[256:] *= 0.3
    total = int(total_frac * 3 * 256)
    assert np.array_equal(O.tvw_var_counts(W, 128, total), _brute_counts(W, 128, total))


def test_counts_ties_go_to_lower_flat_index():
    W = np.ones((256, 128), dtype=np.float32)       # every score equal
    # top 128 of the flat order are all of tile 0; tile 1 gets nothing -> clamped to 64
    assert O.tvw_var_counts(W, 128, 128).tolist() == [128, 64]
    assert O.tvw_var_counts(W, 128, 192).tolist() == [128, 64]   # raw [128, 64]
    assert O.tvw_var_counts(W, 128, 159).tolist() == [128, 64]   # raw [128, 31] -> 0 -> 64


def test_rounding_and_density():
    W = workloads.random_matrix((1024, 512), seed=4, sigma=0.02)
    W[:256] *= 2.0
    total = 1024 // 128 * 512 // 2
    c = O.tvw_var_counts(W, 128, total)
    assert (c % 64 == 0).all() and (c >= 64).all() and (c <= 512).all()
    assert abs(int(c.sum()) - total) <= 32 * len(c)
    assert c[:2].min() > c[2:].max()          # the scaled-up tiles keep more


def test_equal_counts_reduce_to_fixed_keep():
    W = workloads.random_matrix((256, 256), seed=5, sigma=0.02)
    counts = np.array([128, 128], dtype=np.int32)
    tiles = O.tvw_var_compress(W, 128, counts)
    kept, values, meta = O.tvw_compress(W, 128, 128)
    for t in range(2):
        assert np.array_equal(tiles[t][0], kept[t])
        assert np.array_equal(tiles[t][1], values[t * 128:(t + 1) * 128])
        assert np.array_equal(tiles[t][2], meta[t * 128:(t + 1) * 128])


def test_device_storage_and_order():
    W = workloads.random_matrix((300, 256), seed=6, sigma=0.02)     # partial last tile
    counts = np.array([192, 64, 128], dtype=np.int32)
    tiles = O.tvw_var_compress(W, 128, counts)
    kept, dv, dm, off = O.tvw_var_device(tiles, counts)
    assert off.tolist() == [0, 192, 256, 384]
    assert kept.size == 384 and dv.size == 128 * 384 // 2 and dm.size == 16 * 384 // 4
    for t, c in enumerate(counts):
        a, b = O.to_device_layout(tiles[t][1], tiles[t][2], int(c))
        assert np.array_equal(dv[off[t] * 64: off[t + 1] * 64], a)
        assert np.array_equal(dm[off[t] * 4: off[t + 1] * 4], b)
        assert np.array_equal(kept[off[t]:off[t + 1]], tiles[t][0])
    assert O.tvw_var_order(counts).tolist() == [0, 2, 1]
    assert O.tvw_var_order(np.array([64, 128, 128, 64])).tolist() == [1, 2, 0, 3]


def test_decompress_scatter_brute_force():
    W = workloads.random_matrix((256, 192), seed=7, sigma=0.02)
    counts = np.array([128, 64], dtype=np.int32)
    tiles = O.tvw_var_compress(W, 128, counts)
    Wd = O.tvw_var_decompress(tiles, 256, 192, 128)
    for t, (kept, values, meta) in enumerate(tiles):
        dense_c = O.decompress_24(values, meta, len(kept))
        for r in range(128):
            row = np.zeros(192, dtype=np.uint16)
            row[kept] = dense_c[r]
            assert np.array_equal(Wd[t * 128 + r], row)
    # every tile keeps exactly half of its compacted columns nonzero at most
    nz = (Wd != 0).sum(axis=1)
    assert (nz[:128] <= 64).all() and (nz[128:] <= 32).all()
