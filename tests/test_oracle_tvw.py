"""Pins for the oracle's tile-vector-wise (TVW) selection and compression.

"Accelerating Sparse DNNs Based on Tiled GEMM" (Abstract, Figure 3): tile-wise
sparsity keeps a regular structure inside each GEMM tile but prunes
irregularly across tiles, at the global-memory level; TVW then applies the 2:4
pattern inside the tile.  Readings: tile = 128 output rows, column score = L1
norm over the tile's rows (fp64, ascending rows), keep the top half (ties to
the lower column), 2:4 along the compacted axis.

Pins: the hand-worked fixture, brute force over every subset on a tiny tile,
exact integer scores, keep_k == K reducing to plain 2:4, and the 25% density.
"""
import itertools

import numpy as np

from oracle import prune24 as O
from workloads import random_matrix, small_int_matrix


def test_hand_example(golden):
    ex = golden["tvw"]
    W = np.array(ex["W"], dtype=np.float32)
    assert O.tvw_scores(W, ex["tile_m"]).tolist() == ex["scores"]
    kept, values, meta = O.tvw_compress(W, ex["tile_m"], ex["keep_k"])
    assert kept.tolist() == ex["kept"]
    assert O.bf16_to_f64(values).tolist() == ex["values"]
    assert [f"{int(w):08X}" for w in meta[:, 0]] == ex["meta_hex"]


def test_bruteforce_subsets_tiny_tile():
    # integer data with many tied scores; K = 16, keep 8 -> all C(16, 8) = 12870 subsets
    for seed in range(4):
        W = small_int_matrix((4, 16), seed=100 + seed, lo=-2, hi=2)
        kept = O.tvw_select(W, 4, 8)[0]
        score = np.abs(W.astype(np.float64)).sum(0)
        winners = []
        for S in itertools.combinations(range(16), 8):
            drop = [k for k in range(16) if k not in S]
            if all(score[a] > score[b] or (score[a] == score[b] and a < b) for a in S for b in drop):
                winners.append(S)
        assert len(winners) == 1
        assert tuple(kept.tolist()) == winners[0]


def test_scores_exact_on_integers_and_partial_tile():
    W = small_int_matrix((300, 64), seed=7)
    sc = O.tvw_scores(W, 128)
    assert sc.shape == (3, 64)
    for t, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        exact = np.abs(W[r0:r1].astype(np.int64)).sum(0)
        assert np.array_equal(sc[t], exact.astype(np.float64))


def test_keep_all_is_plain_24():
    W = random_matrix((256, 128), seed=8, sigma=0.02)
    kept, values, meta = O.tvw_compress(W, 128, 128)
    assert (kept == np.arange(128)).all()
    v2, m2 = O.compress_24(W, "f32")
    assert np.array_equal(values, v2) and np.array_equal(meta, m2)


def test_density_and_tile_structure():
    M, K, tile, keep = 512, 256, 128, 128
    W = random_matrix((M, K), seed=9, sigma=0.02)
    kept, values, meta = O.tvw_compress(W, tile, keep)
    assert kept.shape == (4, keep) and (np.diff(kept, axis=1) > 0).all()
    Wd = O.tvw_decompress(kept, values, meta, M, K, tile)
    assert (Wd != 0).mean() == 0.25
    for t in range(4):
        blk = Wd[t * tile:(t + 1) * tile]
        dropped = np.setdiff1d(np.arange(K), kept[t])
        assert (blk[:, dropped] == 0).all()
        # kept columns satisfy 2:4 along the compacted axis
        comp = blk[:, kept[t]].reshape(tile, -1, 4)
        assert ((comp != 0).sum(-1) <= 2).all()
    # the kept columns have scores no lower than the dropped ones
    sc = O.tvw_scores(W, tile)
    for t in range(4):
        dropped = np.setdiff1d(np.arange(K), kept[t])
        assert sc[t, kept[t]].min() >= sc[t, dropped].max()
