"""Pins for the BW (block-wise) and EW (unstructured) comparison oracles.

BW block scores equal the exact block sums of |W| on integer-valued weights;
the chosen blocks beat every dropped block under (score desc, block asc),
checked by brute force over every subset; keeping every block keeps every
column.  EW is re-derived by brute force over all (key, flat index) pairs,
ties fall in row-major order, and the CSR form scatters back to the kept
entries exactly.
"""
import itertools

import numpy as np
import pytest

import workloads
from oracle import prune24 as O


def test_bw_block_scores_exact_sums():
    W = workloads.small_int_matrix((300, 256), seed=71)
    bs = O.bw_block_scores(W)
    for t in range(3):
        for j in range(4):
            blk = W[128 * t: min(300, 128 * t + 128), 64 * j: 64 * j + 64]
            assert bs[t, j] == np.abs(blk.astype(np.float64)).sum()


def test_bw_selection_brute_force():
    W = workloads.small_int_matrix((256, 256), seed=72, lo=-3, hi=3)
    W[:, 64:128] = W[:, 0:64]                      # blocks 0 and 1 tie in every tile
    bs = O.bw_block_scores(W)
    for keep in range(1, 5):
        kept = O.bw_select(W, keep)
        for t in range(2):
            best = None
            for sub in itertools.combinations(range(4), keep):
                rest = [j for j in range(4) if j not in sub]
                rank = lambda j: (-bs[t, j], j)
                if all(max(rank(j) for j in sub) < rank(r) for r in rest):
                    best = sub
            assert best is not None
            cols = np.concatenate([np.arange(64 * j, 64 * j + 64) for j in best])
            assert np.array_equal(kept[t], cols)


def test_bw_keep_all_and_values():
    W = workloads.random_matrix((200, 192), seed=73, sigma=0.05)
    kept, Wc = O.bw_compress(W, 3)
    assert (kept == np.arange(192)).all()
    assert np.array_equal(Wc, O.bf16_rne(W))
    kept, Wc = O.bw_compress(W, 1)
    assert kept.shape == (2, 64) and all((k[1:] - k[:-1] == 1).all() and k[0] % 64 == 0 for k in kept)


def _ew_brute(W, keep):
    M, K = W.shape
    bits = W.view(np.uint32) & 0x7FFFFFFF
    items = sorted(((-int(bits[m, k]), m * K + k) for m in range(M) for k in range(K)))[:keep]
    return sorted(f for _, f in items)


@pytest.mark.parametrize("keep", [1, 17, 100, 24 * 20])
def test_ew_brute_force(keep):
    W = workloads.random_matrix((24, 20), seed=74, sigma=0.05)
    W[3, :] = 0.25                                  # a row of ties
    W[5, 2] = -0.25                                 # a tie of opposite sign
    rp, cols, vals = O.ew_compress(W, keep)
    flat = _ew_brute(W, keep)
    assert rp[-1] == keep and (np.diff(rp) >= 0).all()
    got = [m * 20 + int(c) for m in range(24) for c in cols[rp[m]:rp[m + 1]]]
    assert got == flat
    assert np.array_equal(vals, O.bf16_rne(W.reshape(-1)[flat]))


def test_ew_ties_row_major_and_scatter():
    W = np.full((8, 16), 0.5, dtype=np.float32)
    rp, cols, vals = O.ew_compress(W, 20)
    assert rp.tolist() == [0, 16, 20, 20, 20, 20, 20, 20, 20]
    assert cols.tolist() == list(range(16)) + [0, 1, 2, 3]
    W2 = workloads.random_matrix((32, 48), seed=75, sigma=0.05)
    rp, cols, vals = O.ew_compress(W2, 300)
    Wd = O.ew_decompress(rp, cols, vals, 32, 48)
    assert (Wd != 0).sum() == 300
    thr = np.sort(np.abs(W2).reshape(-1))[-300]
    assert np.array_equal(Wd != 0, np.abs(W2) >= thr)          # continuous data: no ties at the cut
