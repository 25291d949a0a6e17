"""Pins for the oracle's 2:4 magnitude selection and pruning.

The rule (NVIDIA A100 sparsity blog page, body text): in every contiguous run
of four weights along K at least two are zero; the pages' 2:4 pattern keeps
half ("Accelerating Sparse Deep Neural Networks", Abstract).  Criterion and tie
order are readings: magnitude, ties to the lower index.

Pins: brute force over the six pairs of every group, an exhaustive alphabet of
signed zeros / ties / Inf / NaN, the hand-worked fixture, idempotence, the
per-group nonzero bound and exact half density.
"""
import itertools

import numpy as np
import pytest

from oracle import prune24 as O
from workloads import random_matrix, small_int_matrix

PAIRS = list(itertools.combinations(range(4), 2))


def _brute_pair(keys):
    """The unique pair whose every member beats every dropped member under (key desc, idx asc)."""
    winners = []
    for p in PAIRS:
        drop = [i for i in range(4) if i not in p]
        beats = all((keys[a] > keys[b]) or (keys[a] == keys[b] and a < b) for a in p for b in drop)
        if beats:
            winners.append(p)
    assert len(winners) == 1
    return winners[0]


def test_bruteforce_random_groups():
    W = small_int_matrix((64, 256), seed=3, lo=-3, hi=3)     # many ties
    kept = O.select_24(W, "f32")
    key = O.magnitude_key(W, "f32").reshape(64, 64, 4)
    for m in range(64):
        for g in range(64):
            assert tuple(kept[m, g]) == _brute_pair([int(k) for k in key[m, g]])


def test_exhaustive_special_alphabet():
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, np.inf, np.nan], dtype=np.float32)
    tuples = np.array(list(itertools.product(range(8), repeat=4)))
    W = alphabet[tuples].reshape(1, -1)                          # 4096 groups in one row
    kept = O.select_24(W, "f32")[0]
    key = O.magnitude_key(W, "f32").reshape(-1, 4)
    for g in range(len(tuples)):
        assert tuple(kept[g]) == _brute_pair([int(k) for k in key[g]])
    # spot checks of the reading: NaN ranks above Inf, -0 ties +0, ties go low
    def pick(vals):
        return tuple(O.select_24(np.array([vals], dtype=np.float32), "f32")[0, 0])
    assert pick([np.inf, 1.0, np.nan, 2.0]) == (0, 2)
    assert pick([-0.0, 0.0, 0.0, -0.0]) == (0, 1)
    assert pick([1.0, -1.0, 1.0, -1.0]) == (0, 1)
    assert pick([0.0, 0.0, -5.0, 0.0]) == (0, 2)


def test_prune_properties_and_idempotence():
    W = random_matrix((96, 512), seed=5)
    P = O.prune_24(W, "f32")
    g = P.reshape(96, -1, 4)
    assert ((g != 0).sum(-1) <= 2).all()
    assert ((g != 0).sum(-1) == 2).all()                         # continuous data: exactly two survive
    assert (P != 0).mean() == 0.5
    # kept magnitudes dominate dropped ones in each group
    a = np.abs(W.reshape(96, -1, 4))
    kept_min = np.where(g != 0, a, np.inf).min(-1)
    drop_max = np.where(g == 0, a, -np.inf).max(-1)
    assert (kept_min >= drop_max).all()
    # kept entries are bit-identical, dropped become +0
    keep = P != 0
    assert np.array_equal(P[keep].view(np.uint32), W[keep].view(np.uint32))
    assert (P[~keep].view(np.uint32) == 0).all()
    assert np.array_equal(O.prune_24(P, "f32").view(np.uint32), P.view(np.uint32))


def test_bf16_input_mode_matches_f32_of_same_values():
    W32 = random_matrix((32, 128), seed=9)
    Wb = (W32.view(np.uint32) >> 16).astype(np.uint16)           # exact bf16 numbers
    Wf = (Wb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(O.select_24(Wb, "bf16"), O.select_24(Wf, "f32"))
    Pb = O.prune_24(Wb, "bf16")
    assert np.array_equal(O.prune_24(Pb, "bf16"), Pb)


def test_k_not_multiple_of_four_rejected():
    with pytest.raises(ValueError):
        O.select_24(np.zeros((2, 6), np.float32), "f32")


def test_hand_example_positions(golden):
    ex = golden["prune24"]
    W = np.array(ex["W"], dtype=np.float32)
    assert O.select_24(W, "f32").tolist() == ex["positions"]
