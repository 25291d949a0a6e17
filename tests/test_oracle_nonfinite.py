"""Pins for the ranking of non-finite computed scores (TVW, per-tile keep, BW).

"Accelerating Sparse DNNs Based on Tiled GEMM" (Abstract, Figure 3) ranks the
columns of a tile by importance and says nothing of weights that are NaN or
infinite.  The reading: a score (a sum of magnitudes) that is NaN ranks above
+Inf, every NaN score ties with every other, and ties go to the lower index.
NaN payloads are not part of the order: IEEE 754 does not fix the payload of
the NaN an addition returns, so two implementations may legally differ there.

The pins compare the oracle with a brute force written on Python floats
(math.isnan and ordinary comparisons, no bit patterns), on tiles whose NaN
weights carry different payloads, and check that the two plausible mistakes --
ranking by the raw bit pattern (NaN order by payload) and sorting by -score
(NaN last) -- both give a different answer on the same fixtures.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import prune24 as O


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# quiet NaNs with distinct payloads (one with the sign bit set)
NAN_SMALL = 0x7FC00001
NAN_MID = 0x7FC01000
NAN_BIG = 0x7FC7F000
NAN_NEG = 0xFFC00100
INF = 0x7F800000


def _better(sa, a, sb, b):
    """True if (score sa, index a) ranks before (score sb, index b) in the reading."""
    na, nb = math.isnan(sa), math.isnan(sb)
    if na and nb:
        return a < b
    if na != nb:
        return na
    return sa > sb or (sa == sb and a < b)


def _brute_keep(scores, keep):
    """The unique keep-subset whose every member ranks before every non-member."""
    n = len(scores)
    winners = [S for S in itertools.combinations(range(n), keep)
               if all(_better(scores[a], a, scores[b], b) for a in S for b in range(n) if b not in S)]
    assert len(winners) == 1
    return list(winners[0])


def _plant(W, where):
    for (r, c), bits in where.items():
        W[r, c] = _f32(bits)
    return W


def _fixture_nan_cut():
    """One 4-row tile, 16 columns: five NaN columns (payload largest at the highest
    column, smallest at the lowest), keep 4, so the cut falls among the NaN ties."""
    W = (np.arange(64, dtype=np.float32).reshape(4, 16) % 7 + 1) * 0.25
    return _plant(W, {(1, 2): NAN_SMALL, (0, 5): NAN_MID, (3, 9): NAN_NEG, (2, 12): NAN_BIG,
                      (1, 14): NAN_BIG, (0, 3): INF, (2, 3): INF})


def _fixture_nan_over_inf():
    """Two NaN columns and three +Inf columns (one +Inf column also holds a NaN), keep 4."""
    W = (np.arange(64, dtype=np.float32).reshape(4, 16) % 5 + 1) * 0.5
    return _plant(W, {(0, 1): INF, (3, 4): INF, (1, 7): INF, (2, 7): NAN_SMALL, (0, 11): NAN_BIG,
                      (3, 15): INF})


def _scores_f(W):
    # plain Python floats summed in row order; NaN/Inf arithmetic of floats
    return [sum(abs(float(W[m, k])) for m in range(W.shape[0])) for k in range(W.shape[1])]


@pytest.mark.parametrize("fixture", [_fixture_nan_cut, _fixture_nan_over_inf])
def test_tvw_select_matches_float_brute_force(fixture):
    W = fixture()
    with np.errstate(invalid="ignore"):
        kept = O.tvw_select(W, 4, 4)[0].tolist()
    assert kept == _brute_keep(_scores_f(W), 4)


def test_plausible_mistakes_fail():
    for fixture in (_fixture_nan_cut, _fixture_nan_over_inf):
        W = fixture()
        with np.errstate(invalid="ignore"):
            sc = O.tvw_scores(W, 4)[0]
            want = O.tvw_select(W, 4, 4)[0].tolist()
        # NaN last (argsort of -score)
        minus = sorted(np.argsort(-sc, kind="stable")[:4].tolist())
        assert minus != want
    # ordering by the raw bit pattern puts the big-payload NaNs first
    W = _fixture_nan_cut()
    with np.errstate(invalid="ignore"):
        sc = O.tvw_scores(W, 4)[0]
        want = O.tvw_select(W, 4, 4)[0].tolist()
    raw = sorted(np.argsort(np.iinfo(np.uint64).max - sc.view(np.uint64), kind="stable")[:4].tolist())
    assert raw != want
    assert want == [2, 5, 9, 12]


def test_payloads_really_differ_in_the_scores():
    # the fixture is only a pin if its NaN scores carry different bit patterns
    W = _fixture_nan_cut()
    with np.errstate(invalid="ignore"):
        sc = O.tvw_scores(W, 4)[0]
    nan_bits = {int(b) for b in sc.view(np.uint64)[np.isnan(sc)]}
    assert len(nan_bits) >= 3
    assert all(k == O.SCORE_NAN_KEY for k in O.score_key(sc)[np.isnan(sc)])


def test_var_counts_nan_tiles_rank_first():
    # 3 tiles of 128 rows, K = 128: tile 2 holds NaN columns, tile 0 holds +Inf columns
    rng = np.random.default_rng(11)
    W = rng.standard_normal((384, 128)).astype(np.float32) * 0.02
    for c in range(0, 128, 2):
        W[256 + (c % 128), c] = _f32(NAN_BIG if c % 4 else NAN_SMALL)
    for c in range(1, 40, 2):
        W[5, c] = _f32(INF)
    with np.errstate(invalid="ignore"):
        sc = O.tvw_scores(W, 128)
    T, K = sc.shape
    flat = [(float(sc[t, k]), t * K + k) for t in range(T) for k in range(K)]
    # rank every (tile, column) with the float comparator, by insertion
    ranked = []
    for s, f in flat:
        i = 0
        while i < len(ranked) and _better(ranked[i][0], ranked[i][1], s, f):
            i += 1
        ranked.insert(i, (s, f))
    for total in (64, 84, 100, 192):
        raw = [0] * T
        for _, f in ranked[:total]:
            raw[f // K] += 1
        want = [min(max(64 * ((c + 32) // 64), 64), K) for c in raw]
        with np.errstate(invalid="ignore"):
            got = O.tvw_var_counts(W, 128, total).tolist()
        assert got == want
    # the NaN tile's kept columns are exactly its NaN columns when its count is 64
    with np.errstate(invalid="ignore"):
        counts = O.tvw_var_counts(W, 128, 64)
        tiles = O.tvw_var_compress(W, 128, counts)
    assert counts.tolist()[2] == 64
    assert tiles[2][0].tolist() == list(range(0, 128, 2))


def test_bw_select_nan_and_inf_blocks():
    # 1 tile, K = 512: 8 blocks; NaN in blocks 6 and 2 (different payloads), +Inf in blocks 4 and 7
    rng = np.random.default_rng(12)
    W = np.abs(rng.standard_normal((128, 512))).astype(np.float32)
    W[3, 6 * 64 + 5] = _f32(NAN_BIG)
    W[9, 2 * 64 + 1] = _f32(NAN_SMALL)
    W[0, 4 * 64] = _f32(INF)
    W[1, 7 * 64 + 63] = _f32(INF)
    with np.errstate(invalid="ignore"):
        bs = O.bw_block_scores(W)[0]
        for keep in (1, 2, 3, 5):
            got = O.bw_select(W, keep)[0].reshape(keep, 64)[:, 0] // 64
            assert got.tolist() == _brute_keep([float(x) for x in bs], keep)
    with np.errstate(invalid="ignore"):
        assert (O.bw_select(W, 1)[0] // 64 == 2).all()       # NaN tie -> lower block
        assert sorted(set((O.bw_select(W, 3)[0] // 64).tolist())) == [2, 4, 6]
