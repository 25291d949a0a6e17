"""Pins for the TW (tile column drop, no 2:4) oracle and the dense device layout.

The kept columns follow the already-pinned TVW selection; the stored values
are each element's own bf16 rounding (checked element by element against the
pinned bf16_rne of a scalar); keeping every column reduces TW to the plain
bf16 cast of W; and the dense device layout, driven through a model of the
dense MFMA's lane semantics, reproduces the dense product exactly.
"""
import numpy as np
import pytest

import workloads
from mfma_models import mfma32x32x16_model
from oracle import prune24 as O


def test_tw_elements_brute_force():
    W = workloads.random_matrix((200, 64), seed=11, sigma=0.05)
    kept, Wc = O.tw_compress(W, 128, 32)
    assert np.array_equal(kept, O.tvw_select(W, 128, 32))
    for m in range(200):
        t = m // 128
        for j in range(32):
            assert Wc[m, j] == O.bf16_rne(np.float32(W[m, kept[t, j]]))


def test_tw_keep_all_is_plain_cast():
    W = workloads.random_matrix((256, 128), seed=12, sigma=0.05)
    kept, Wc = O.tw_compress(W, 128, 128)
    assert (kept == np.arange(128)).all()
    assert np.array_equal(Wc, O.bf16_rne(W))
    assert np.array_equal(O.tw_decompress(list(kept), [Wc[:128], Wc[128:]], 256, 128, 128), O.bf16_rne(W))


def test_tw_var_matches_tvw_columns_and_scatter():
    W = workloads.random_matrix((300, 256), seed=13, sigma=0.05)
    W[:128] *= 1.3
    counts = O.tvw_var_counts(W, 128, 300)
    tiles = O.tw_var_compress(W, 128, counts)
    tv = O.tvw_var_compress(W, 128, counts)
    Wd = O.tw_decompress([k for k, _ in tiles], [w for _, w in tiles], 300, 256, 128)
    for t, ((k, w), (k2, _, _)) in enumerate(zip(tiles, tv)):
        assert np.array_equal(k, k2)
        r0, r1 = 128 * t, min(300, 128 * t + 128)
        dropped = np.setdiff1d(np.arange(256), k)
        assert not Wd[r0:r1][:, dropped].any()
        assert np.array_equal(Wd[r0:r1][:, k], O.bf16_rne(W[r0:r1][:, k]))
    kept, dv = O.tw_var_device(tiles, counts)
    assert kept.size == dv.size // 128 == counts.sum()


def test_dense_layout_through_instruction_model():
    M, K, N = 40, 64, 32
    Wb = workloads.truncate_to_bf16_bits(workloads.small_int_matrix((M, K), seed=14))
    Xb = workloads.truncate_to_bf16_bits(workloads.small_int_matrix((K, N), seed=15))
    dv = O.bf16_to_f64(O.dense_device_layout(Wb, 64).reshape(2, K // 16, 64, 8))
    Xf = O.bf16_to_f64(Xb)
    Y = np.zeros((64, N))
    for rb in range(2):
        acc = np.zeros((64, 16))
        for s in range(K // 16):
            b = np.array([Xf[16 * s + 8 * (L // 32): 16 * s + 8 * (L // 32) + 8, L % 32] for L in range(64)])
            acc = mfma32x32x16_model(dv[rb, s], b, acc)
        for lo in range(64):
            for i in range(16):
                Y[32 * rb + 8 * (i // 4) + 4 * (lo // 32) + i % 4, lo % 32] = acc[lo, i]
    y_ref, _ = O.gemm_ref(Wb, Xb)
    assert np.array_equal(Y[:M], y_ref)
    assert not Y[M:].any()


def test_dense_layout_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.dense_device_layout(np.zeros((40, 64), np.uint16), 32)
    with pytest.raises(ValueError):
        O.dense_device_layout(np.zeros((32, 24), np.uint16), 32)
