"""Pins for the oracle's compressed representation (values + 2-bit positions).

The pages name a compressed form with low metadata overhead (NVIDIA A100
sparsity blog page, Figure 1, whose drawing is missing); the bit layout is a
reading: value s's in-group position at bits [2s, 2s+2) of the row's bit stream.

Pins: hand-worked fixture, closed-form sizes, legal nibble alphabet,
decompress(compress(W)) == bf16(prune(W)) bitwise, the device layout as a
bijection, and the device layout driven through a lane-level model of the
gfx950 sparse MFMA (whose lane map was measured on the hardware) reproducing
the dense product exactly on integer data.
"""
import numpy as np
import pytest

from oracle import prune24 as O
from mfma_models import smfmac32_model
from workloads import random_matrix, small_int_matrix

LEGAL_NIBBLES = {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}


def test_hand_example(golden):
    ex = golden["prune24"]
    W = np.array(ex["W"], dtype=np.float32)
    values, meta = O.compress_24(W, "f32")
    assert [[f"{v:04X}" for v in row] for row in values] == ex["values_bf16_hex"]
    assert [f"{int(w):08X}" for w in meta[:, 0]] == ex["meta_hex"]
    X = np.array(ex["X"], dtype=np.float32)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)
    y, bnd = O.gemm_ref(O.decompress_24(values, meta, 8), Xb)
    assert y.tolist() == ex["Y"]
    assert bnd[0, 0] == ex["bound_00"]
    ys = O.spmm_ref_sparse(values, meta, 8, Xb)
    assert ys.tolist() == ex["Y"]


@pytest.mark.parametrize("M,K", [(1, 4), (3, 12), (5, 32), (7, 36), (16, 100), (64, 768)])
def test_sizes_alphabet_roundtrip(M, K):
    W = random_matrix((M, K), seed=M * 1000 + K)
    values, meta = O.compress_24(W, "f32")
    assert values.shape == (M, K // 2) and values.dtype == np.uint16
    assert meta.shape == (M, (K + 31) // 32) and meta.dtype == np.uint32
    # metadata is 2 bits per kept value = 1/8 byte per dense element
    assert values.nbytes + (M * K) // 8 == M * K * 2 * 9 // 16
    nib = np.array([(meta[:, g // 8] >> (4 * (g % 8))) & 0xF for g in range(K // 4)]).T
    assert set(np.unique(nib).tolist()) <= LEGAL_NIBBLES
    if K % 32:
        used_bits = K % 32                                   # (K % 32) / 2 values x 2 bits
        assert (meta[:, -1] >> np.uint32(used_bits) == 0).all()
    dec = O.decompress_24(values, meta, K)
    assert np.array_equal(dec, O.bf16_rne(O.prune_24(W, "f32")))


def test_bf16_input_compress_copies_bits():
    Wb = (random_matrix((8, 64), seed=2).view(np.uint32) >> 16).astype(np.uint16)
    values, meta = O.compress_24(Wb, "bf16")
    assert np.array_equal(O.decompress_24(values, meta, 64), O.prune_24(Wb, "bf16"))


@pytest.mark.parametrize("M,K", [(32, 64), (45, 128), (96, 256)])
def test_device_layout_bijection(M, K):
    W = random_matrix((M, K), seed=K + M)
    values, meta = O.compress_24(W, "f32")
    dv, dm = O.to_device_layout(values, meta, K)
    Mp = O.device_rows(M)
    assert dv.size == Mp * K // 2
    assert dm.size == (Mp // 32) * (K // 64) * 64
    v2, m2 = O.from_device_layout(dv, dm, M, K)
    assert np.array_equal(v2, values) and np.array_equal(m2, meta)
    # padded rows: zero values and position pattern 0x4 per group
    rows_pad = Mp - M
    if rows_pad:
        full_v, full_m = O.from_device_layout(dv, dm, Mp, K)
        assert (full_v[M:] == 0).all()
        assert (full_m[M:] == 0x44444444).all()


# ---- lane-level model of v_smfmac_f32_32x32x32_bf16: tests/mfma_models.py ----
def test_device_layout_through_instruction_model():
    M, K, N = 64, 128, 32
    W = small_int_matrix((M, K), seed=21)
    X = small_int_matrix((K, N), seed=22)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)
    values, meta = O.compress_24(W, "f32")
    dv, dm = O.to_device_layout(values, meta, K)
    RB, S, T = O.device_rows(M) // 32, K // 32, K // 64
    dv = O.bf16_to_f64(dv.reshape(RB, S, 64, 8))
    dm = dm.reshape(RB // 4, T, 4, 64).transpose(0, 2, 1, 3).reshape(RB, T, 64)   # [rb // 4, t, rb % 4, L]
    Xf = O.bf16_to_f64(Xb)
    Y = np.zeros((RB * 32, N))
    for rb in range(RB):
        acc = np.zeros((64, 16))
        for s in range(S):
            b = np.zeros((64, 16))
            for lb in range(64):
                n, h = lb % 32, lb // 32
                for e in range(16):
                    k = 8 * h + e if e < 8 else 16 + 8 * h + (e - 8)
                    b[lb, e] = Xf[32 * s + k, n]
            acc = smfmac32_model(dv[rb, s], b, dm[rb, s // 2], s % 2, acc)
        for lo in range(64):
            for i in range(16):
                Y[32 * rb + 8 * (i // 4) + 4 * (lo // 32) + i % 4, lo % 32] = acc[lo, i]
    y_ref, _ = O.gemm_ref(O.decompress_24(values, meta, K), Xb)
    assert np.array_equal(Y[:M], y_ref)
    assert not Y[M:].any()          # padded rows: zero values
