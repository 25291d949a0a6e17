"""Pins for the oracle's two-layer chain (layer 1 2:4 with a fused epilogue, its
output stored as bf16, layer 2 TVW): "Accelerating Sparse DNNs Based on Tiled
GEMM", TL;DR (kernel fusion).

Pins: a brute-force loop on integer data where every value is exact; the chain
with W2 = I reducing to layer 1's result plus a bias and activation; the
tolerance admitting the bf16-rounded intermediate computed the plain way and
rejecting planted mistakes (bias dropped, activation skipped, W2 transposed,
intermediate not rounded vs a wrong activation)."""
import numpy as np

from oracle import prune24 as O
from workloads import random_bf16, random_matrix, small_int_matrix


def _layers(M1, K1, M2, N, seed, sigma=0.05):
    W1 = random_matrix((M1, K1), seed=seed, sigma=sigma)
    v1, m1 = O.compress_24(W1, "f32")
    W1d = O.decompress_24(v1, m1, K1)
    W2 = random_matrix((M2, M1), seed=seed + 1, sigma=sigma)
    kept, v2, m2 = O.tvw_compress(W2, 128, M1 // 2)
    W2d = O.tvw_decompress(kept, v2, m2, M2, M1, 128)
    X = random_bf16((K1, N), seed=seed + 2)
    b1 = (0.1 * np.random.default_rng(seed + 3).standard_normal(M1)).astype(np.float32)
    b2 = (0.1 * np.random.default_rng(seed + 4).standard_normal(M2)).astype(np.float32)
    return W1d, W2d, X, b1, b2


def test_integer_chain_is_exact_against_a_loop():
    M1, K1, M2, N = 8, 16, 6, 5
    W1 = small_int_matrix((M1, K1), seed=1, lo=-3, hi=3)
    W1d = O.decompress_24(*O.compress_24(W1, "f32"), K1)
    W2d = O.bf16_rne(small_int_matrix((M2, M1), seed=2, lo=-3, hi=3))
    X = O.bf16_rne(small_int_matrix((K1, N), seed=3, lo=-3, hi=3))
    b1 = np.arange(M1, dtype=np.float32) - 4
    b2 = np.arange(M2, dtype=np.float32) - 2
    y2, z2, bnd2, carried = O.chain_ref(W1d, X, b1, O.ACT_RELU, W2d, b2, O.ACT_NONE)
    w1, w2, x = O.bf16_to_f64(W1d), O.bf16_to_f64(W2d), O.bf16_to_f64(X)
    for i in range(M2):
        for n in range(N):
            acc = float(b2[i])
            for j in range(M1):
                h = sum(w1[j, k] * x[k, n] for k in range(K1)) + float(b1[j])
                acc += w2[i, j] * max(h, 0.0)
            assert y2[i, n] == acc and z2[i, n] == acc
    assert (carried >= 0).all() and (bnd2 >= np.abs(w2) @ np.abs(np.maximum(w1 @ x + b1[:, None], 0))).all()


def test_identity_second_layer_reduces_to_layer_one():
    M1, K1, N = 128, 64, 40
    W1d, _, X, b1, b2 = _layers(M1, K1, 128, N, seed=10)
    I = O.bf16_rne(np.eye(M1, dtype=np.float32))
    y2, z2, _, _ = O.chain_ref(W1d, X, b1, O.ACT_GELU, I, b2[:M1], O.ACT_RELU)
    h, _, _ = O.fused_ref(W1d, X, b1, O.ACT_GELU)
    assert np.allclose(z2, h + b2[:M1, None].astype(np.float64), rtol=0, atol=1e-12)
    assert np.array_equal(y2, O.act_ref(z2, O.ACT_RELU))


def _plain_chain(W1d, X, b1, act1, W2d, b2, act2, round_h=True):
    """The chain as a caller would compute it: layer 1 in fp32, H rounded to bf16, layer 2 in fp32."""
    w1 = O.bf16_to_f64(W1d).astype(np.float32)
    x = O.bf16_to_f64(X).astype(np.float32)
    h = O.act_ref((w1 @ x).astype(np.float64) + b1.astype(np.float64)[:, None], act1).astype(np.float32)
    if round_h:
        h = O.bf16_to_f64(O.bf16_rne(h)).astype(np.float32)
    w2 = O.bf16_to_f64(W2d).astype(np.float32)
    return O.act_ref((w2 @ h).astype(np.float64) + b2.astype(np.float64)[:, None], act2)


def test_tolerance_admits_the_plain_chain_and_rejects_mistakes():
    W1d, W2d, X, b1, b2 = _layers(256, 128, 256, 96, seed=20)
    for act1, act2 in ((O.ACT_GELU, O.ACT_NONE), (O.ACT_RELU, O.ACT_GELU)):
        ref = O.chain_ref(W1d, X, b1, act1, W2d, b2, act2)
        good = _plain_chain(W1d, X, b1, act1, W2d, b2, act2)
        for out in ("f32", "bf16"):
            ok, worst = O.check_chain(good, *ref, act2, out)
            assert ok, (act1, act2, out, worst)
        bad = {
            "bias2 dropped": _plain_chain(W1d, X, b1, act1, W2d, np.zeros_like(b2), act2),
            "bias1 dropped": _plain_chain(W1d, X, np.zeros_like(b1), act1, W2d, b2, act2),
            "act1 skipped": _plain_chain(W1d, X, b1, O.ACT_NONE, W2d, b2, act2),
            "W2 transposed": _plain_chain(W1d, X, b1, act1, np.ascontiguousarray(W2d.T), b2, act2),
        }
        for name, y in bad.items():
            assert not O.check_chain(y, *ref, act2, "f32")[0], name


def test_carried_bound_covers_the_rounding_of_h():
    """|bf16(h) - h| never exceeds layer 1's bf16 tolerance, so the carried term covers it."""
    W1d, _, X, b1, _ = _layers(256, 128, 128, 200, seed=30)
    for act in (O.ACT_NONE, O.ACT_RELU, O.ACT_GELU):
        h, z, bnd = O.fused_ref(W1d, X, b1, act)
        hr = O.bf16_to_f64(O.bf16_rne(h.astype(np.float32)))
        assert (np.abs(hr - h) <= O.fused_tolerance(h, z, bnd, act, "bf16")).all()
