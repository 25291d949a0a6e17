"""Pins for the oracle's fused epilogue (bias + activation) and its tolerance.

The activation values are fixed by closed forms and by the normal CDF's known
values; the fused result by a brute-force loop; the GELU slope bound by a dense
numerical scan; the tolerance by planted mistakes it must reject.
"""
import math

import numpy as np

import workloads
from oracle import prune24 as O


def test_relu_closed_form():
    z = np.array([-2.0, -0.0, 0.0, 1e-30, 3.5, np.inf, -np.inf, np.nan])
    assert np.array_equal(O.act_ref(z, O.ACT_RELU), np.array([0, 0, 0, 1e-30, 3.5, np.inf, 0, 0.0]))


def test_gelu_known_values():
    # z * Phi(z); Phi(1) = 0.8413447460685429, Phi(-1) = 1 - Phi(1), Phi(2) = 0.9772498680518208
    g = O.act_ref(np.array([0.0, 1.0, -1.0, 2.0, 40.0, -40.0]), O.ACT_GELU)
    ref = [0.0, 0.8413447460685429, -0.15865525393145707, 2 * 0.9772498680518208, 40.0, -0.0]
    assert np.allclose(g, ref, rtol=1e-15, atol=1e-300)
    # against the textbook integral of the normal density (midpoint rule, fine grid)
    for z in (-3.0, -0.5, 0.25, 1.7):
        t = np.linspace(-12.0, z, 400001)
        mid = 0.5 * (t[1:] + t[:-1])
        phi = np.sum(np.exp(-mid * mid / 2.0)) * (t[1] - t[0]) / math.sqrt(2.0 * math.pi)
        assert abs(O.act_ref(np.array([z]), O.ACT_GELU)[0] - z * phi) < 1e-9


def test_gelu_lipschitz_constant():
    z = np.linspace(-10.0, 10.0, 2000001)
    g = O.act_ref(z, O.ACT_GELU)
    slope = np.abs(np.diff(g) / np.diff(z))
    assert 1.128 < slope.max() <= O.GELU_LIPSCHITZ


def test_fused_brute_force():
    rng = np.random.default_rng(5)
    M, K, N = 6, 8, 5
    Wb = workloads.truncate_to_bf16_bits(workloads.random_matrix((M, K), seed=6))
    Xb = workloads.truncate_to_bf16_bits(workloads.random_matrix((K, N), seed=7))
    bias = rng.standard_normal(M).astype(np.float32)
    Wf, Xf = O.bf16_to_f64(Wb), O.bf16_to_f64(Xb)
    for act in (O.ACT_NONE, O.ACT_RELU, O.ACT_GELU):
        y, z, bnd = O.fused_ref(Wb, Xb, bias, act)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += Wf[m, k] * Xf[k, n]
                zz = acc + float(bias[m])
                assert abs(z[m, n] - zz) <= 1e-12 * (1 + abs(zz))
                if act == O.ACT_RELU:
                    want = zz if zz > 0 else 0.0
                elif act == O.ACT_GELU:
                    want = 0.5 * zz * (1.0 + math.erf(zz / math.sqrt(2.0)))
                else:
                    want = zz
                assert abs(y[m, n] - want) <= 1e-12 * (1 + abs(want))
    # rows selection and no-bias agree with the full computation
    y_all, _, _ = O.fused_ref(Wb, Xb, None, O.ACT_RELU)
    y_sel, _, _ = O.fused_ref(Wb, Xb, None, O.ACT_RELU, rows=[1, 4])
    assert np.array_equal(y_all[[1, 4]], y_sel)


def test_fused_tolerance_rejects_planted_mistakes():
    M, K, N = 64, 128, 48
    W = workloads.random_matrix((M, K), seed=8, sigma=0.1)
    v, m = O.compress_24(W, "f32")
    Wd = O.decompress_24(v, m, K)
    Xb = workloads.random_bf16((K, N), seed=9)
    bias = np.random.default_rng(10).standard_normal(M).astype(np.float32)
    for act in (O.ACT_RELU, O.ACT_GELU):
        y, z, bnd = O.fused_ref(Wd, Xb, bias, act)
        # the exact result and its fp32 / bf16 roundings pass
        assert O.check_fused(y.astype(np.float32), y, z, bnd, act, "f32")[0]
        assert O.check_fused(O.bf16_to_f64(O.bf16_rne(y.astype(np.float32))), y, z, bnd, act, "bf16")[0]
        # bias dropped, bias on the wrong axis, activation skipped, wrong activation: all rejected
        y_nob, _, _ = O.fused_ref(Wd, Xb, None, act)
        assert not O.check_fused(y_nob, y, z, bnd, act, "f32")[0]
        y_col = O.act_ref(z - bias[:, None] + bias[:N][None, :], act)
        assert not O.check_fused(y_col, y, z, bnd, act, "f32")[0]
        assert not O.check_fused(z, y, z, bnd, act, "f32")[0]
        other = O.ACT_GELU if act == O.ACT_RELU else O.ACT_RELU
        assert not O.check_fused(O.act_ref(z, other), y, z, bnd, act, "f32")[0]
