"""Pins for the oracle's GEMM reference, bound and tolerance check.

The sparse product must equal the dense product of the pruned matrix (the
pages' premise that the zeros can be skipped: NVIDIA A100 sparsity blog page,
body text; "Accelerating Sparse Deep Neural Networks", Abstract).

Pins: a brute-force triple loop, two independent routes (dense library matmul
vs metadata-driven gather) agreeing to fp64 rounding, exact integer products,
X = identity returning the decompressed matrix, and planted mistakes (a dropped
term, a wrong position, a transposed operand) failing the tolerance check while
a correct fp32-accumulated product passes it.
"""
import numpy as np

from oracle import prune24 as O
from workloads import random_bf16, random_matrix, small_int_matrix


def _bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bruteforce_triple_loop():
    W = small_int_matrix((5, 8), seed=1)
    X = small_int_matrix((8, 3), seed=2)
    values, meta = O.compress_24(W, "f32")
    y, bnd = O.gemm_ref(O.decompress_24(values, meta, 8), _bits(X))
    P = O.prune_24(W, "f32")
    for m in range(5):
        for n in range(3):
            s = 0.0
            b = 0.0
            for k in range(8):
                s += float(P[m, k]) * float(X[k, n])
                b += abs(float(P[m, k])) * abs(float(X[k, n]))
            assert y[m, n] == s and bnd[m, n] == b


def test_two_routes_agree():
    M, K, N = 48, 512, 40
    W = random_matrix((M, K), seed=3, sigma=0.02)
    Xb = random_bf16((K, N), seed=4)
    values, meta = O.compress_24(W, "f32")
    y1, bnd = O.gemm_ref(O.decompress_24(values, meta, K), Xb)
    y2 = O.spmm_ref_sparse(values, meta, K, Xb)
    assert (np.abs(y1 - y2) <= K * 2.0 ** -53 * bnd).all()
    rows = np.array([0, 17, 47])
    y3, b3 = O.gemm_ref(O.decompress_24(values, meta, K), Xb, rows=rows)
    assert np.array_equal(y3, y1[rows]) and np.array_equal(b3, bnd[rows])


def test_integer_exact():
    M, K, N = 32, 256, 24
    W = small_int_matrix((M, K), seed=5)
    X = small_int_matrix((K, N), seed=6)
    values, meta = O.compress_24(W, "f32")
    y1, _ = O.gemm_ref(O.decompress_24(values, meta, K), _bits(X))
    y2 = O.spmm_ref_sparse(values, meta, K, _bits(X))
    exact = O.prune_24(W, "f32").astype(np.int64) @ X.astype(np.int64)
    assert np.array_equal(y1, exact) and np.array_equal(y2, exact)


def test_identity_returns_decompressed():
    K = 128
    W = random_matrix((16, K), seed=7)
    values, meta = O.compress_24(W, "f32")
    I = _bits(np.eye(K, dtype=np.float32))
    y, _ = O.gemm_ref(O.decompress_24(values, meta, K), I)
    assert np.array_equal(y, O.bf16_to_f64(O.decompress_24(values, meta, K)))


def test_tolerance_accepts_fp32_accumulation_and_rejects_planted_mistakes():
    M, K, N = 64, 768, 64
    W = random_matrix((M, K), seed=8, sigma=0.02)
    Xb = random_bf16((K, N), seed=9)
    values, meta = O.compress_24(W, "f32")
    Wd = O.decompress_24(values, meta, K)
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    # a correct fp32-accumulating product, sequential in k (worst common order)
    Wf, Xf = O.bf16_to_f32(Wd), O.bf16_to_f32(Xb)
    acc = np.zeros((M, N), dtype=np.float32)
    for k in range(K):
        acc += np.outer(Wf[:, k], Xf[k]).astype(np.float32)
    assert O.check(acc, y_ref, bnd, "f32")[0]
    # its bf16 rounding passes the bf16 bound
    assert O.check(O.bf16_to_f64(O.bf16_rne(acc)), y_ref, bnd, "bf16")[0]
    # planted mistake 1: one kept value dropped
    v_bad = values.copy(); v_bad[5, 100] = 0
    yb, _ = O.gemm_ref(O.decompress_24(v_bad, meta, K), Xb)
    assert not O.check(yb, y_ref, bnd, "f32")[0]
    # planted mistake 2: one position index wrong (first group of row 3 shifted)
    pos = O.meta_positions(meta, K)
    m_bad = meta.copy()
    old = int(pos[3, 0]); new = next(p for p in range(4) if p != old and p != pos[3, 1])
    m_bad[3, 0] = (int(meta[3, 0]) & ~3) | new
    yb, _ = O.gemm_ref(O.decompress_24(values, m_bad, K), Xb)
    assert not O.check(yb, y_ref, bnd, "f32")[0]
    # planted mistake 3: transposed operand (square case)
    Ws = random_matrix((64, 64), seed=10)
    Xs = random_bf16((64, 64), seed=11)
    vs, ms = O.compress_24(Ws, "f32")
    yr, br = O.gemm_ref(O.decompress_24(vs, ms, 64), Xs)
    yt, _ = O.gemm_ref(O.decompress_24(vs, ms, 64), Xs.T.copy())
    assert not O.check(yt, yr, br, "f32")[0]
    # planted mistake 4: sign flip of one value
    v_bad = values.copy(); v_bad[0, 0] ^= 0x8000
    yb, _ = O.gemm_ref(O.decompress_24(v_bad, meta, K), Xb)
    assert not O.check(yb, y_ref, bnd, "f32")[0]
    # non-finite output fails
    y_nan = y_ref.copy(); y_nan[0, 0] = np.nan
    assert not O.check(y_nan, y_ref, bnd, "f32")[0]
