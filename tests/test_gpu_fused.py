"""GPU parity for the fused products: Y = act(W X + b) with the bias add and
activation run in the GEMM kernel's epilogue (spmm24 / spmm24_xt, the TVW
products, and TW alone on the dense MFMA).

Every result is checked elementwise against the oracle's fp64 act(W X + b)
within ``oracle.prune24.fused_tolerance``; with no bias and no activation the
fused call must reproduce the plain product bit for bit.
"""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu

ACTS = {"none": O.ACT_NONE, "relu": O.ACT_RELU, "gelu": O.ACT_GELU}


def _run(W, Xb, bias, act, out, order):
    c = p24.compress(f32_dev(W))
    dt = torch.float32 if out == "f32" else torch.bfloat16
    b = None if bias is None else torch.from_numpy(bias).cuda()
    if order == "kn":
        Y = p24.spmm24(c, bf16_dev(Xb, pad_cols=(-Xb.shape[1]) % 8), out_dtype=dt, bias=b, act=act)
    else:
        Y = p24.spmm24_xt(c, bf16_dev(np.ascontiguousarray(Xb.T)), out_dtype=dt, bias=b, act=act)
    torch.cuda.synchronize()
    return c, Y


def _check(Y, W, Xb, bias, act, out):
    v, m = O.compress_24(W, "f32")
    y_ref, z_ref, bnd = O.fused_ref(O.decompress_24(v, m, W.shape[1]), Xb, bias, ACTS[act])
    ok, worst = O.check_fused(y_host(Y), y_ref, z_ref, bnd, ACTS[act], out)
    assert ok, f"worst err/tol {worst}"


@pytest.mark.parametrize("M,K,N", [(300, 256, 200), (96, 128, 72), (257, 192, 1001)])
@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("order", ["kn", "nk"])
def test_fused_parity(M, K, N, act, with_bias, out, order):
    need_gpu()
    print(f"[fused] {M}x{K}x{N} {act} bias={with_bias} {out} {order}", flush=True)
    W = workloads.random_matrix((M, K), seed=M + 3 * K, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 11)
    bias = np.random.default_rng(M).standard_normal(M).astype(np.float32) if with_bias else None
    _, Y = _run(W, Xb, bias, act, out, order)
    _check(Y, W, Xb, bias, act, out)


@pytest.mark.parametrize("order", ["kn", "nk"])
def test_fused_noop_is_plain_product(order):
    need_gpu()
    M, K, N = 544, 320, 600
    W = workloads.random_matrix((M, K), seed=31, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=32)
    c = p24.compress(f32_dev(W))
    if order == "kn":
        X = bf16_dev(Xb)
        Y1 = p24.spmm24(c, X, out_dtype=torch.float32)
        Y2 = torch.empty_like(Y1)
        p24.lib().spmm24_fused(p24._ptr(c.values), p24._ptr(c.meta), c.layout, M, K, p24._ptr(X), N, 0, N,
                               p24._ptr(Y2), 0, N, None, 0, p24._stream(X.device))
    else:
        XT = bf16_dev(np.ascontiguousarray(Xb.T))
        Y1 = p24.spmm24_xt(c, XT, out_dtype=torch.float32)
        Y2 = torch.empty_like(Y1)
        p24.lib().spmm24_fused(p24._ptr(c.values), p24._ptr(c.meta), c.layout, M, K, p24._ptr(XT), K, 1, N,
                               p24._ptr(Y2), 0, N, None, 0, p24._stream(XT.device))
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


@pytest.mark.parametrize("tile", ["256x256", "192x256", "128x256", "128x128", "64x128"])
def test_fused_every_tile(tile, monkeypatch):
    need_gpu()
    monkeypatch.setenv("P24_TILE", tile)
    M, K, N = 544, 320, 600
    W = workloads.random_matrix((M, K), seed=41, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=42)
    bias = np.random.default_rng(43).standard_normal(M).astype(np.float32)
    _, Y = _run(W, Xb, bias, "gelu", "f32", "kn")
    _check(Y, W, Xb, bias, "gelu", "f32")


@pytest.mark.parametrize("key,act", [("c2", "gelu"), ("c3a", "relu"), ("c3b", "relu")])
def test_fused_workloads(key, act):
    """The pages' layer shapes with their usual epilogue: BERT FFN up-projection
    + GELU, ResNet-50 convolutions + ReLU; bias ~ N(0, 0.1^2)."""
    need_gpu()
    wl = workloads.WORKLOADS[key]
    print(f"[fused] {key} {act}", flush=True)
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    bias = (0.1 * np.random.default_rng(7).standard_normal(wl.M)).astype(np.float32)
    _, Y = _run(W, Xb, bias, act, "bf16", "kn")
    _check(Y, W, Xb, bias, act, "bf16")
    if act == "relu":
        assert (Y >= 0).all().item()


def test_gelu_activation_sweep():
    """W = 0 makes every output exactly act(bias): the activation alone, over a
    dense sweep of [-12, 12] (the bound term of the tolerance is zero here)."""
    need_gpu()
    M, K, N = 8192, 64, 16
    W = np.zeros((M, K), dtype=np.float32)
    Xb = workloads.random_bf16((K, N), seed=3)
    bias = np.linspace(-12.0, 12.0, M).astype(np.float32)
    for act in ("gelu", "relu"):
        _, Y = _run(W, Xb, bias, act, "f32", "kn")
        y_ref, z_ref, bnd = O.fused_ref(np.zeros((M, K), dtype=np.uint16), Xb, bias, ACTS[act])
        assert not bnd.any()
        ok, worst = O.check_fused(y_host(Y), y_ref, z_ref, bnd, ACTS[act], "f32")
        assert ok, f"{act}: worst err/tol {worst}"


@pytest.mark.parametrize("var,tile", [(False, "128x256"), (False, "128x512"), (True, None)])
@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_tvw_fused_parity(var, tile, act, out, monkeypatch):
    """The TVW products with the fused epilogue (fixed keep at both block widths, and
    per-tile keep), ragged M and N."""
    need_gpu()
    if tile:
        monkeypatch.setenv("P24_GATHER_TILE", tile)
    M, K, N = 300, 512, 1000
    print(f"[fused] tvw var={var} tile={tile} {act} {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=41, sigma=0.05)
    W[:128] *= 1.2
    Xb = workloads.random_bf16((K, N), seed=42)
    bias = np.random.default_rng(43).standard_normal(M).astype(np.float32)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    b = torch.from_numpy(bias).cuda()
    X = bf16_dev(Xb)
    if var:
        t = p24.tvw_var_compress(f32_dev(W), total_keep=3 * 256)
        Y = p24.spmm_tvw_var(t, X, out_dtype=dt, bias=b, act=act)
        Yp = p24.spmm_tvw_var(t, X, out_dtype=dt)
        counts = O.tvw_var_counts(W, 128, 3 * 256)
        Wd = O.tvw_var_decompress(O.tvw_var_compress(W, 128, counts), M, K, 128)
    else:
        t = p24.tvw_compress(f32_dev(W), tile_m=128, keep_k=256)
        Y = p24.spmm_tvw(t, X, out_dtype=dt, bias=b, act=act)
        Yp = p24.spmm_tvw(t, X, out_dtype=dt)
        kept, v, m = O.tvw_compress(W, 128, 256)
        Wd = O.tvw_decompress(kept, v, m, M, K, 128)
    torch.cuda.synchronize()
    y_ref, z_ref, bnd = O.fused_ref(Wd, Xb, bias, ACTS[act], rows=None)
    ok, worst = O.check_fused(y_host(Y), y_ref, z_ref, bnd, ACTS[act], out)
    assert ok, f"worst err/tol {worst}"
    # no bias and no activation: the fused kernel reproduces the plain product bit for bit
    Yn = (p24.spmm_tvw_var(t, X, out_dtype=dt, bias=torch.zeros_like(b)) if var
          else p24.spmm_tvw(t, X, out_dtype=dt, bias=torch.zeros_like(b)))
    torch.cuda.synchronize()
    assert torch.equal(Yn, Yp)


@pytest.mark.parametrize("var,tile", [(False, "128x256"), (False, "128x512"), (True, None)])
@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_tw_fused_parity(var, tile, act, out, monkeypatch):
    """TW alone (dense MFMA on the kept columns) with the fused epilogue, fixed keep at both
    block widths and per-tile keep, ragged M and N."""
    need_gpu()
    if tile:
        monkeypatch.setenv("P24_GATHER_TILE", tile)
    M, K, N = 300, 512, 1000
    print(f"[fused] tw var={var} tile={tile} {act} {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=51, sigma=0.05)
    W[128:256] *= 1.3
    Xb = workloads.random_bf16((K, N), seed=52)
    bias = np.random.default_rng(53).standard_normal(M).astype(np.float32)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    b = torch.from_numpy(bias).cuda()
    X = bf16_dev(Xb)
    if var:
        t = p24.tw_var_compress(f32_dev(W), total_keep=3 * 256)
        Y = p24.spmm_tw_var(t, X, out_dtype=dt, bias=b, act=act)
        Yp = p24.spmm_tw_var(t, X, out_dtype=dt)
        tiles = O.tw_var_compress(W, 128, O.tvw_var_counts(W, 128, 3 * 256))
        Wd = O.tw_decompress([k for k, _ in tiles], [w for _, w in tiles], M, K, 128)
    else:
        t = p24.tw_compress(f32_dev(W), tile_m=128, keep_k=256)
        Y = p24.spmm_tw(t, X, out_dtype=dt, bias=b, act=act)
        Yp = p24.spmm_tw(t, X, out_dtype=dt)
        kept, Wc = O.tw_compress(W, 128, 256)
        Wd = O.tw_decompress(list(kept), [Wc[128 * i:128 * i + 128] for i in range(kept.shape[0])], M, K, 128)
    torch.cuda.synchronize()
    y_ref, z_ref, bnd = O.fused_ref(Wd, Xb, bias, ACTS[act], rows=None)
    ok, worst = O.check_fused(y_host(Y), y_ref, z_ref, bnd, ACTS[act], out)
    assert ok, f"worst err/tol {worst}"
    # no bias and no activation: the fused kernel reproduces the plain product bit for bit
    Yn = (p24.spmm_tw_var(t, X, out_dtype=dt, bias=torch.zeros_like(b)) if var
          else p24.spmm_tw(t, X, out_dtype=dt, bias=torch.zeros_like(b)))
    torch.cuda.synchronize()
    assert torch.equal(Yn, Yp)
