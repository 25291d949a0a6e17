"""GPU parity for TW alone (tile column drop, kept columns dense): the kept
lists and the dense operand bit-exact against the oracle, spmm_tw /
spmm_tw_var within the GEMM tolerance; fixed and per-tile keep counts."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, u16_host, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _scaled(M, K, seed, spread=0.1):
    W = workloads.random_matrix((M, K), seed=seed, sigma=0.02)
    T = -(-M // 128)
    s = 1.0 + spread * np.random.default_rng(seed + 1).uniform(-1, 1, T)
    return (W * s.astype(np.float32)[np.arange(M) // 128][:, None]).astype(np.float32)


def _compare_fixed(W, tile, keep):
    M, K = W.shape
    print(f"[tw] compress M={M} K={K} tile={tile} keep={keep}", flush=True)
    t = p24.tw_compress(f32_dev(W), tile_m=tile, keep_k=keep)
    torch.cuda.synchronize()
    kept, Wc = O.tw_compress(W, tile, keep)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    dv = O.dense_device_layout(Wc, -(-M // 32) * 32)
    assert np.array_equal(u16_host(t.Wp)[:dv.size], dv)
    return t, kept, Wc


def _compare_var(W, total):
    M, K = W.shape
    print(f"[tw_var] compress M={M} K={K} total={total}", flush=True)
    t = p24.tw_var_compress(f32_dev(W), total_keep=total)
    torch.cuda.synchronize()
    counts = O.tvw_var_counts(W, 128, total)
    tiles = O.tw_var_compress(W, 128, counts)
    kept, dv = O.tw_var_device(tiles, counts)
    off = np.concatenate([[0], np.cumsum(counts)])
    assert np.array_equal(t.offsets.cpu().numpy(), off)
    assert np.array_equal(t.order.cpu().numpy(), O.tvw_var_order(counts))
    assert np.array_equal(t.kept.cpu().numpy()[:kept.size], kept)
    assert np.array_equal(u16_host(t.Wp)[:dv.size], dv)
    return t, counts, tiles


@pytest.mark.parametrize("M,K,tile,keep", [
    (256, 256, 128, 128),
    (300, 256, 128, 64),      # partial last tile, rows padded to 32
    (200, 320, 32, 192),      # small tiles (compress only)
    (128, 2304, 128, 1152),
])
def test_tw_compress(M, K, tile, keep):
    need_gpu()
    _compare_fixed(workloads.random_matrix((M, K), seed=M + K + keep, sigma=0.02), tile, keep)


@pytest.mark.parametrize("M,K,N,keep", [(256, 256, 200, 128), (384, 512, 1000, 256), (300, 256, 72, 192),
                                         (256, 256, 1096, 128)])
@pytest.mark.parametrize("tile", ["128x256", "128x512"])
def test_spmm_tw_small(M, K, N, keep, tile, monkeypatch):
    """Both block widths of the fixed-keep gathered product, ragged N included."""
    need_gpu()
    monkeypatch.setenv("P24_GATHER_TILE", tile)
    W = workloads.random_matrix((M, K), seed=N + keep, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N)
    t, kept, Wc = _compare_fixed(W, 128, keep)
    print(f"[tw] spmm M={M} K={K} N={N} keep={keep}", flush=True)
    Y = p24.spmm_tw(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    T = kept.shape[0]
    Wd = O.tw_decompress(list(kept), [Wc[128 * i:128 * i + 128] for i in range(T)], M, K, 128)
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.parametrize("M,K,N,keep", [(512, 512, 600, 256), (400, 256, 264, 128)])
@pytest.mark.parametrize("tile", ["128x256", "128x512"])
def test_spmm_tw_tall_tiles(M, K, N, keep, tile, monkeypatch):
    """TW tiles of 256 output rows (two 128-row block rows per kept list; ragged last tile in
    the second case), at both block widths."""
    need_gpu()
    monkeypatch.setenv("P24_GATHER_TILE", tile)
    W = workloads.random_matrix((M, K), seed=M + N + 1, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 8)
    t, kept, Wc = _compare_fixed(W, 256, keep)
    print(f"[tw] tall tiles spmm M={M} K={K} N={N} keep={keep} tile={tile}", flush=True)
    Y = p24.spmm_tw(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    T = kept.shape[0]
    Wd = O.tw_decompress(list(kept), [Wc[256 * i:256 * i + 256] for i in range(T)], M, K, 256)
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


def test_tw_keep_all_equals_dense():
    """Keeping every column is the dense product of the bf16 cast, bit for bit."""
    need_gpu()
    M, K, N = 256, 256, 128
    W = workloads.random_matrix((M, K), seed=31, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=32)
    Wt = f32_dev(W)
    t = p24.tw_compress(Wt, tile_m=128, keep_k=K)
    X = bf16_dev(Xb)
    Yt = p24.spmm_tw(t, X, out_dtype=torch.float32)
    Wp = p24.pack_dense(bf16_dev(O.bf16_rne(W)))
    Yd = p24.gemm_bf16(Wp, M, K, X, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (t.kept.cpu().numpy() == np.arange(K)).all()
    assert torch.equal(Yt, Yd)


@pytest.mark.parametrize("M,K,frac,seed", [(256, 256, 0.5, 1), (300, 256, 0.5, 2), (1024, 512, 0.3, 3),
                                           (640, 320, 1.0, 4), (384, 128, 1.0 / 384, 5)])
def test_tw_var_compress(M, K, frac, seed):
    need_gpu()
    _compare_var(_scaled(M, K, seed), max(1, int(frac * -(-M // 128) * K)))


@pytest.mark.parametrize("M,K,N,frac", [(256, 256, 200, 0.5), (1000, 512, 1000, 0.4), (300, 256, 72, 0.7)])
def test_spmm_tw_var_small(M, K, N, frac):
    need_gpu()
    W = _scaled(M, K, M + N)
    Xb = workloads.random_bf16((K, N), seed=N)
    t, counts, tiles = _compare_var(W, int(frac * -(-M // 128) * K))
    print(f"[tw_var] spmm M={M} K={K} N={N}", flush=True)
    Y = p24.spmm_tw_var(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    Wd = O.tw_decompress([k for k, _ in tiles], [w for _, w in tiles], M, K, 128)
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.parametrize("var", [False, True])
def test_tw_c5_shape(var):
    """The TVW workload's shape and keep (fixed: c5, 2048 per tile; per tile: c5v's counts)."""
    need_gpu()
    wl = workloads.WORKLOADS["c5v" if var else "c5"]
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    if var:
        t, counts, tiles = _compare_var(W, wl.total_keep)
        Wd = O.tw_decompress([k for k, _ in tiles], [w for _, w in tiles], wl.M, wl.K, 128)
        run = lambda X, dt: p24.spmm_tw_var(t, X, out_dtype=dt)
    else:
        t, kept, Wc = _compare_fixed(W, wl.tile_m, wl.keep_k)
        Wd = O.tw_decompress(list(kept), [Wc[128 * i:128 * i + 128] for i in range(kept.shape[0])],
                             wl.M, wl.K, 128)
        run = lambda X, dt: p24.spmm_tw(t, X, out_dtype=dt)
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    X = bf16_dev(Xb)
    for out, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        print(f"[tw] {wl.key} spmm {out}", flush=True)
        Y = run(X, dt)
        torch.cuda.synchronize()
        ok, worst = O.check(y_host(Y), y_ref, bnd, out)
        assert ok, worst
