"""GPU parity for TVW with per-tile keep counts: the plan (offsets, batching
order), the kept lists and the compressed storage bit-exact against the
oracle; spmm_tvw_var within the GEMM tolerance."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, u16_host, u32_host, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _scaled(M, K, seed, spread=0.1):
    W = workloads.random_matrix((M, K), seed=seed, sigma=0.02)
    T = -(-M // 128)
    s = 1.0 + spread * np.random.default_rng(seed + 1).uniform(-1, 1, T)
    return (W * s.astype(np.float32)[np.arange(M) // 128][:, None]).astype(np.float32)


def _compare(W, total):
    M, K = W.shape
    print(f"[tvw_var] compress M={M} K={K} total={total}", flush=True)
    t = p24.tvw_var_compress(f32_dev(W), total_keep=total)
    torch.cuda.synchronize()
    counts = O.tvw_var_counts(W, 128, total)
    tiles = O.tvw_var_compress(W, 128, counts)
    kept, dv, dm, off = O.tvw_var_device(tiles, counts)
    assert np.array_equal(t.offsets.cpu().numpy(), off.astype(np.int64))
    assert np.array_equal(t.order.cpu().numpy(), O.tvw_var_order(counts))
    n = int(off[-1])
    assert np.array_equal(t.kept.cpu().numpy()[:n], kept)
    assert np.array_equal(u16_host(t.values)[:dv.size], dv)
    assert np.array_equal(u32_host(t.meta)[:dm.size], dm)
    return t, counts, tiles


@pytest.mark.parametrize("M,K,frac,seed", [
    (256, 256, 0.5, 1),
    (300, 256, 0.5, 2),          # partial last tile
    (1024, 512, 0.3, 3),
    (1024, 512, 0.9, 4),
    (128, 2304, 0.5, 5),         # one tile
    (640, 320, 1.0, 6),          # keep everything
    (640, 320, 1.0 / 640, 7),    # one column in total: every tile at the floor of 64
])
def test_compress_small(M, K, frac, seed):
    need_gpu()
    W = _scaled(M, K, seed)
    T = -(-M // 128)
    _compare(W, max(1, int(frac * T * K)))


def test_compress_ties_across_tiles():
    """Equal scores across tiles: the tied keys go to the lower flat index first."""
    need_gpu()
    W = np.ones((512, 256), dtype=np.float32)
    for total in (1, 300, 512, 700):
        _, counts, _ = _compare(W, total)
    assert counts.tolist() == [256, 256, 192, 64]          # total 700: raw 256, 256, 188, 0


def test_compress_zero_matrix():
    need_gpu()
    _compare(np.zeros((384, 128), dtype=np.float32), 200)


def test_compress_many_tiles():
    """Over 1024 tiles: the count scan and the ordering run over several chunks and blocks."""
    need_gpu()
    W = _scaled(128 * 1100 - 50, 256, 8, spread=0.1)
    _, counts, _ = _compare(W, 1100 * 128)
    assert len(set(counts.tolist())) == 4                  # every count 64 .. 256 occurs


@pytest.mark.parametrize("M,K,N,frac", [(256, 256, 200, 0.5), (1000, 512, 1000, 0.4), (300, 256, 72, 0.7)])
def test_spmm_small(M, K, N, frac):
    need_gpu()
    W = _scaled(M, K, M + N)
    Xb = workloads.random_bf16((K, N), seed=N)
    T = -(-M // 128)
    t, counts, tiles = _compare(W, int(frac * T * K))
    print(f"[tvw_var] spmm M={M} K={K} N={N}", flush=True)
    Y = p24.spmm_tvw_var(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, bnd = O.gemm_ref(O.tvw_var_decompress(tiles, M, K, 128), Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


def test_equal_counts_match_fixed_keep():
    """Identical tiles split the top-ranked columns evenly: the result equals spmm_tvw's bit for bit."""
    need_gpu()
    M, K, N = 512, 512, 256
    W = np.tile(workloads.random_matrix((128, K), seed=9, sigma=0.02), (4, 1))
    Xb = workloads.random_bf16((K, N), seed=10)
    t = p24.tvw_var_compress(f32_dev(W), total_keep=4 * 256)
    f = p24.tvw_compress(f32_dev(W), tile_m=128, keep_k=256)
    X = bf16_dev(Xb)
    Yv = p24.spmm_tvw_var(t, X, out_dtype=torch.float32)
    Yf = p24.spmm_tvw(f, X, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert t.offsets.cpu().tolist() == [0, 256, 512, 768, 1024]
    assert torch.equal(t.kept[:1024].view(4, 256), f.kept)
    assert torch.equal(Yv, Yf)


def test_c5v_full():
    need_gpu()
    wl = workloads.WORKLOADS["c5v"]
    W = workloads.weights(wl)
    t, counts, tiles = _compare(W, wl.total_keep)
    assert counts.max() > 1.5 * counts.mean()        # the workload really is irregular across tiles
    Xb = workloads.activations(wl)
    Wd = O.tvw_var_decompress(tiles, wl.M, wl.K, 128)
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    for out, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        print(f"[tvw_var] c5v spmm {out}", flush=True)
        Y = p24.spmm_tvw_var(t, bf16_dev(Xb), out_dtype=dt)
        torch.cuda.synchronize()
        ok, worst = O.check(y_host(Y), y_ref, bnd, out)
        assert ok, worst
