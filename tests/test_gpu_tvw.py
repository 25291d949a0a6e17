"""GPU parity for tile-vector-wise sparsity: tvw_compress bit-exact, spmm_tvw in tolerance."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, u16_host, u32_host, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _compare_compress(W, tile, keep, layout):
    t = p24.tvw_compress(f32_dev(W), tile_m=tile, keep_k=keep, layout=layout)
    torch.cuda.synchronize()
    kept, values, meta = O.tvw_compress(W, tile, keep)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    if layout == "device":
        values, meta = O.to_device_layout(values, meta, keep)
    ov, om = values.reshape(-1), meta.reshape(-1)
    assert np.array_equal(u16_host(t.values)[:ov.size], ov)
    assert np.array_equal(u32_host(t.meta)[:om.size], om)
    return t, kept, values, meta


@pytest.mark.parametrize("M,K,tile,keep,layout", [
    (256, 256, 128, 128, "device"),
    (300, 256, 128, 128, "device"),       # partial last tile
    (300, 200, 64, 100, "canonical"),
    (256, 512, 128, 512, "device"),       # keep everything
    (128, 2304, 128, 1152, "device"),
])
def test_compress_small(M, K, tile, keep, layout):
    need_gpu()
    W = workloads.random_matrix((M, K), seed=M + K + keep, sigma=0.02)
    _compare_compress(W, tile, keep, layout)


def test_compress_ties():
    need_gpu()
    W = workloads.small_int_matrix((256, 256), seed=5, lo=-1, hi=1)   # many tied scores and groups
    _compare_compress(W, 128, 128, "device")


@pytest.mark.parametrize("fill", [0.5, 0.0])
def test_select_all_tied(fill):
    """Every column scores the same: the lowest keep_k columns are kept."""
    need_gpu()
    W = np.full((256, 3000), fill, dtype=np.float32)
    t, kept, _, _ = _compare_compress(W, 128, 1500, "canonical")
    assert np.array_equal(kept, np.tile(np.arange(1500, dtype=np.int32), (2, 1)))


def test_select_many_chunks():
    """K spans several 1024-column scan chunks with a ragged tail."""
    need_gpu()
    W = workloads.random_matrix((160, 5000), seed=77, sigma=0.02)
    _compare_compress(W, 128, 2500, "canonical")


@pytest.mark.parametrize("K", [8192, 8320])
def test_select_wide_tiles(K):
    """Wide tiles (8192 and 8320 columns: 8 and 9 scan chunks, the second ragged) with
    a tie straddling the cut."""
    need_gpu()
    W = workloads.random_matrix((130, K), seed=79, sigma=0.02)
    W[:, 3000:3400] = 0.25
    _compare_compress(W, 128, K // 2 + 64, "canonical")


def test_select_cut_bin_all_tied_and_kept():
    """keep_k equals the number of columns at or above a block of 300 tied columns,
    so the bin holding the cut is kept whole (the selection stops early there)."""
    need_gpu()
    W = workloads.random_matrix((128, 1024), seed=80, sigma=0.02)
    W[:, 600:700] = 1.0                  # 100 columns above everything
    W[:, 100:400] = 0.25                 # 300 tied columns, above every random one
    t, kept, _, _ = _compare_compress(W, 128, 400, "canonical")
    assert np.array_equal(kept[0], np.r_[100:400, 600:700])


def test_select_threshold_tie():
    """A tie straddling the cut: only the lowest-index tied columns make it."""
    need_gpu()
    W = workloads.random_matrix((128, 1024), seed=78, sigma=0.02)
    W[:, 100:400] = 0.25                 # 300 equal columns around the keep_k-th score
    W[:, 600:700] = 1.0                  # 100 columns above every other score
    _compare_compress(W, 128, 256, "device")


def test_c5_full():
    need_gpu()
    wl = workloads.WORKLOADS["c5"]
    print("[tvw] c5 compress", flush=True)
    W = workloads.weights(wl)
    t, kept, values, meta = _compare_compress(W, wl.tile_m, wl.keep_k, "device")
    Xb = workloads.activations(wl)
    v, m = O.from_device_layout(values, meta, wl.M, wl.keep_k)
    y_ref, bnd = O.gemm_ref(O.tvw_decompress(kept, v, m, wl.M, wl.K, wl.tile_m), Xb)
    for out, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        print(f"[tvw] c5 spmm {out}", flush=True)
        Y = p24.spmm_tvw(t, bf16_dev(Xb), out_dtype=dt)
        torch.cuda.synchronize()
        ok, worst = O.check(y_host(Y), y_ref, bnd, out)
        assert ok, worst


@pytest.mark.parametrize("M,K,N,keep", [(256, 256, 200, 128), (384, 512, 1000, 256), (300, 256, 72, 128),
                                         (256, 256, 1096, 128), (384, 1024, 1000, 448), (256, 256, 520, 64)])
@pytest.mark.parametrize("tile", ["128x256", "128x512"])
def test_spmm_tvw_small(M, K, N, keep, tile, monkeypatch):
    """Both block widths of the fixed-keep gathered product (the width is forced; by default
    only grids of at least 160 wide blocks take 128 x 512), ragged N included, with one K
    step (keep 64) and an odd number of them (keep 448: seven)."""
    need_gpu()
    monkeypatch.setenv("P24_GATHER_TILE", tile)
    print(f"[tvw] spmm M={M} K={K} N={N} keep={keep} tile={tile}", flush=True)
    W = workloads.random_matrix((M, K), seed=N + keep, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N)
    t = p24.tvw_compress(f32_dev(W), tile_m=128, keep_k=keep)
    Y = p24.spmm_tvw(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    kept, values, meta = O.tvw_compress(W, 128, keep)
    y_ref, bnd = O.gemm_ref(O.tvw_decompress(kept, values, meta, M, K, 128), Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.parametrize("M,K,N,keep", [(512, 512, 600, 256), (400, 256, 264, 128)])
@pytest.mark.parametrize("tile", ["128x256", "128x512"])
def test_spmm_tvw_tall_tiles(M, K, N, keep, tile, monkeypatch):
    """TVW tiles of 256 output rows: the two 128-row block rows of a tile gather by the same
    kept list (the last tile ragged in the second case), at both block widths."""
    need_gpu()
    monkeypatch.setenv("P24_GATHER_TILE", tile)
    print(f"[tvw] tall tiles M={M} K={K} N={N} keep={keep} tile={tile}", flush=True)
    W = workloads.random_matrix((M, K), seed=M + N, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 7)
    t = p24.tvw_compress(f32_dev(W), tile_m=256, keep_k=keep)
    Y = p24.spmm_tvw(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    kept, values, meta = O.tvw_compress(W, 256, keep)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    y_ref, bnd = O.gemm_ref(O.tvw_decompress(kept, values, meta, M, K, 256), Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


def test_keep_all_equals_plain_24():
    need_gpu()
    M, K, N = 256, 256, 128
    W = workloads.random_matrix((M, K), seed=77, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=78)
    Wt = f32_dev(W)
    t = p24.tvw_compress(Wt, tile_m=128, keep_k=K)
    Yt = p24.spmm_tvw(t, bf16_dev(Xb), out_dtype=torch.float32)
    Yp = p24.spmm24(p24.compress(Wt), bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (t.kept.cpu().numpy() == np.arange(K)).all()
    assert torch.equal(Yt, Yp)
