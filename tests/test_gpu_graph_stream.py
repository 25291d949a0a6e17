"""Stream and graph behaviour of the library calls: every call enqueues on the caller's
current stream, and the products can be captured in a HIP graph and replayed.  The kernels
are deterministic (fixed reduction order), so results are compared bit for bit."""
import numpy as np
import pytest

import workloads
from gpu_util import DEV, bf16_dev, f32_dev, need_gpu, torch

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu

M, K, N = 512, 512, 384


def _inputs():
    W = workloads.random_matrix((M, K), seed=31, sigma=0.05)
    X1 = workloads.random_bf16((K, N), seed=32)
    X2 = workloads.random_bf16((K, N), seed=33)
    return W, X1, X2


def test_side_stream_matches_default_stream():
    """Compression, TVW selection and both products on a side stream (default priority)
    equal the same calls on the default stream."""
    need_gpu()
    print("[stream] side stream", flush=True)
    W, X1, _ = _inputs()
    Wt, X = f32_dev(W), bf16_dev(X1)
    c = p24.compress(Wt)
    t = p24.tvw_compress(Wt, tile_m=128, keep_k=256)
    Y, Yt = p24.spmm24(c, X), p24.spmm_tvw(t, X)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c2 = p24.compress(Wt)
        t2 = p24.tvw_compress(Wt, tile_m=128, keep_k=256)
        Y2, Yt2 = p24.spmm24(c2, X), p24.spmm_tvw(t2, X)
    s.synchronize()
    assert torch.equal(c.values.view(torch.int16), c2.values.view(torch.int16))
    assert torch.equal(c.meta, c2.meta)
    assert torch.equal(t.kept, t2.kept)
    assert torch.equal(Y, Y2) and torch.equal(Yt, Yt2)


def test_graph_replays_match_eager_calls():
    """spmm24 and spmm_tvw captured in one graph; three replays with eager changes of the
    input (and of the outputs) in between each equal the eager calls on that input."""
    need_gpu()
    print("[graph] capture and replay", flush=True)
    W, X1, X2 = _inputs()
    Wt = f32_dev(W)
    c = p24.compress(Wt)
    t = p24.tvw_compress(Wt, tile_m=128, keep_k=256)
    refs = {}
    for key, xb in (("x1", X1), ("x2", X2)):
        xd = bf16_dev(xb)
        refs[key] = (p24.spmm24(c, xd), p24.spmm_tvw(t, xd))
    X = bf16_dev(X1)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    Yt = torch.empty_like(Y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            p24.spmm24(c, X, out=Y)
            p24.spmm_tvw(t, X, out=Yt)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p24.spmm24(c, X, out=Y)
        p24.spmm_tvw(t, X, out=Yt)
    for key, xb in (("x2", X2), ("x1", X1), ("x2", X2)):
        X.copy_(bf16_dev(xb))
        Y.fill_(0.0)
        Yt.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r, rt = refs[key]
        assert torch.equal(Y, r), f"spmm24 replay on {key}"
        assert torch.equal(Yt, rt), f"spmm_tvw replay on {key}"
