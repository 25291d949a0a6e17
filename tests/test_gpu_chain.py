"""GPU parity for the two-layer chain spmm24_tvw_chain: layer 1 (2:4, bias and
activation in its epilogue) writes H as bf16 in the row-major layout layer 2's
TVW gather reads; layer 2 multiplies it.  H is checked against the oracle's fused
reference and Y2 against the composed oracle (oracle.prune24.chain_ref) within
chain_tolerance; the chain equals its two products called one after the other,
bit for bit."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu

ACTS = {"none": O.ACT_NONE, "relu": O.ACT_RELU, "gelu": O.ACT_GELU}


def _run(M1, K1, M2, N, keep2, act1, act2, out, seed, with_b2=True, sigma1=0.05, sigma2=0.05):
    print(f"[chain] M1={M1} K1={K1} M2={M2} N={N} keep2={keep2} {act1}/{act2} {out}", flush=True)
    W1 = workloads.random_matrix((M1, K1), seed=seed, sigma=sigma1)
    W2 = workloads.random_matrix((M2, M1), seed=seed + 1, sigma=sigma2)
    Xb = workloads.random_bf16((K1, N), seed=seed + 2)
    b1 = (0.1 * np.random.default_rng(seed + 3).standard_normal(M1)).astype(np.float32)
    b2 = (0.1 * np.random.default_rng(seed + 4).standard_normal(M2)).astype(np.float32) if with_b2 else None
    c1 = p24.compress(f32_dev(W1))
    t2 = p24.tvw_compress(f32_dev(W2), tile_m=128, keep_k=keep2)
    X = bf16_dev(Xb)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    B1 = f32_dev(b1)
    B2 = None if b2 is None else f32_dev(b2)
    Y2, H = p24.spmm24_tvw_chain(c1, t2, X, bias1=B1, act1=act1, bias2=B2, act2=act2, out_dtype=dt)
    # the same two products called one after the other
    H_s = p24.spmm24(c1, X, out_dtype=torch.bfloat16, bias=B1, act=act1)
    Y2_s = p24.spmm_tvw(t2, H_s, out_dtype=dt, bias=B2, act=act2)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if dt == torch.bfloat16 else (lambda t: t.view(torch.int32))
    assert torch.equal(H.view(torch.int16), H_s.view(torch.int16))
    assert torch.equal(bits(Y2), bits(Y2_s))
    # oracle
    W1d = O.decompress_24(*O.compress_24(W1, "f32"), K1)
    kept, v2, m2 = O.tvw_compress(W2, 128, keep2)
    W2d = O.tvw_decompress(kept, v2, m2, M2, M1, 128)
    h, z1, bnd1 = O.fused_ref(W1d, Xb, b1, ACTS[act1])
    ok, worst = O.check_fused(y_host(H), h, z1, bnd1, ACTS[act1], "bf16")
    assert ok, f"H: worst err/tol {worst}"
    ref = O.chain_ref(W1d, Xb, b1, ACTS[act1], W2d, b2, ACTS[act2])
    ok, worst = O.check_chain(y_host(Y2), *ref, ACTS[act2], out)
    assert ok, f"Y2: worst err/tol {worst}"
    return worst


@pytest.mark.parametrize("M1,K1,M2,N,keep2", [
    (256, 128, 256, 200, 128),
    (384, 256, 300, 72, 192),      # ragged M2 and N, a partial last TVW tile
    (128, 64, 128, 1000, 64),      # one TVW tile
])
@pytest.mark.parametrize("act1,act2", [("gelu", "none"), ("relu", "gelu"), ("none", "relu")])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_chain_parity(M1, K1, M2, N, keep2, act1, act2, out):
    need_gpu()
    _run(M1, K1, M2, N, keep2, act1, act2, out, seed=M1 + K1 + N)


def test_chain_without_layer2_epilogue():
    need_gpu()
    _run(256, 256, 256, 136, 128, "gelu", "none", "bf16", seed=5, with_b2=False)


def test_chain_tvw_workload_shape():
    """Layer 1 the BERT-like 4096 x 4096 2:4 projection with GELU, layer 2 the TVW workload
    (4096 x 4096, tile 128, keep 2048), 4096 tokens: every output element checked."""
    need_gpu()
    _run(4096, 4096, 4096, 4096, 2048, "gelu", "none", "bf16", seed=41, sigma1=0.02, sigma2=0.02)


def test_chain_argument_errors():
    need_gpu()
    L = p24.lib()
    c1 = p24.compress(f32_dev(workloads.random_matrix((256, 128), seed=1)))
    t2 = p24.tvw_compress(f32_dev(workloads.random_matrix((256, 256), seed=2)), tile_m=128, keep_k=128)
    X = bf16_dev(workloads.random_bf16((128, 64), seed=3))
    H = torch.empty((256, 64), dtype=torch.bfloat16, device=X.device)
    Y = torch.empty((256, 64), dtype=torch.bfloat16, device=X.device)
    args = lambda h, y, k2=t2.keep_k, ldh=64: (
        p24._ptr(c1.values), p24._ptr(c1.meta), 256, 128, None, p24.P24_ACT_GELU, p24._ptr(t2.kept),
        p24._ptr(t2.values), p24._ptr(t2.meta), 256, 128, k2, p24._ptr(X), 64, 64, h, ldh, y, p24.P24_BF16, 64,
        None, p24.P24_ACT_NONE, None)
    assert L.spmm24_tvw_chain(*args(p24._ptr(X), p24._ptr(Y))) == p24.P24_ERR_UNSUPPORTED    # H is X
    assert L.spmm24_tvw_chain(*args(p24._ptr(H), p24._ptr(H))) == p24.P24_ERR_UNSUPPORTED    # H is Y2
    assert L.spmm24_tvw_chain(*args(None, p24._ptr(Y))) == p24.P24_ERR_NULL
    assert L.spmm24_tvw_chain(*args(p24._ptr(H), p24._ptr(Y), k2=100)) == p24.P24_ERR_UNSUPPORTED
    assert L.spmm24_tvw_chain(*args(p24._ptr(H), p24._ptr(Y), ldh=60)) == p24.P24_ERR_SHAPE
    with pytest.raises(ValueError, match="layer 2 takes"):
        p24.spmm24_tvw_chain(c1, p24.tvw_compress(f32_dev(workloads.random_matrix((128, 128), seed=4)),
                                                  tile_m=128, keep_k=64), X)
