"""GPU test of tvw_compress_noalloc, the entry point for callers that cannot allocate:
its kept lists, values and metadata equal tvw_compress's (which uses a caller-supplied
workspace) and the oracle's, bit for bit, on two calls in a row -- the second on a
smaller matrix, so any score left in the fixed scratch by the first call would show --
and a problem larger than the scratch is refused before anything runs."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import f32_dev, need_gpu, torch, u16_host, u32_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _same(a, b):
    torch.cuda.synchronize()
    assert torch.equal(a.kept, b.kept)
    assert torch.equal(a.values.view(torch.int16), b.values.view(torch.int16))
    assert torch.equal(a.meta, b.meta)


def _oracle(W, tile, keep, layout, t):
    kept, values, meta = O.tvw_compress(W, tile, keep)
    if layout == "device":
        values, meta = O.to_device_layout(values, meta, keep)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    ov, om = values.reshape(-1), meta.reshape(-1)
    assert np.array_equal(u16_host(t.values)[:ov.size], ov)
    assert np.array_equal(u32_host(t.meta)[:om.size], om)


@pytest.mark.parametrize("layout", ["device", "canonical"])
def test_noalloc_matches_workspace_call_twice(layout):
    need_gpu()
    cases = [(4096, 4096, 128, 2048, 0.02),     # the TVW workload's shape (1 MiB of scores)
             (640, 1024, 128, 512, 0.05)]       # smaller: 5 tiles, on top of the first call's scores
    for M, K, tile, keep, sigma in cases:
        print(f"[noalloc] {layout} {M}x{K} tile {tile} keep {keep}", flush=True)
        W = workloads.random_matrix((M, K), seed=M + K, sigma=sigma)
        Wd = f32_dev(W)
        got = p24.tvw_compress_noalloc(Wd, tile_m=tile, keep_k=keep, layout=layout)
        ref = p24.tvw_compress(Wd, tile_m=tile, keep_k=keep, layout=layout)
        _same(got, ref)
        _oracle(W, tile, keep, layout, got)


def test_noalloc_into_existing_outputs_and_limit():
    """Results written into the caller's tensors (no allocation on either side), twice with
    different weights; a problem whose scores exceed the scratch is refused."""
    need_gpu()
    M, K, tile, keep = 1024, 2048, 128, 1024
    out = None
    for seed in (5, 6):
        W = workloads.random_matrix((M, K), seed=seed, sigma=0.02)
        Wd = f32_dev(W)
        if out is None:
            out = p24.tvw_compress_noalloc(Wd, tile_m=tile, keep_k=keep)
        else:
            p24.tvw_compress_noalloc(Wd, tile_m=tile, keep_k=keep, out=out)
        _same(out, p24.tvw_compress(Wd, tile_m=tile, keep_k=keep))
    limit = p24.lib().tvw_noalloc_scratch_bytes()
    big = torch.zeros((128 * (limit // (8 * 1024) + 1), 1024), dtype=torch.float32, device=Wd.device)
    with pytest.raises(p24.P24Error, match="status -9"):
        p24.tvw_compress_noalloc(big, tile_m=128, keep_k=512)
