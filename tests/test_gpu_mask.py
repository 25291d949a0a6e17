"""GPU parity for masked fine-tuning: prune24_refresh (compress + in-place
zeroing of the dropped entries) and prune24_mask_apply (zeroing by stored
metadata), bit-exact against the oracle on fp32 and bf16 weights, both
layouts, ragged shapes and strided rows."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, check_full, f32_dev, need_gpu, pruned_workload_ref, torch, u16_host, u32_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _dev(W, dtype, pad=0):
    """fp32 array or bf16 bits -> cuda tensor (optionally a strided view with `pad` extra columns)."""
    if dtype == "f32":
        full = np.zeros((W.shape[0], W.shape[1] + pad), dtype=np.float32)
        full[:, :W.shape[1]] = W
        return f32_dev(full)[:, :W.shape[1]]
    return bf16_dev(W, pad_cols=pad) if pad else bf16_dev(W)


def _host(t, dtype):
    return t.contiguous().cpu().numpy().view(np.uint32) if dtype == "f32" else u16_host(t)


def _bits(W, dtype):
    return np.ascontiguousarray(W).view(np.uint32) if dtype == "f32" else W


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,layout,pad", [(64, 128, "device", 0), (200, 320, "device", 4), (37, 36, "canonical", 0),
                                            (130, 64, "canonical", 8)])
def test_refresh(dtype, M, K, layout, pad):
    need_gpu()
    print(f"[mask] refresh {dtype} {M}x{K} {layout} pad {pad}", flush=True)
    W = workloads.random_matrix((M, K), seed=M + K, sigma=0.05)
    if dtype == "bf16":
        W = workloads.truncate_to_bf16_bits(W)
    Wd = _dev(W, dtype, pad)
    c = p24.refresh(Wd, layout=layout)
    torch.cuda.synchronize()
    Wp, values, meta = O.refresh(W, dtype)
    assert np.array_equal(_host(Wd, dtype), _bits(Wp, dtype))
    if layout == "device":
        values, meta = O.to_device_layout(values, meta, K)
    assert np.array_equal(u16_host(c.values)[:values.size], np.asarray(values).reshape(-1))
    assert np.array_equal(u32_host(c.meta)[:meta.size], np.asarray(meta).reshape(-1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,layout,pad", [(64, 128, "device", 0), (200, 320, "device", 4), (37, 36, "canonical", 0)])
def test_mask_apply_foreign(dtype, M, K, layout, pad):
    """The mask of one matrix applied to another (the per-step masking after an update)."""
    need_gpu()
    print(f"[mask] apply {dtype} {M}x{K} {layout} pad {pad}", flush=True)
    W = workloads.random_matrix((M, K), seed=M + 1, sigma=0.05)
    V = workloads.random_matrix((M, K), seed=M + 2, sigma=0.05)
    if dtype == "bf16":
        W, V = workloads.truncate_to_bf16_bits(W), workloads.truncate_to_bf16_bits(V)
    c = p24.compress(_dev(V, dtype), layout=layout)
    Wd = _dev(W, dtype, pad)
    p24.mask_apply(Wd, c)
    torch.cuda.synchronize()
    _, meta_v = O.compress_24(V, dtype)
    assert np.array_equal(_host(Wd, dtype), _bits(O.mask_apply(W, meta_v, dtype), dtype))


def test_mask_apply_special_values():
    """Selected entries pass bit for bit (NaN payloads, -0, inf); unselected ones become +0."""
    need_gpu()
    rng = np.random.default_rng(45)
    W = rng.standard_normal((32, 64)).astype(np.float32)
    bits = W.view(np.uint32)
    bits[0, :8] = [0x80000000, 0x7FC01234, 0x7F800000, 0xFF800000, 0x00000001, 0x80000001, 0x3F800000, 0xBF800000]
    V = workloads.random_matrix((32, 64), seed=46, sigma=0.05)
    c = p24.compress(f32_dev(V), layout="canonical")
    Wd = f32_dev(W)
    p24.mask_apply(Wd, c)
    torch.cuda.synchronize()
    _, meta_v = O.compress_24(V)
    assert np.array_equal(_host(Wd, "f32"), O.mask_apply(W, meta_v).view(np.uint32))


def test_fine_tune_loop():
    """refresh, then updates each followed by mask_apply: the pattern stays, and the product of the
    re-compressed weights matches the oracle's masked weights."""
    need_gpu()
    M, K, N = 256, 256, 128
    W = workloads.random_matrix((M, K), seed=47, sigma=0.05)
    Wd = f32_dev(W)
    c = p24.refresh(Wd)
    Wh = O.refresh(W)[0]
    _, meta0 = O.compress_24(W)
    for step in range(3):
        U = workloads.random_matrix((M, K), seed=50 + step, sigma=0.01)
        Wd += f32_dev(U)
        p24.mask_apply(Wd, c)
        Wh = O.mask_apply((Wh + U).astype(np.float32), meta0)
    torch.cuda.synchronize()
    assert np.array_equal(_host(Wd, "f32"), Wh.view(np.uint32))
    Xb = workloads.random_bf16((K, N), seed=60)
    Y = p24.spmm24(p24.compress(Wd), bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, bnd = O.gemm_ref(O.decompress_24(*O.compress_24(Wh), K), Xb)
    ok, worst = O.check(Y.cpu().numpy().astype(np.float64), y_ref, bnd, "f32")
    assert ok, worst


def test_refresh_and_mask_at_bench_size():
    """The 8192 x 8192 fp32 weight the benchmark re-prunes: every row of the in-place result,
    of a foreign mask and of the product with the re-compressed weight against the oracle."""
    need_gpu()
    wl = workloads.WORKLOADS["c4"]
    W = workloads.weights(wl)
    print("[mask] refresh 8192^2", flush=True)
    Wd = f32_dev(W)
    c = p24.refresh(Wd)
    torch.cuda.synchronize()
    assert np.array_equal(Wd.cpu().numpy().view(np.uint32), O.prune_24(W).view(np.uint32))
    print("[mask] mask_apply 8192^2", flush=True)
    Vh = workloads.random_matrix((wl.M, wl.K), seed=11, sigma=0.02)
    V = f32_dev(Vh)
    p24.mask_apply(V, c)
    torch.cuda.synchronize()
    _, meta = O.compress_24(W)
    assert np.array_equal(V.cpu().numpy().view(np.uint32), O.mask_apply(Vh, meta).view(np.uint32))
    print("[mask] spmm24 on the re-pruned weight", flush=True)
    Xb = workloads.activations(wl)
    Y = p24.spmm24(c, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_full(Y, *pruned_workload_ref("c4"), "f32")
