"""GPU parity: prune24_compress / prune24_decompress are bit-exact with the oracle.

Covers every workload shape at full size, both input dtypes, both layouts,
ragged M and K, the adversarial tie / signed-zero / Inf / NaN alphabet, and
run-to-run determinism.
"""
import itertools

import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, u16_host, u32_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _oracle(W, dtype, layout):
    values, meta = O.compress_24(W, dtype)
    if layout == "device":
        return O.to_device_layout(values, meta, W.shape[1])
    return values.reshape(-1), meta.reshape(-1)


def _gpu(Wt, layout):
    c = p24.compress(Wt, layout=layout)
    torch.cuda.synchronize()
    return c, u16_host(c.values), u32_host(c.meta)


@pytest.mark.parametrize("key", ["c1", "c2", "c3a", "c3b", "c4", "c5"])
def test_workload_shapes_f32_device(key):
    need_gpu()
    wl = workloads.WORKLOADS[key]
    print(f"[compress] {key} {wl.M}x{wl.K}", flush=True)
    W = workloads.weights(wl)
    _, gv, gm = _gpu(f32_dev(W), "device")
    ov, om = _oracle(W, "f32", "device")
    assert np.array_equal(gv, ov)
    assert np.array_equal(gm, om)


@pytest.mark.parametrize("M,K", [(256, 256), (45, 128), (33, 64), (3072, 768)])
@pytest.mark.parametrize("layout", ["canonical", "device"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layouts_dtypes_ragged(M, K, layout, dtype):
    need_gpu()
    W = workloads.random_matrix((M, K), seed=M + K, sigma=0.5)
    if dtype == "bf16":
        Wh = workloads.truncate_to_bf16_bits(W)
        Wt = bf16_dev(Wh)
    else:
        Wh = W
        Wt = f32_dev(W)
    c, gv, gm = _gpu(Wt, layout)
    ov, om = _oracle(Wh, dtype, layout)
    assert np.array_equal(gv[:ov.size], ov) and np.array_equal(gm[:om.size], om)
    # decompress goes back to bf16(prune(W))
    D = p24.decompress(c)
    torch.cuda.synchronize()
    want = O.prune_24(Wh, dtype) if dtype == "bf16" else O.bf16_rne(O.prune_24(Wh, dtype))
    assert np.array_equal(u16_host(D), want)


@pytest.mark.parametrize("M,K", [(5, 4), (7, 36), (16, 100), (2, 1000)])
def test_canonical_odd_k(M, K):
    need_gpu()
    W = workloads.random_matrix((M, K), seed=3 * K + M)
    _, gv, gm = _gpu(f32_dev(W), "canonical")
    ov, om = _oracle(W, "f32", "canonical")
    assert np.array_equal(gv[:ov.size], ov) and np.array_equal(gm[:om.size], om)


@pytest.mark.parametrize("layout", ["canonical", "device"])
def test_adversarial_alphabet(layout):
    need_gpu()
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, np.inf, np.nan], dtype=np.float32)
    tuples = np.array(list(itertools.product(range(8), repeat=4)))
    W = alphabet[tuples].reshape(64, 256)                     # 4096 groups
    _, gv, gm = _gpu(f32_dev(W), layout)
    ov, om = _oracle(W, "f32", layout)
    assert np.array_equal(gv, ov) and np.array_equal(gm, om)
    # the same alphabet in bf16
    Wb = workloads.truncate_to_bf16_bits(W)
    _, gv, gm = _gpu(bf16_dev(Wb), layout)
    ov, om = _oracle(Wb, "bf16", layout)
    assert np.array_equal(gv, ov) and np.array_equal(gm, om)


def test_rounding_edges():
    need_gpu()
    # halfway and overflow cases of the fp32 -> bf16 cast, placed where they survive selection
    vals = np.array([0x3F808000, 0x3F818000, 0x7F7FFFFF, 0x7F7F7FFF, 0xC0400000, 0x00000001, 0x80008000,
                     0x7F800001], dtype=np.uint32).view(np.float32)
    W = np.zeros((32, 64), dtype=np.float32)
    W[:, 0::4] = np.resize(vals, (32, 16))
    W[:, 1::4] = np.resize(vals[::-1], (32, 16))
    _, gv, gm = _gpu(f32_dev(W), "device")
    ov, om = _oracle(W, "f32", "device")
    assert np.array_equal(gv, ov) and np.array_equal(gm, om)


def test_deterministic_and_zero_sized():
    need_gpu()
    W = f32_dev(workloads.random_matrix((512, 512), seed=1))
    a = _gpu(W, "device")
    b = _gpu(W, "device")
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    L = p24.lib()
    assert L.prune24_compress(None, 0, 0, 64, 64, None, None, 1, None) == p24.P24_OK
