"""The hardware's lane mapping of the two matrix instructions the kernels use,
against the lane-level models (tests/mfma_models.py) through which the CPU tests
check the oracle's device layouts.  One wavefront runs one instruction
(tests/hw_probe/mfma_probe.hip) on random integer-valued bf16 operands, so every
result is exact and must match the model bit for bit.

For the sparse instruction the index words hold only the six position pairs a 2:4
group can have (p0 < p1), as the device layout writes them, and both index halves
(abid 0 and 1) are exercised; the half not selected holds different pairs, so a
wrong half shows.  The pages describe only NVIDIA's Sparse Tensor Core ("Accelerating
Sparse Deep Neural Networks", Abstract); the gfx950 operand order is measured."""
import ctypes
import os

import numpy as np
import pytest

from gpu_util import need_gpu, torch
from mfma_models import mfma32x32x16_model, smfmac32_model

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw_probe", "libp24_mfma_probe.so")
PAIRS = [0x4, 0x8, 0xC, 0x9, 0xD, 0xE]      # p0 | p1 << 2 with p0 < p1


def _lib():
    import structured_sparse_gemm_prune24_amd as p24
    p24.lib()                    # torch and the library first: one HIP runtime in the process
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    L.p24probe_smfmac32.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp]
    L.p24probe_smfmac32.restype = ctypes.c_int
    L.p24probe_mfma32x32x16.argtypes = [vp, vp, vp, vp]
    L.p24probe_mfma32x32x16.restype = ctypes.c_int
    return L


def _bf16_ints(rng, shape, lo=-8, hi=8):
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16), v.astype(np.float64)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("abid", [0, 1])
@pytest.mark.parametrize("seed", range(8))
def test_smfmac_lane_map(abid, seed):
    need_gpu()
    L = _lib()
    rng = np.random.default_rng(100 * abid + seed)
    a_bits, a_val = _bf16_ints(rng, (64, 8))
    b_bits, b_val = _bf16_ints(rng, (64, 16))
    nib = np.array(PAIRS, dtype=np.uint32)[rng.integers(0, 6, size=(64, 8))]
    idx = np.zeros(64, dtype=np.uint32)
    for q in range(8):
        idx |= nib[:, q] << np.uint32(4 * q)
    a, b, ix = _dev(a_bits.view(np.int16)), _dev(b_bits.view(np.int16)), _dev(idx.view(np.int32))
    d = torch.zeros((64, 16), dtype=torch.float32, device=a.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.p24probe_smfmac32(a.data_ptr(), b.data_ptr(), ix.data_ptr(), abid, d.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    want = smfmac32_model(a_val, b_val, idx, abid, np.zeros((64, 16)))
    assert np.array_equal(d.cpu().numpy().astype(np.float64), want)
    # the other half selects other positions, so it gives another result
    assert not np.array_equal(want, smfmac32_model(a_val, b_val, idx, 1 - abid, np.zeros((64, 16))))


@pytest.mark.parametrize("seed", range(4))
def test_mfma_lane_map(seed):
    need_gpu()
    L = _lib()
    rng = np.random.default_rng(500 + seed)
    a_bits, a_val = _bf16_ints(rng, (64, 8))
    b_bits, b_val = _bf16_ints(rng, (64, 8))
    a, b = _dev(a_bits.view(np.int16)), _dev(b_bits.view(np.int16))
    d = torch.zeros((64, 16), dtype=torch.float32, device=a.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.p24probe_mfma32x32x16(a.data_ptr(), b.data_ptr(), d.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy().astype(np.float64), mfma32x32x16_model(a_val, b_val, np.zeros((64, 16))))
