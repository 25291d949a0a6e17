"""Helpers shared by the GPU parity tests (host-side plumbing only)."""
from collections import OrderedDict

import numpy as np
import pytest

import workloads
from oracle import prune24 as O

torch = pytest.importorskip("torch")

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def bf16_dev(bits: np.ndarray, pad_cols: int = 0):
    """uint16 bf16 bits [R, C] -> cuda bf16 tensor; optional extra row padding (a strided view)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if pad_cols:
        full = np.zeros((bits.shape[0], bits.shape[1] + pad_cols), dtype=np.uint16)
        full[:, :bits.shape[1]] = bits
        t = torch.from_numpy(full.view(np.int16)).to(DEV).view(torch.bfloat16)
        return t[:, :bits.shape[1]]
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def f32_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def u16_host(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u32_host(t) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint32)


def y_host(t, rows=None) -> np.ndarray:
    """Output tensor (fp32 or bf16) -> float64 numpy, optionally only some rows."""
    if rows is not None:
        t = t[torch.as_tensor(rows, device=t.device)]
    return t.float().cpu().numpy().astype(np.float64)


_REFS: "OrderedDict[tuple, tuple]" = OrderedDict()
_REFS_KEPT = 2


def cached_ref(tag: tuple, make):
    """(y_ref, bound) from `make()` (an oracle call), computed once per session under
    `tag`: several tests multiply the same full-size weight, and an fp64 reference of
    every row of the 8192^3 product takes seconds on the host.  The two most
    recently used references are kept (about 1 GiB each at that size)."""
    if tag in _REFS:
        _REFS.move_to_end(tag)
        return _REFS[tag]
    while len(_REFS) >= _REFS_KEPT:
        _REFS.popitem(last=False)
    _REFS[tag] = make()
    return _REFS[tag]


def pruned_workload_ref(key: str):
    """Oracle (y_ref, bound) over every output row of the named workload: its weight
    magnitude-pruned 2:4 and rounded to bf16, times its activations."""
    def make():
        wl = workloads.WORKLOADS[key]
        W = workloads.weights(wl)
        values, meta = O.compress_24(W, "f32")
        return O.gemm_ref(O.decompress_24(values, meta, wl.K), workloads.activations(wl))
    return cached_ref(("pruned", key), make)


def check_full(Y, y_ref, bound, out: str):
    """Every output element of Y against the oracle's bound; returns the worst err/tol."""
    ok, worst = O.check(y_host(Y), y_ref, bound, out)
    assert ok, f"worst err/tol {worst}"
    return worst
