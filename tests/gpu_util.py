"""Helpers shared by the GPU parity tests (host-side plumbing only)."""
import numpy as np
import pytest

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


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist())
    rows.update({0, M - 1})
    return np.array(sorted(rows))
