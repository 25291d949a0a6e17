"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only draws inputs.  It holds none of the method's arithmetic (no
pruning, no compression, no rounding to nearest, no GEMM) and imports neither
the oracle nor the HIP package, so both sides can take their inputs from it.

Shapes follow the layers the pages evaluate on ("Accelerating Sparse DNNs Based
on Tiled GEMM", TL;DR: CNNs, NMT and BERT; SparseRT Abstract: ResNet-50 1x1 and
3x3 convolutions).  Orientation: W is M x K (out x in), X is K x N (in x
tokens), Y = W X is M x N, all row-major; 2:4 groups run along K.

Recipe: numpy PCG64 ``default_rng``; W uses seed 0 and X seed 1.  W is fp32
N(0, sigma^2).  X is drawn in fp32 (N(0,1), or |N(0,1)| for ReLU-like
activations) and its low 16 bits are cleared, which makes every value an exact
bf16 number; bf16 values travel as uint16 bit patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

W_SEED = 0
X_SEED = 1


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    M: int
    K: int
    N: int
    w_sigma: float
    x_dist: str            # "normal" or "halfnormal"
    out_dtype: str         # "f32" or "bf16"
    tile_m: int = 0        # TVW tile rows (0: plain 2:4)
    keep_k: int = 0        # TVW kept columns per tile (with per-tile keep counts: the average)
    tile_spread: float = 0.0   # per-tile keep counts: row scale of tile t is 1 + tile_spread * U(-1, 1)

    @property
    def dense_flops(self) -> float:
        """Dense-equivalent flops of Y = W X: 2 M N K."""
        return 2.0 * self.M * self.N * self.K

    @property
    def kept_flops(self) -> float:
        """Flops the sparse method actually performs (kept multiply-adds x 2)."""
        k_eff = self.keep_k if self.tile_m else self.K
        return 2.0 * self.M * self.N * (k_eff // 2)

    @property
    def total_keep(self) -> int:
        """Per-tile keep counts: columns kept over all tiles (keep_k per tile on average)."""
        return -(-self.M // self.tile_m) * self.keep_k


WORKLOADS = {
    "c1": Workload("c1", "single 2:4 SpMM 256x256 . 256x64", 256, 256, 64, 1.0, "normal", "f32"),
    "c2": Workload("c2", "BERT-base FFN up-projection 3072x768 . 768x4096", 3072, 768, 4096, 0.02,
                   "normal", "bf16"),
    "c3a": Workload("c3a", "ResNet-50 1x1 conv as GEMM 2048x512 . 512x1568", 2048, 512, 1568,
                    math.sqrt(2.0 / 512), "halfnormal", "bf16"),
    "c3b": Workload("c3b", "ResNet-50 3x3 conv (im2col) 256x2304 . 2304x6272", 256, 2304, 6272,
                    math.sqrt(2.0 / 2304), "halfnormal", "bf16"),
    "c4": Workload("c4", "large 2:4 SpMM 8192x8192 . 8192x8192", 8192, 8192, 8192, 0.02,
                   "normal", "bf16"),
    # one GPU's share of c4 when the product is split over 8 GPUs (no exchange step):
    # by tokens (N) or by output rows (M)
    "c4n8": Workload("c4n8", "8192^3 split 8 ways by tokens: 8192x8192 . 8192x1024", 8192, 8192, 1024, 0.02,
                     "normal", "bf16"),
    "c4m8": Workload("c4m8", "8192^3 split 8 ways by output rows: 1024x8192 . 8192x8192", 1024, 8192, 8192, 0.02,
                     "normal", "bf16"),
    "c5": Workload("c5", "TVW 4096x4096 . 4096x4096, tile 128 rows, keep 2048 columns", 4096, 4096,
                   4096, 0.02, "normal", "bf16", tile_m=128, keep_k=2048),
    "c5v": Workload("c5v", "TVW with per-tile keep counts 4096x4096 . 4096x4096, tile 128 rows, "
                           "2048 columns per tile on average", 4096, 4096, 4096, 0.02, "normal", "bf16",
                    tile_m=128, keep_k=2048, tile_spread=0.1),
}

TILE_SCALE_SEED = 2


def weights(wl: Workload, seed: int = W_SEED, rows: int | None = None) -> np.ndarray:
    """fp32 W [M, K] ~ N(0, w_sigma^2).  ``rows`` draws only the first rows (same values)."""
    rng = np.random.default_rng(seed)
    m = wl.M if rows is None else rows
    w = rng.standard_normal((m, wl.K), dtype=np.float32)
    w = (w * np.float32(wl.w_sigma)).astype(np.float32)
    if wl.tile_spread:
        w *= tile_scales(wl)[np.arange(m) // wl.tile_m][:, None]
    return w


def tile_scales(wl: Workload) -> np.ndarray:
    """fp32 row scale per tile: 1 + tile_spread * U(-1, 1), so that tiles differ in importance."""
    T = -(-wl.M // wl.tile_m)
    u = np.random.default_rng(TILE_SCALE_SEED).uniform(-1.0, 1.0, T)
    return (1.0 + wl.tile_spread * u).astype(np.float32)


def truncate_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Keep the high 16 bits of each fp32 value (an exact bf16 number, rounded toward zero)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def activations(wl: Workload, seed: int = X_SEED) -> np.ndarray:
    """bf16 bits X [K, N]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((wl.K, wl.N), dtype=np.float32)
    if wl.x_dist == "halfnormal":
        x = np.abs(x)
    return truncate_to_bf16_bits(x)


def random_matrix(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """Generic seeded fp32 N(0, sigma^2) matrix for ad-hoc shapes in tests."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def random_bf16(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    return truncate_to_bf16_bits(random_matrix(shape, seed, sigma))


def small_int_matrix(shape, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integer-valued fp32 matrix (exact in bf16 for |v| <= 256)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)
