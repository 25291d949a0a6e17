"""Lane-level models of the two gfx950 matrix instructions the kernels use (test
infrastructure).  The CPU tests drive the oracle's device layouts through them;
tests/test_gpu_mfma_lanes.py checks them against the hardware instruction itself.

v_smfmac_f32_32x32x32_bf16 (A 32 x 32 with two of every four k kept, B 32 x 32,
D 32 x 32 fp32):
  A lane L: row L % 32, logical k 16 (L // 32) .. +16, as 8 stored values; the
    index half `abid` of lane L's word gives, for stored value i, its position
    p = bits [4 (i // 2) + 2 (i % 2), +2) inside the group of four k at
    16 (L // 32) + 4 (i // 2).
  B lane L: column L % 32; elements e < 8 are k = 8 (L // 32) + e, e >= 8 are
    k = 16 + 8 (L // 32) + (e - 8).
  D lane L, element i: row 8 (i // 4) + 4 (L // 32) + i % 4, column L % 32.
v_mfma_f32_32x32x16_bf16: A lane L = row L % 32, k 8 (L // 32) .. +8; B lane L =
  column L % 32, the same k; D as above.
"""
import numpy as np


def smfmac32_model(a_lanes, b_lanes, idx_lanes, abid, acc):
    """a_lanes [64, 8], b_lanes [64, 16] (float64 values), idx_lanes [64] uint32, acc [64, 16]."""
    A = np.zeros((32, 32))
    for L in range(64):
        r, h = L % 32, L // 32
        bits = (int(idx_lanes[L]) >> (16 * abid)) & 0xFFFF
        for i in range(8):
            q, j = i // 2, i % 2
            p = (bits >> (4 * q + 2 * j)) & 3
            A[r, 16 * h + 4 * q + p] += a_lanes[L, i]
    B = np.zeros((32, 32))
    for lb in range(64):
        n, h = lb % 32, lb // 32
        for e in range(16):
            k = 8 * h + e if e < 8 else 16 + 8 * h + (e - 8)
            B[k, n] = b_lanes[lb, e]
    D = A @ B
    out = np.array(acc, dtype=np.float64, copy=True)
    for lo in range(64):
        n = lo % 32
        for i in range(16):
            out[lo, i] += D[8 * (i // 4) + 4 * (lo // 32) + i % 4, n]
    return out


def mfma32x32x16_model(a, b, acc):
    """a [64, 8], b [64, 8] (float64 values), acc [64, 16]."""
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for L in range(64):
        A[L % 32, 8 * (L // 32): 8 * (L // 32) + 8] = a[L]
        B[8 * (L // 32): 8 * (L // 32) + 8, L % 32] = b[L]
    D = A @ B
    out = np.array(acc, dtype=np.float64, copy=True)
    for lo in range(64):
        for i in range(16):
            out[lo, i] += D[8 * (i // 4) + 4 * (lo // 32) + i % 4, lo % 32]
    return out
