"""Pins for the oracle's fp32 -> bf16 round-to-nearest-even (the cast applied to kept values).

Pinned by closed-form bit patterns, by the definition of "nearest, ties to
even" checked by brute force against both neighbours, and by a library routine
(torch's CPU bfloat16 conversion, which rounds to nearest even).
"""
import numpy as np
import pytest

from oracle import prune24 as O


def _f(u):
    return np.array([u], dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("bits,expect", [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # 1 + 2^-8: halfway, even neighbour is 0x3F80
    (0x3F818000, 0x3F82),   # halfway between 0x3F81 and 0x3F82 -> even 0x3F82
    (0x3F808001, 0x3F81),   # just above halfway -> up
    (0x3F807FFF, 0x3F80),   # just below halfway -> down
    (0x80000000, 0x8000),   # -0
    (0x00000001, 0x0000),   # smallest subnormal rounds to +0
    (0x7F7FFFFF, 0x7F80),   # largest finite rounds to +Inf
    (0x7F7F7FFF, 0x7F7F),   # stays finite
    (0x7F800000, 0x7F80),   # +Inf
    (0xFF800000, 0xFF80),   # -Inf
    (0x7FC00000, 0x7FC0),   # quiet NaN
    (0xFFC00001, 0xFFC0),   # negative NaN keeps its sign
    (0x7F800001, 0x7FC0),   # signalling NaN is quieted, never turned into Inf
    (0xC0400000, 0xC040),   # -3.0
])
def test_rne_closed_forms(bits, expect):
    assert int(O.bf16_rne(_f(bits))[0]) == expect


def test_rne_is_nearest_ties_even_bruteforce():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 0x7F7F0000, size=200_000, dtype=np.uint64).astype(np.uint32)
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000            # exact halfway cases
    sign = rng.integers(0, 2, size=u.size, dtype=np.uint32) << 31
    x = (u | sign).view(np.float32)
    got = O.bf16_rne(x)
    lo = (x.view(np.uint32) >> 16).astype(np.uint32)        # truncation toward zero
    hi = lo + 1
    vx = x.astype(np.float64)
    vlo = (lo << 16).view(np.float32).astype(np.float64)
    vhi = (hi << 16).view(np.float32).astype(np.float64)
    dlo, dhi = np.abs(vx - vlo), np.abs(vx - vhi)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(got.astype(np.uint32), want)


def test_rne_matches_torch_cpu():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-30, 30, 100_000))).astype(np.float32)
    x[:500] = ((x[:500].view(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_rne(x), t)


def test_bf16_to_f64_roundtrip():
    b = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f64(b)
    finite = np.isfinite(f)
    back = O.bf16_rne(f[finite].astype(np.float32))
    assert np.array_equal(back, b[finite])
