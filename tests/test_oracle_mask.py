"""Pins for the masked fine-tuning oracle (mask_apply, refresh).

The mask read back from a matrix's own metadata must reproduce the pinned
pruning bit for bit (fp32 and bf16, including signed zeros and NaN); every one
of the six legal position pairs keeps exactly its two slots; masking is
idempotent and never changes a kept entry; a mask from another matrix zeros
exactly that matrix's dropped slots.
"""
import itertools

import numpy as np
import pytest

import workloads
from oracle import prune24 as O


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_own_mask_is_the_pruning(dtype):
    W = workloads.random_matrix((64, 96), seed=41, sigma=0.05)
    if dtype == "bf16":
        W = workloads.truncate_to_bf16_bits(W)
    _, meta = O.compress_24(W, dtype)
    out = O.mask_apply(W, meta, dtype)
    ref = O.prune_24(W, dtype)
    view = (lambda a: a.view(np.uint32)) if dtype == "f32" else (lambda a: a)
    assert np.array_equal(view(out), view(ref))


def test_every_position_pair():
    for p0, p1 in itertools.combinations(range(4), 2):
        meta = np.array([[p0 | (p1 << 2)]], dtype=np.uint32)
        W = np.array([[1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
        out = O.mask_apply(W, meta)
        keep = np.zeros(4, dtype=bool)
        keep[[p0, p1]] = True
        assert np.array_equal(out[0], np.where(keep, W[0], 0.0))


def test_special_values_kept_bitwise():
    W = np.array([[-0.0, np.nan, np.inf, -1.0, 3.0, -3.0, 0.5, 7.0]], dtype=np.float32)
    W.view(np.uint32)[0, 1] = 0x7FC01234                   # NaN with a payload
    meta = np.array([[0x1 | (0x2 << 2) | ((0x0 | (0x3 << 2)) << 4)]], dtype=np.uint32)
    out = O.mask_apply(W, meta).view(np.uint32)[0]
    src = W.view(np.uint32)[0]
    assert out[1] == 0x7FC01234 and out[2] == src[2]      # positions 1, 2 of group 0
    assert out[0] == 0 and out[3] == 0                     # dropped -> +0, not -0
    assert out[4] == src[4] and out[7] == src[7] and out[5] == 0 and out[6] == 0


def test_idempotent_and_foreign_mask():
    W = workloads.random_matrix((32, 64), seed=42, sigma=0.05)
    V = workloads.random_matrix((32, 64), seed=43, sigma=0.05)
    _, meta_v = O.compress_24(V)
    once = O.mask_apply(W, meta_v)
    assert np.array_equal(O.mask_apply(once, meta_v).view(np.uint32), once.view(np.uint32))
    dropped = O.prune_24(V).view(np.uint32) == 0           # V has no zeros, so 0 marks a dropped slot
    assert not once.view(np.uint32)[dropped].any()
    assert np.array_equal(once[~dropped], W[~dropped])


def test_refresh_pairs_pruning_with_compression():
    W = workloads.random_matrix((48, 64), seed=44, sigma=0.05)
    Wp, values, meta = O.refresh(W)
    assert np.array_equal(O.mask_apply(W, meta).view(np.uint32), Wp.view(np.uint32))
    assert np.array_equal(O.decompress_24(values, meta, 64), O.bf16_rne(Wp))
