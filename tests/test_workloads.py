"""The seeded input generators (no GPU)."""
import numpy as np
import torch

import workloads
from oracle import brute


def test_dense_is_seeded():
    a = workloads.dense_inputs(2, 3, 17, 8, seed=7)
    b = workloads.dense_inputs(2, 3, 17, 8, seed=7)
    c = workloads.dense_inputs(2, 3, 17, 8, seed=8)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[1], c[1])
    assert [t.shape for t in a] == [(3, 8), (2, 3, 17, 8), (2, 3, 17, 8)]


def test_score_span_stretches_every_head():
    """Long-sequence recipe: per (b,h) the largest |score| reaches the span
    (up to bfloat16 rounding of the keys)."""
    B, H, N, d = 2, 3, 500, 128
    q, k, v = workloads.dense_inputs(B, H, N, d, seed=3, dtype="bf16", score_span=80.0)
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16
    scale = workloads.default_scale(d)
    for b in range(B):
        for h in range(H):
            s = brute.scores(q[h].float().numpy(), k[b, h].float().numpy(), scale)
            assert abs(np.abs(s).max() - 80.0) < 0.8, np.abs(s).max()


def test_lengths_and_offsets():
    L = workloads.segment_lengths(4096, 8192, seed=4)
    assert L.dtype == np.int64 and L.min() >= 1 and L.max() <= 8192
    assert np.array_equal(L, workloads.segment_lengths(4096, 8192, seed=4))
    offs = workloads.offsets_of(L)
    assert offs[0] == 0 and offs[-1] == L.sum() and np.all(np.diff(offs) == L)
    # the expected total is 4096 * 4096.5; a seeded draw stays within a few percent
    assert abs(offs[-1] / (4096 * 4096.5) - 1) < 0.05


def test_segmented_and_step_shapes():
    q, k, v, offs = workloads.segmented_inputs(np.array([3, 1, 4]), 2, 8, seed=4)
    assert k.shape == (8, 2, 8) and offs.tolist() == [0, 3, 4, 8]
    q, k, v = workloads.step_inputs(5, 2, 8, steps=3, seed=5)
    assert k.shape == (3, 5, 2, 8) and q.shape == (2, 8)


def test_default_scale_is_float32():
    s = workloads.default_scale(64)
    assert s == 0.125 and np.float32(workloads.default_scale(128)) == workloads.default_scale(128)
