"""Pins of the top-K-then-softmax router oracle (CPU).

Each pin fixes the oracle against something other than itself: the library
softmax when K = E, brute force over every K-subset on tiny inputs, closed
forms for equal logits and a hand-worked example, and shift invariance.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

from oracle.router import topk_softmax


def test_k_equals_e_is_the_library_softmax():
    """With K = E every expert is selected: the weights, put back in expert order,
    are the ordinary softmax (torch, float64)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    z = rng.standard_normal((50, 16)) * 3
    idx, w = topk_softmax(z, 16)
    back = np.zeros_like(w)
    np.put_along_axis(back, idx.astype(np.int64), w, axis=1)
    ref = torch.softmax(torch.from_numpy(z), dim=-1).numpy()
    assert np.abs(back - ref).max() <= 1e-15


@pytest.mark.parametrize("e,k", [(5, 1), (6, 2), (6, 3), (7, 4)])
def test_brute_force_subsets(e, k):
    """The selected set is the unique K-subset whose every member outranks every
    non-member (larger logit, or equal logit and lower index), listed in rank order,
    and the weights are e^{z_i} / sum over the subset of e^{z_j} (no max shift)."""
    rng = np.random.default_rng(e * 10 + k)
    z = rng.integers(-3, 4, size=(40, e)).astype(np.float64)  # many ties
    idx, w = topk_softmax(z, k)
    outranks = lambda a, b, row: row[a] > row[b] or (row[a] == row[b] and a < b)
    for t in range(z.shape[0]):
        row = z[t]
        good = [s for s in itertools.combinations(range(e), k)
                if all(outranks(i, j, row) for i in s for j in range(e) if j not in s)]
        assert len(good) == 1
        ranked = sorted(good[0], key=lambda i: (-row[i], i))
        assert list(idx[t]) == ranked
        den = sum(math.exp(row[j]) for j in ranked)
        assert np.allclose(w[t], [math.exp(row[i]) / den for i in ranked], rtol=1e-14, atol=0)


def test_equal_logits_closed_form():
    """All logits equal: experts 0 .. K-1 in order, each weight exactly 1/K."""
    idx, w = topk_softmax(np.full((3, 8), 0.75), 4)
    assert (idx == np.arange(4)).all()
    assert np.abs(w - 0.25).max() <= 1e-16


def test_hand_worked():
    """Logits (1, 3, 2, 3): K = 2 picks experts 1 and 3 (equal logits, lower index
    first) with weights 1/2; K = 3 adds expert 2 with weights
    (1, 1, e^-1) / (2 + e^-1)."""
    z = np.array([[1.0, 3.0, 2.0, 3.0]])
    idx, w = topk_softmax(z, 2)
    assert list(idx[0]) == [1, 3] and np.allclose(w[0], [0.5, 0.5], rtol=0, atol=1e-16)
    idx, w = topk_softmax(z, 3)
    den = 2 + math.exp(-1)
    assert list(idx[0]) == [1, 3, 2]
    assert np.allclose(w[0], [1 / den, 1 / den, math.exp(-1) / den], rtol=1e-15, atol=0)


def test_shift_invariance():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((20, 32))
    i1, w1 = topk_softmax(z, 4)
    i2, w2 = topk_softmax(z + 17.25, 4)
    assert (i1 == i2).all() and np.abs(w1 - w2).max() <= 1e-14


def test_rejects():
    with pytest.raises(ValueError):
        topk_softmax(np.zeros((2, 4)), 5)
    with pytest.raises(ValueError):
        topk_softmax(np.zeros(4), 1)
