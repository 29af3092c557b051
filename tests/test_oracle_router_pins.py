"""Pins of the router oracle (oracle/moe_router.py): closed forms, ties, and
finite differences of the backward against the forward."""
import math

import numpy as np
import pytest

from oracle import moe_router as rt


def test_two_of_four_closed_form():
    """logits (2, 1, 0, -1), k = 2: experts 0, 1; renormalised weights are
    sigmoid(1) and 1 - sigmoid(1); without renormalisation e^2 / S, e / S
    with S = e^2 + e + 1 + 1/e."""
    idx, w = rt.route(np.array([[2.0, 1.0, 0.0, -1.0]]), 2)
    assert idx.tolist() == [[0, 1]]
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(w, [[s1, 1.0 - s1]], rtol=0, atol=1e-15)
    idx, w = rt.route(np.array([[2.0, 1.0, 0.0, -1.0]]), 2, renorm=False)
    S = math.e ** 2 + math.e + 1.0 + math.exp(-1.0)
    assert np.allclose(w, [[math.e ** 2 / S, math.e / S]], rtol=0, atol=1e-15)


def test_order_and_ties():
    """Descending logits; equal logits go to the lower expert id first."""
    z = np.array([[0.5, 3.0, 0.5, 3.0, -2.0, 0.5],
                  [1.0, 1.0, 1.0, 1.0, 1.0, 1.0]])
    idx, w = rt.route(z, 4)
    assert idx.tolist() == [[1, 3, 0, 2], [0, 1, 2, 3]]
    assert np.allclose(w[1], 0.25)
    assert np.allclose(w.sum(axis=1), 1.0)


@pytest.mark.parametrize("renorm", [True, False])
def test_backward_matches_finite_differences(renorm):
    rng = np.random.default_rng(0)
    T, E, k = 5, 12, 3
    z = rng.standard_normal((T, E)) * 2.0
    idx, w = rt.route(z, k, renorm)
    dw = rng.standard_normal((T, k))
    d = rt.route_backward(z, idx, dw, renorm)
    h = 1e-6
    num = np.zeros_like(z)
    for t in range(T):
        for i in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, i] += h
            zm[t, i] -= h
            # the selection is held fixed (it is piecewise constant in z)
            wp = _weights(zp, idx, renorm)
            wm = _weights(zm, idx, renorm)
            num[t, i] = np.sum(dw[t] * (wp[t] - wm[t])) / (2 * h)
    assert np.allclose(d, num, rtol=1e-6, atol=1e-8)
    if renorm:  # experts outside the selection get no gradient
        mask = np.ones_like(z, dtype=bool)
        np.put_along_axis(mask, idx, False, axis=1)
        assert not d[mask].any()


def _weights(z, idx, renorm):
    """Weights of a fixed selection, by the textbook formulas (not the
    oracle's code): renormalised p_S, or p_S."""
    p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, idx, axis=1)
    return ps / ps.sum(axis=1, keepdims=True) if renorm else ps


def test_k_equals_e_is_a_permutation_and_softmax():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((3, 7))
    idx, w = rt.route(z, 7, renorm=False)
    for t in range(3):
        assert sorted(idx[t].tolist()) == list(range(7))
        assert np.all(np.diff(z[t, idx[t]]) <= 0)
    assert np.allclose(w.sum(axis=1), 1.0)
