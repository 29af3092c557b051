"""CPU oracle of the router step before the layer: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module; it shares no code with the HIP
path.

The pages leave the router outside the measured layer and criticise exactly
that, together with uniform random routing (ic.work analysis, section on the
benchmark's idealised assumptions: the router's cost is excluded and real
token distributions are skewed). What a router computes is not on the pages;
the plain reading used here:

* probabilities p = softmax(z) over the E logits of a token;
* the k experts with the largest logits (equivalently probabilities), in
  descending order, ties broken towards the lower expert id;
* the routing weights are those probabilities, optionally renormalised to sum
  to one over the k selected (then w = softmax of the selected logits);
* the backward maps d_topk_w to d_logits through that function (the choice
  of experts is piecewise constant and has no gradient).

Everything is float64 on the exact fp32 logits.
"""
from __future__ import annotations

import numpy as np

__all__ = ["route", "route_backward"]


def _softmax(z: np.ndarray) -> np.ndarray:
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def route(logits, k: int, renorm: bool = True):
    """topk_idx int64 [T, k], topk_w float64 [T, k] for logits [T, E]."""
    z = np.asarray(logits, dtype=np.float64)
    T, E = z.shape
    ids = np.arange(E)
    idx = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((ids, -z[t]))   # by descending logit, then ascending id
        idx[t] = order[:k]
    p = _softmax(z)
    w = np.take_along_axis(p, idx, axis=1)
    if renorm:
        w = w / np.sum(w, axis=1, keepdims=True)
    return idx, w


def route_backward(logits, topk_idx, d_topk_w, renorm: bool = True):
    """d_logits float64 [T, E] of L given dL/dtopk_w, for the experts that
    route() selected (topk_idx)."""
    z = np.asarray(logits, dtype=np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    dw = np.asarray(d_topk_w, dtype=np.float64)
    d = np.zeros_like(z)
    if renorm:
        # w = softmax(z_S): dL/dz_S = w * (dw - <w, dw>), zero off S
        w = _softmax(np.take_along_axis(z, idx, axis=1))
        g = w * (dw - np.sum(w * dw, axis=1, keepdims=True))
        np.put_along_axis(d, idx, g, axis=1)
        return d
    # w = p_S with p = softmax(z): dL/dz = p * (G - <p, G>), G = dw scattered to S
    p = _softmax(z)
    G = np.zeros_like(z)
    np.put_along_axis(G, idx, dw, axis=1)
    return p * (G - np.sum(p * G, axis=1, keepdims=True))
