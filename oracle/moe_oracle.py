"""CPU oracle for the trainable MoE expert layer: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The product path (the HIP library and its
binding) never imports, links or calls it, and shares no code with it.

What it computes is the plain definition of one MoE expert layer, in float64
on the exact input values (bf16 / fp32 inputs are converted to float64, which
is exact), with no intermediate rounding:

* The layer: every token is routed to a few experts; each expert is a small
  matrix product pair; expert outputs are summed with the routing weights
  (kongchang.com explainer, section "Why MoE training needs fused kernels",
  first paragraph and the grouped-GEMM note).
* Each expert is two bias-free linear layers with SwiGLU between them
  (MarkTechPost article "Prime Intellect Releases Prime Mega MoE", section
  "How does the fused kernel work?": dispatch, the two expert linears, SwiGLU
  and combine; ic.work analysis, section on hardware constraints: only
  bias-free gated experts).
* Training needs the backward: activation gradients and weight gradients
  (ic.work analysis, section "From 3.11x to 1.32x": backward adds weight
  gradients on top of activation gradients).

Readings where the pages are silent:

* W13 is [E, 2I, H]: rows [0, I) are the gate projection W1, rows [I, 2I) the
  up projection W3. W2 is [E, H, I]. Both are nn.Linear-style (h = W x).
* SwiGLU: a = silu(g) * u with silu(g) = g * sigmoid(g); no clamp, no bias.
* topk_w is used as given (no renormalisation); d_topk_w is the raw dL/dw.
* The permutation groups the (token, slot) pairs of each expert in ascending
  flat index f = t * k + j (stable); offsets are unpadded prefix sums.
* An expert id outside [0, E) drops its pair (it contributes nothing).
* The loss for the backward is L = <dY, y>, so the incoming gradient is dY.

Every floating-point function here groups the pairs of one expert with a
boolean mask and uses numpy's float64 matmul as its only library step.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "permute", "forward", "backward", "expert_pairs", "restrict_to_expert",
    "silu", "sigmoid", "as_f64", "as_i64",
]


def as_f64(a) -> np.ndarray:
    """float64 copy of a numpy array or a CPU torch tensor (bf16 included)."""
    if hasattr(a, "detach"):
        t = a.detach().cpu()
        if str(t.dtype) in ("torch.bfloat16", "torch.float16"):
            t = t.float()
        return t.double().numpy()
    return np.asarray(a, dtype=np.float64)


def as_i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().cpu().long().numpy()
    return np.asarray(a, dtype=np.int64)


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    return z * sigmoid(z)


def permute(topk_idx, E: int):
    """Expert-contiguous reorder of the routed (token, slot) pairs.

    The fused pipeline starts by turning routing indices into a token reorder
    so that each expert's rows are contiguous, indexed by group offsets
    (kongchang.com explainer, grouped-GEMM note).

    Returns (counts[E], offsets[E+1], row_of[T*k], src_of[M]) as int64:
      counts[e]  = number of pairs f with topk_idx.flat[f] == e
      offsets    = exclusive prefix sum of counts, offsets[E] = M
      row_of[f]  = offsets[e] + #{f' < f : idx[f'] == e}, or -1 if idx[f]
                   is not a valid expert id
      src_of[r]  = the pair f with row_of[f] == r
    """
    flat = as_i64(topk_idx).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    # a stable sort by expert id is exactly "ascending f inside each expert";
    # invalid pairs get the key E so they sort after every valid one
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    M = int(offsets[E])
    src_of = order[:M].astype(np.int64)
    row_of = np.full(flat.shape[0], -1, dtype=np.int64)
    row_of[src_of] = np.arange(M, dtype=np.int64)
    return counts, offsets, row_of, src_of


def expert_pairs(topk_idx, e: int) -> np.ndarray:
    """Flat pair indices f (ascending) routed to expert e."""
    flat = as_i64(topk_idx).reshape(-1)
    return np.nonzero(flat == e)[0]


def forward(x, topk_idx, topk_w, W13, W2, return_pairs: bool = False):
    """y[t] = sum_j w[t,j] * W2[e] (silu(W1[e] x[t]) * (W3[e] x[t])),  e = idx[t,j].

    Returns y [T, H] (float64). With return_pairs, also a dict of per-pair
    float64 arrays indexed by the flat pair f: g, u, a [T*k, I] and o [T*k, H]
    (o is the expert output before the routing weight).
    """
    x = as_f64(x)
    W13 = as_f64(W13)
    W2 = as_f64(W2)
    w = as_f64(topk_w)
    idx = as_i64(topk_idx)
    T, H = x.shape
    E, I2, H2 = W13.shape
    assert H2 == H and I2 % 2 == 0
    I = I2 // 2
    k = idx.shape[1]
    wf = w.reshape(-1)
    y = np.zeros((T, H))
    pairs = None
    if return_pairs:
        pairs = {"g": np.zeros((T * k, I)), "u": np.zeros((T * k, I)),
                 "a": np.zeros((T * k, I)), "o": np.zeros((T * k, H))}
    for e in range(E):
        f = expert_pairs(idx, e)
        if f.size == 0:
            continue
        t = f // k
        X = x[t]
        G = X @ W13[e, :I].T
        U = X @ W13[e, I:].T
        A = silu(G) * U
        O = A @ W2[e].T
        np.add.at(y, t, wf[f][:, None] * O)
        if return_pairs:
            pairs["g"][f] = G
            pairs["u"][f] = U
            pairs["a"][f] = A
            pairs["o"][f] = O
    if return_pairs:
        return y, pairs
    return y


def backward(dy, x, topk_idx, topk_w, W13, W2):
    """Gradients of L = <dY, y> for the forward above.

    For each pair f = (t, j) routed to expert e, with g, u, a, o as in the
    forward and w = topk_w[t, j]:
      d_topk_w[t, j] = <dY[t], o>
      dO  = w * dY[t]
      dA  = W2[e]^T dO
      dg  = dA * u * sigmoid(g) * (1 + g * (1 - sigmoid(g)))
      du  = dA * silu(g)
      dx[t]    += W13[e]^T [dg; du]
      dW13[e]  += [dg; du] x[t]^T
      dW2[e]   += dO a^T
    Returns (dx [T,H], d_topk_w [T,k], dW13 [E,2I,H], dW2 [E,H,I]) in float64.
    Experts with no pairs get exactly-zero weight gradients.
    """
    dy = as_f64(dy)
    x = as_f64(x)
    W13 = as_f64(W13)
    W2 = as_f64(W2)
    w = as_f64(topk_w)
    idx = as_i64(topk_idx)
    T, H = x.shape
    E, I2, _ = W13.shape
    I = I2 // 2
    k = idx.shape[1]
    wf = w.reshape(-1)
    dx = np.zeros((T, H))
    dwf = np.zeros(T * k)
    dW13 = np.zeros((E, I2, H))
    dW2 = np.zeros((E, H, I))
    for e in range(E):
        f = expert_pairs(idx, e)
        if f.size == 0:
            continue
        t = f // k
        X = x[t]
        G = X @ W13[e, :I].T
        U = X @ W13[e, I:].T
        S = sigmoid(G)
        A = G * S * U
        O = A @ W2[e].T
        D = dy[t]
        dwf[f] = np.sum(D * O, axis=1)
        dO = wf[f][:, None] * D
        dA = dO @ W2[e]
        dG = dA * U * S * (1.0 + G * (1.0 - S))
        dU = dA * G * S
        dH = np.concatenate([dG, dU], axis=1)
        np.add.at(dx, t, dH @ W13[e])
        dW13[e] = dH.T @ X
        dW2[e] = dO.T @ A
    return dx, dwf.reshape(T, k), dW13, dW2


def restrict_to_expert(x, topk_idx, topk_w, dy, e: int):
    """The sub-problem that alone determines dW13[e] and dW2[e]: the pairs
    routed to expert e, each as its own token with k = 1 and E = 1.

    Returns (f, x_e [n,H], idx_e [n,1] zeros, w_e [n,1], dy_e [n,H]) as
    float64/int64 arrays; f are the flat pair ids (ascending).
    """
    idx = as_i64(topk_idx)
    k = idx.shape[1]
    f = expert_pairs(idx, e)
    t = f // k
    xe = _take_rows(x, t)
    we = as_f64(topk_w).reshape(-1)[f].reshape(-1, 1)
    dye = None if dy is None else _take_rows(dy, t)
    return f, xe, np.zeros((f.size, 1), dtype=np.int64), we, dye


def _take_rows(a, rows: np.ndarray) -> np.ndarray:
    """float64 rows of a numpy array or a (possibly device) torch tensor,
    gathering before the host copy so only the rows travel."""
    if hasattr(a, "detach"):
        import torch
        return as_f64(a[torch.as_tensor(rows, dtype=torch.long, device=a.device)])
    return as_f64(a)[rows]
