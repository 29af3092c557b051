"""Pins for the CPU oracle: each check compares the oracle with something other
than itself (a brute-force loop written out from the definition, a dense
SwiGLU MLP computed by torch, finite differences, exact identities).

A plausible mistake anywhere in the oracle fails at least one of these:
a wrong gate/up half or transposed weight breaks the dense-MLP cases
(H != I everywhere), a wrong sign or dropped term in the SwiGLU derivative
breaks the finite differences, a missing routing weight in a weight gradient
breaks the identities, a wrong stable order breaks the permutation loop.
"""
import math

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs
from oracle import moe_oracle as orc


def _rand_layer(T, H, I, E, k, seed, distinct=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g, dtype=torch.float64)
    W13 = 0.3 * torch.randn(E, 2 * I, H, generator=g, dtype=torch.float64)
    W2 = 0.3 * torch.randn(E, H, I, generator=g, dtype=torch.float64)
    if distinct:
        idx = torch.rand(T, E, generator=g).topk(k, dim=1).indices.int()
    else:
        idx = torch.randint(0, E, (T, k), generator=g, dtype=torch.int32)
    w = torch.softmax(torch.randn(T, k, generator=g, dtype=torch.float64), 1)
    dy = torch.randn(T, H, generator=g, dtype=torch.float64)
    return [t.numpy() for t in (x, idx, w, W13, W2, dy)]


# ---------------------------------------------------------------- permutation

def _permute_by_definition(flat, E):
    """Written out from the definition with plain loops."""
    n = len(flat)
    counts = [0] * E
    for v in flat:
        if 0 <= v < E:
            counts[v] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    row_of = [-1] * n
    for f in range(n):
        e = flat[f]
        if not (0 <= e < E):
            continue
        earlier = sum(1 for g in range(f) if flat[g] == e)
        row_of[f] = offsets[e] + earlier
    src_of = [None] * offsets[E]
    for f in range(n):
        if row_of[f] >= 0:
            src_of[row_of[f]] = f
    return counts, offsets, row_of, src_of


@pytest.mark.parametrize("seed", range(6))
def test_permute_matches_definition_loops(seed):
    rng = np.random.default_rng(seed)
    T, k, E = 37, 3, 7
    idx = rng.integers(-2, E + 2, size=(T, k))  # includes invalid ids
    counts, offsets, row_of, src_of = orc.permute(idx, E)
    c2, o2, r2, s2 = _permute_by_definition(list(idx.reshape(-1)), E)
    assert counts.tolist() == c2
    assert offsets.tolist() == o2
    assert row_of.tolist() == r2
    assert src_of.tolist() == s2


def test_permute_invariants_at_30b_shape():
    T, E, k = 16384, 128, 8
    idx, _ = inputs.make_random_routing_only(T, E, k, seed=1)
    counts, offsets, row_of, src_of = orc.permute(idx, E)
    assert counts.sum() == T * k                      # per-expert counts sum to T*k
    assert offsets[0] == 0 and offsets[E] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(src_of), np.arange(T * k))   # a permutation
    assert np.array_equal(row_of[src_of], np.arange(T * k))    # inverse pair
    flat = idx.numpy().reshape(-1)
    for e in range(E):
        seg = src_of[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)               # stable: ascending f


def test_permute_zipf_has_empty_and_hot_experts():
    cfg = inputs.CONFIGS["zipf"]
    idx, _ = inputs.make_random_routing_only(cfg.T, cfg.E, cfg.k, seed=cfg.seed, routing="zipf")
    counts, *_ = orc.permute(idx, cfg.E)
    assert counts.sum() == cfg.T * cfg.k
    assert (counts == 0).sum() >= 1
    assert counts.max() > 0.10 * cfg.T * cfg.k
    # each token's experts are distinct
    srt = np.sort(idx.numpy(), axis=1)
    assert np.all(np.diff(srt, axis=1) > 0)


# ------------------------------------------------------------------- forward

def _forward_by_loops(x, idx, w, W13, W2):
    """Per-token, per-slot loops with math.exp; no matrix library."""
    T, H = x.shape
    I = W13.shape[1] // 2
    k = idx.shape[1]
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            a = []
            for i in range(I):
                g = sum(W13[e, i, h] * x[t, h] for h in range(H))
                u = sum(W13[e, I + i, h] * x[t, h] for h in range(H))
                a.append(g / (1.0 + math.exp(-g)) * u)
            for h in range(H):
                o = sum(W2[e, h, i] * a[i] for i in range(I))
                y[t][h] += w[t, j] * o
    return np.array(y)


def test_forward_matches_per_token_loops():
    x, idx, w, W13, W2, _ = _rand_layer(T=5, H=6, I=4, E=3, k=2, seed=11)
    y = orc.forward(x, idx, w, W13, W2)
    np.testing.assert_allclose(y, _forward_by_loops(x, idx, w, W13, W2), rtol=1e-12, atol=1e-12)


def _dense_mlp_torch(x, W13e, W2e):
    xt = torch.from_numpy(x)
    I = W13e.shape[0] // 2
    g = xt @ torch.from_numpy(W13e[:I]).T
    u = xt @ torch.from_numpy(W13e[I:]).T
    return (torch.nn.functional.silu(g) * u) @ torch.from_numpy(W2e).T


def test_top1_unit_weight_identical_experts_is_dense_mlp():
    T, H, I, E = 40, 24, 10, 5
    x, _, _, W13, W2, _ = _rand_layer(T, H, I, E, 1, seed=3)
    W13[:] = W13[0]
    W2[:] = W2[0]
    idx = np.random.default_rng(0).integers(0, E, size=(T, 1))
    w = np.ones((T, 1))
    y = orc.forward(x, idx, w, W13, W2)
    ref = _dense_mlp_torch(x, W13[0], W2[0]).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_topk_identical_experts_weights_summing_to_one_is_dense_mlp():
    T, H, I, E, k = 33, 16, 12, 6, 4
    x, idx, w, W13, W2, _ = _rand_layer(T, H, I, E, k, seed=4)
    W13[:] = W13[2]
    W2[:] = W2[2]
    y = orc.forward(x, idx, w, W13, W2)
    ref = _dense_mlp_torch(x, W13[2], W2[2]).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-11)


def test_single_expert_is_one_dense_gemm_pair():
    T, H, I = 19, 12, 20
    x, _, _, W13, W2, _ = _rand_layer(T, H, I, 1, 1, seed=5)
    idx = np.zeros((T, 1), dtype=np.int64)
    w = np.full((T, 1), 0.75)
    y = orc.forward(x, idx, w, W13, W2)
    ref = 0.75 * _dense_mlp_torch(x, W13[0], W2[0]).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_forward_is_linear_in_routing_weights():
    x, idx, w, W13, W2, _ = _rand_layer(T=20, H=16, I=8, E=4, k=2, seed=6)
    y1 = orc.forward(x, idx, w, W13, W2)
    y2 = orc.forward(x, idx, -2.5 * w, W13, W2)
    np.testing.assert_allclose(y2, -2.5 * y1, rtol=1e-12, atol=1e-12)


def test_duplicate_expert_in_one_token_sums_two_rows():
    x, idx, w, W13, W2, _ = _rand_layer(T=6, H=8, I=4, E=3, k=2, seed=7)
    idx[:, 1] = idx[:, 0]
    y = orc.forward(x, idx, w, W13, W2)
    y1 = orc.forward(x, idx[:, :1], (w[:, 0] + w[:, 1])[:, None], W13, W2)
    np.testing.assert_allclose(y, y1, rtol=1e-12, atol=1e-12)


def test_invalid_expert_id_drops_the_pair():
    x, idx, w, W13, W2, dy = _rand_layer(T=10, H=8, I=4, E=3, k=2, seed=8)
    bad = idx.copy()
    bad[3, 1] = 3
    bad[7, 0] = -1
    ref_w = w.copy()
    ref_w[3, 1] = 0.0
    ref_w[7, 0] = 0.0
    np.testing.assert_allclose(orc.forward(x, bad, w, W13, W2), orc.forward(x, idx, ref_w, W13, W2),
                               rtol=1e-12, atol=1e-12)
    dx, dw, dW13, dW2 = orc.backward(dy, x, bad, w, W13, W2)
    rx, rw, r13, r2 = orc.backward(dy, x, idx, ref_w, W13, W2)
    np.testing.assert_allclose(dx, rx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW13, r13, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW2, r2, rtol=1e-12, atol=1e-12)
    assert dw[3, 1] == 0.0 and dw[7, 0] == 0.0


# ------------------------------------------------------------------ backward

def _loss(dy, x, idx, w, W13, W2):
    return float(np.sum(dy * orc.forward(x, idx, w, W13, W2)))


def _tiny_layer_f64():
    """The tiny configuration's shapes (T=64, H=256, I=128, E=8, top-2)."""
    cfg = inputs.CONFIGS["tiny"]
    d = inputs.make_layer_inputs(cfg, "cpu")
    return [orc.as_f64(d[n]) if n != "topk_idx" else orc.as_i64(d[n])
            for n in ("x", "topk_idx", "topk_w", "W13", "W2", "dy")]


@pytest.fixture(scope="module")
def tiny():
    x, idx, w, W13, W2, dy = _tiny_layer_f64()
    grads = orc.backward(dy, x, idx, w, W13, W2)
    return (x, idx, w, W13, W2, dy), grads


def test_backward_directional_finite_differences(tiny):
    (x, idx, w, W13, W2, dy), (dx, dw, dW13, dW2) = tiny
    rng = np.random.default_rng(0)
    h = 1e-5
    names = {"x": (x, dx), "w": (w, dw), "W13": (W13, dW13), "W2": (W2, dW2)}
    for name, (p, gp) in names.items():
        for _ in range(20):
            v = rng.standard_normal(p.shape)
            v /= np.linalg.norm(v)
            args = {"x": x, "w": w, "W13": W13, "W2": W2}
            args[name] = p + h * v
            lp = _loss(dy, args["x"], idx, args["w"], args["W13"], args["W2"])
            args[name] = p - h * v
            lm = _loss(dy, args["x"], idx, args["w"], args["W13"], args["W2"])
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(gp * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_sampled_coordinate_finite_differences(tiny):
    (x, idx, w, W13, W2, dy), (dx, dw, dW13, dW2) = tiny
    rng = np.random.default_rng(1)
    h = 1e-4
    names = {"x": (x, dx), "w": (w, dw), "W13": (W13, dW13), "W2": (W2, dW2)}
    for name, (p, gp) in names.items():
        # 50 coordinates per tensor, half of them from rows that carry gradient
        flat_nz = np.flatnonzero(gp)
        picks = np.concatenate([rng.choice(p.size, 25, replace=False),
                                rng.choice(flat_nz, 25, replace=False)])
        for c in picks:
            args = {"x": x, "w": w, "W13": W13, "W2": W2}
            q = p.copy().reshape(-1)
            q[c] += h
            args[name] = q.reshape(p.shape)
            lp = _loss(dy, args["x"], idx, args["w"], args["W13"], args["W2"])
            q[c] -= 2 * h
            args[name] = q.reshape(p.shape)
            lm = _loss(dy, args["x"], idx, args["w"], args["W13"], args["W2"])
            fd = (lp - lm) / (2 * h)
            an = gp.reshape(-1)[c]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, c, fd, an)


def test_backward_exact_identities(tiny):
    """y is linear in w, in W2 and in the up half W3, so by Euler's theorem
    each of those inner products equals <dY, y>."""
    (x, idx, w, W13, W2, dy), (dx, dw, dW13, dW2) = tiny
    I = W13.shape[1] // 2
    L = float(np.sum(dy * orc.forward(x, idx, w, W13, W2)))
    assert math.isclose(float(np.sum(w * dw)), L, rel_tol=1e-11)
    assert math.isclose(float(np.sum(W2 * dW2)), L, rel_tol=1e-11)
    assert math.isclose(float(np.sum(W13[:, I:] * dW13[:, I:])), L, rel_tol=1e-11)


def test_backward_top1_identical_experts_matches_dense_autograd():
    T, H, I, E = 30, 20, 12, 4
    x, _, _, W13, W2, dy = _rand_layer(T, H, I, E, 1, seed=9)
    W13[:] = W13[1]
    W2[:] = W2[1]
    idx = np.random.default_rng(2).integers(0, E, size=(T, 1))
    w = np.ones((T, 1))
    dx, dw, dW13, dW2 = orc.backward(dy, x, idx, w, W13, W2)
    xt = torch.from_numpy(x).requires_grad_(True)
    W1t = torch.from_numpy(W13[1, :I].copy()).requires_grad_(True)
    W3t = torch.from_numpy(W13[1, I:].copy()).requires_grad_(True)
    W2t = torch.from_numpy(W2[1].copy()).requires_grad_(True)
    y = (torch.nn.functional.silu(xt @ W1t.T) * (xt @ W3t.T)) @ W2t.T
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dW13.sum(0)[:I], W1t.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dW13.sum(0)[I:], W3t.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dW2.sum(0), W2t.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw[:, 0], (y.detach() * torch.from_numpy(dy)).sum(1).numpy(),
                               rtol=1e-11, atol=1e-11)


def test_empty_experts_have_exactly_zero_weight_grads():
    x, idx, w, W13, W2, dy = _rand_layer(T=12, H=8, I=4, E=6, k=2, seed=10)
    idx = np.where(idx >= 4, idx - 4, idx)  # experts 4 and 5 get nothing
    idx[:, 1] = np.where(idx[:, 1] == idx[:, 0], (idx[:, 0] + 1) % 4, idx[:, 1])
    _, _, dW13, dW2 = orc.backward(dy, x, idx, w, W13, W2)
    assert not dW13[4:].any() and not dW2[4:].any()
    assert dW13[:4].any() and dW2[:4].any()


def test_restricted_subproblem_reproduces_one_experts_weight_grads(tiny):
    (x, idx, w, W13, W2, dy), (dx, dw, dW13, dW2) = tiny
    e = 5
    f, xe, ie, we, dye = orc.restrict_to_expert(x, idx, w, dy, e)
    _, _, d13, d2 = orc.backward(dye, xe, ie, we, W13[e:e + 1], W2[e:e + 1])
    np.testing.assert_allclose(d13[0], dW13[e], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(d2[0], dW2[e], rtol=1e-11, atol=1e-12)
