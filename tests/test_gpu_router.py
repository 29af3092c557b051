"""GPU parity of the router step (moe_route, moe_route_bwd) against the
router oracle: expert ids bit-exact (the selection compares the same fp32
logits on both sides), weights and logit gradients within 1e-5 relative to
the row maximum (fp32 exp and sums against float64)."""
import sys

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs
from oracle import moe_router as rt

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from grouped_gemm_02_amd import binding
    binding.lib()
    return binding


CASES = [
    # (T, E, k, renorm, skew, ties)
    (2000, 128, 8, True, 0.0, False),     # the 30B layer's router
    (1500, 128, 8, True, 1.2, False),     # skewed popularity
    (1000, 128, 8, True, 0.0, True),      # many equal logits
    (500, 16, 1, True, 0.0, False),       # top-1
    (300, 1024, 8, False, 0.0, False),    # the largest expert count, no renormalisation
    (40, 1024, 1024, True, 0.0, True),    # every expert selected
    (70, 200, 65, False, 0.5, True),      # k beyond one wave's lanes
    (1, 3, 2, True, 0.0, False),
]


def _run(B, T, E, k, renorm, skew, ties, seed):
    print(f"case route T={T} E={E} k={k} renorm={renorm} skew={skew} ties={ties}", flush=True)
    z = inputs.make_router_logits(T, E, seed, DEV, skew, ties)
    shape = B.make_shape(T, 256, 128, E, k)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), -7.0, dtype=torch.float32, device=DEV)
    B.moe_route(shape, z, renorm, idx, w)
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    dw = torch.randn((T, k), generator=g, device=DEV)
    dz = torch.full((T, E), -7.0, dtype=torch.float32, device=DEV)
    B.moe_route_bwd(shape, z, idx, w, dw, renorm, dz)
    torch.cuda.synchronize()
    return z.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy().astype(np.float64), dw.cpu().numpy(), \
        dz.cpu().numpy().astype(np.float64)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.mark.parametrize("T,E,k,renorm,skew,ties", CASES)
def test_route_and_backward_match_oracle(B, T, E, k, renorm, skew, ties):
    z, idx, w, dw, dz = _run(B, T, E, k, renorm, skew, ties, seed=T + E + k)
    ridx, rw = rt.route(z, k, renorm)
    assert np.array_equal(idx, ridx), int(np.sum(idx != ridx))
    ew = _rel(w, rw)
    edz = _rel(dz, rt.route_backward(z, ridx, dw, renorm))
    print(f"  w {ew:.2e} d_logits {edz:.2e}", flush=True)
    assert ew <= TOL and edz <= TOL, (ew, edz)
    sys.stdout.flush()


def test_skew_concentrates_tokens(B):
    """The skewed logits give a skewed routing (what the router-inclusive
    benchmark relies on): the hottest expert gets several times its share."""
    T, E, k = 16384, 128, 8
    _, idx, _, _, _ = _run(B, T, E, k, True, 1.2, False, seed=5)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert counts.max() > 4 * T * k / E
    assert (idx[:, :, None] != idx[:, None, :]).sum() == T * k * (k - 1)  # distinct per token


FUSED = [
    # (T, E, k, renorm, skew, precision)
    (2000, 128, 8, True, 1.2, "bf16"),    # skewed, chunks of 128 tokens
    (1333, 64, 3, False, 0.0, "bf16"),    # 1024 % k != 0: tokens straddle chunks
    (700, 1024, 8, True, 0.0, "mxfp8"),   # the largest expert count, FP8 forward
    (257, 40, 1, True, 0.5, "bf16"),      # top-1: rows go straight to their tokens
]


@pytest.mark.parametrize("T,E,k,renorm,skew,prec", FUSED)
def test_forward_with_fused_router_matches_route_then_forward(B, T, E, k, renorm, skew, prec):
    """moe_fwd_logits (the router fused with the permutation's histogram pass)
    against moe_route followed by moe_fwd: routing, permutation, saved
    buffers and y bit for bit; the backward from either is then the same."""
    print(f"case fused router T={T} E={E} k={k} renorm={renorm} skew={skew} precision={prec}", flush=True)
    H, I = 256, 128
    z = inputs.make_router_logits(T, E, 70 + T, DEV, skew)
    cfg = inputs.LayerConfig("fused", T, H, I, E, k, "uniform", prec, 71)
    d = inputs.make_layer_inputs(cfg, DEV)
    shape = B.make_shape(T, H, I, E, k, prec)
    ref_buf, got_buf = B.LayerBuffers.allocate(shape), B.LayerBuffers.allocate(shape)
    for b in (ref_buf, got_buf):
        b.saved.fill_(0xEE)
        B.quantize_weights(b, d["W13"], d["W2"])
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), -7.0, dtype=torch.float32, device=DEV)
    B.moe_route(shape, z, renorm, idx, w)
    y_ref = B.forward(ref_buf, d["x"], idx, w, d["W13"], d["W2"])
    idx2 = torch.full((T, k), -9, dtype=torch.int32, device=DEV)
    w2 = torch.full((T, k), -9.0, dtype=torch.float32, device=DEV)
    y = B.forward_logits(got_buf, d["x"], z, renorm, idx2, w2, d["W13"], d["W2"])
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    assert torch.equal(y, y_ref)
    assert torch.equal(ref_buf.saved, got_buf.saved)
    assert B.moe_read_status(got_buf.fwd_ws) == 0
