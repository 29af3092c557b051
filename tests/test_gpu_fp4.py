"""GPU parity of the FP8 x FP4 forward (MOE_FP8_FP4) against the oracle's
emulation (oracle/moe_fp4.py): the E2M1 weight quantizer bit for bit (codes
and scale bytes), the layer forward within the FP8 max-relative-error bound
(normwise), small layers element by element and the Qwen3-30B-A3B shape on
sampled tokens that the oracle computes one by one."""
import sys

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs
from oracle import moe_fp4 as f4
from oracle import moe_oracle as orc
from tests.helpers import TOL_FP8, max_rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from grouped_gemm_02_amd import binding
    binding.lib()
    return binding


def _np(t):
    return t.detach().cpu().numpy()


def _pack(codes):
    """E2M1 codes [..., C] -> bytes [..., C/2], value 2j in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_quantize_fp4_weights_bit_exact(B):
    E, H, I = 3, 512, 384
    _say(f"case quantize_weights fp8_fp4 E={E} H={H} I={I}")
    g = torch.Generator().manual_seed(31)
    W13 = torch.randn(E, 2 * I, H, generator=g) * torch.tensor([1e-3, 1.0, 5e3]).view(E, 1, 1)
    W2 = torch.randn(E, H, I, generator=g) * torch.tensor([7.0, 2e-2, 1e-30]).view(E, 1, 1)
    W13[1, 0, :32] = 0.0                                   # a zero block
    # exact E2M1 midpoints at scale 2^0 (block maximum 6: e = 0)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    W13[1, 1, :32] = mids.repeat(4)
    W13[1, 2, :32] = -mids.repeat(4)
    W13[1, 3, :32] = 7.5                                   # saturates at 6 * 2^0
    W13[1, 4, :32] = torch.randn(32, generator=g) * 1e-39  # bf16 subnormals
    W13, W2 = W13.to(torch.bfloat16), W2.to(torch.bfloat16)
    shape = B.make_shape(1, H, I, E, 1, "fp8_fp4")
    L = B.moe_get_wq_layout(shape)
    wq = torch.zeros(L["total"], dtype=torch.uint8, device=DEV)
    B.moe_quantize_weights(shape, W13.to(DEV), W2.to(DEV), wq)
    torch.cuda.synchronize()
    wq = _np(wq)
    for name, w in (("w13", W13), ("w2", W2)):
        codes, e, _ = f4.quantize_fp4_along_last(orc.as_f64(w))
        want_c = _pack(codes).reshape(-1)
        want_s = (e + 127).astype(np.uint8).reshape(-1)
        got_c = wq[L[name]:L[name] + want_c.size]
        got_s = wq[L[name + "_scale"]:L[name + "_scale"] + want_s.size]
        assert np.array_equal(got_s, want_s), (name, int(np.sum(got_s != want_s)))
        bad = np.nonzero(got_c != want_c)[0]
        assert bad.size == 0, (name, bad[:8], got_c[bad[:8]], want_c[bad[:8]])


def run_fwd(B, cfg, d):
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, "fp8_fp4")
    buf = B.LayerBuffers.allocate(shape)
    buf.fwd_ws.fill_(0xFF)
    buf.saved.fill_(0xFF)
    buf.wq.fill_(0xFF)
    B.quantize_weights(buf, d["W13"], d["W2"])
    y = B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    torch.cuda.synchronize()
    Tk = cfg.T * cfg.k
    return {"y": y, "status": B.moe_read_status(buf.fwd_ws),
            "h13": buf.saved_view("h13", torch.bfloat16, Tk * 2 * cfg.I).view(Tk, 2 * cfg.I).clone(),
            "act": buf.saved_view("act", torch.bfloat16, Tk * cfg.I).view(Tk, cfg.I).clone()}


SMALL = [
    inputs.CONFIGS["tiny"],
    inputs.LayerConfig("mid", 600, 512, 384, 7, 3, "uniform", "bf16", 10),
    inputs.LayerConfig("skew", 333, 256, 128, 16, 4, "zipf", "bf16", 11, zipf_s=1.2, zipf_cold=5),
    inputs.LayerConfig("top1", 257, 768, 128, 40, 1, "uniform", "bf16", 13),
    inputs.LayerConfig("one_token", 1, 256, 128, 8, 8, "uniform", "bf16", 14),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_fp4_forward_matches_oracle_elementwise(B, cfg):
    cfg = cfg.scaled(precision="fp8_fp4")
    _say(f"case fp8_fp4 {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV, with_dy=False)
    out = run_fwd(B, cfg, d)
    assert out["status"] == 0
    y_ref, pairs = f4.forward(d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"], return_pairs=True)
    _, _, _, src_of = orc.permute(d["topk_idx"], cfg.E)
    M, I = src_of.size, cfg.I
    h13 = orc.as_f64(out["h13"])[:M]
    errs = {"y": max_rel_err(orc.as_f64(out["y"]), y_ref),
            "g": max_rel_err(h13[:, :I], pairs["g"][src_of]),
            "u": max_rel_err(h13[:, I:], pairs["u"][src_of]),
            "wa": max_rel_err(orc.as_f64(out["act"])[:M], pairs["wa"][src_of])}
    _say(f"{cfg.name}/fp8_fp4: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL_FP8, (k, v)


def test_fp4_forward_deterministic_bitwise(B):
    cfg = SMALL[1].scaled(precision="fp8_fp4")
    d = inputs.make_layer_inputs(cfg, DEV, with_dy=False)
    a, b = run_fwd(B, cfg, d), run_fwd(B, cfg, d)
    for k in ("y", "h13", "act"):
        assert torch.equal(a[k], b[k]), k


def test_fp4_backward_refused(B):
    cfg = inputs.CONFIGS["tiny"].scaled(precision="fp8_fp4")
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, "fp8_fp4")
    buf = B.LayerBuffers.allocate(shape)
    d = inputs.make_layer_inputs(cfg, DEV)
    B.quantize_weights(buf, d["W13"], d["W2"])
    B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    with pytest.raises(B.MoEError) as ei:
        B.backward(buf, d["dy"], d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    assert ei.value.status == 4


def test_qwen3_30b_shape_fp4_sampled(B):
    """Full size: sampled tokens, each through the oracle on its own k
    experts (the oracle quantizes only those experts' weights)."""
    cfg = inputs.CONFIGS["qwen3_30b"].scaled(name="qwen3_30b_fp4", precision="fp8_fp4")
    _say(f"case full-size {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV, with_dy=False)
    out = run_fwd(B, cfg, d)
    assert out["status"] == 0
    g = np.random.default_rng(cfg.seed)
    toks = np.sort(g.choice(cfg.T, 10, replace=False))
    idx_h = d["topk_idx"].cpu()
    cache = {}  # expert -> its dequantized FP4 weights (the quantization is per expert)

    def wq_of(e):
        if e not in cache:
            cache[e] = f4.quantize_weights(d["W13"][e:e + 1], d["W2"][e:e + 1])
        return cache[e]
    ys, yr = [], []
    for t in toks:
        ex = [int(e) for e in idx_h[t]]
        wq = {key: np.concatenate([wq_of(e)[key] for e in ex]) for key in ("W13q", "W2q")}
        yr.append(f4.forward(d["x"][t:t + 1], torch.arange(cfg.k).view(1, -1), d["topk_w"][t:t + 1],
                             None, None, wq=wq)[0])
        ys.append(orc.as_f64(out["y"][t]))
    err = max_rel_err(np.array(ys), np.array(yr))
    _say(f"{cfg.name}: y={err:.2e}")
    assert err <= TOL_FP8
    assert torch.isfinite(out["y"].float()).all()
