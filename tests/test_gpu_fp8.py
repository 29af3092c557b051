"""GPU parity of the FP8 precisions against the oracle's FP8 emulation.

Quantizers (activation rows and weight stacks) must match the oracle bit for
bit: codes and scale bytes. Layer outputs and gradients must be within the
FP8 max-relative-error bound (normwise by the reference maximum): small
layers element by element, the page-sized layers on sampled tokens and
experts that the oracle computes one by one.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs
from oracle import moe_fp8 as f8
from oracle import moe_oracle as orc
from tests.helpers import TOL_FP8, max_rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
MODES = ["fp8_block", "mxfp8", "fp8_bwd"]            # E8M0 (power-of-two) scales
F32_MODES = ["fp8_block_f32", "fp8_bwd_f32"]         # fp32 block scales
ALL_MODES = MODES + F32_MODES


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


def _rule(mode):
    return (32, "mx_floor") if mode == "mxfp8" else (128, "pow2_ceil")


def _np(t):
    return t.detach().cpu().numpy()


# --------------------------------------------------------------- quantizers

def _awkward_rows(rows, K, seed):
    """bf16 rows spanning the whole exponent range plus the edge cases of
    the encoder: zero blocks, exact ties, saturation, subnormal inputs."""
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(torch.empty(rows, 1).uniform_(-60, 60, generator=g))
    x = torch.randn(rows, K, generator=g) * mag
    x[0] = 0.0                                   # all-zero row
    x[1, :128] = 0.0                             # one zero block
    x[1, 5] = -0.0
    # exact midpoints between E4M3 neighbours in a block scaled by 2^0
    # (max 448 -> blockwise e = 0; MX e = 0 as well since 256 <= 448 < 512)
    mids = torch.tensor([1.0625, 1.1875, 3.25, 0.01171875, 0.001953125 * 1.5, 240.0, 208.0, 448.0])
    x[2] = mids.repeat(K // 8)
    x[3] = -x[2]
    x[4] = torch.randn(K, generator=g) * 1e-39   # bf16 subnormals
    x[5] = torch.randn(K, generator=g) * 6e37    # near the top of the range
    x[6, :] = 1.0
    x[6, ::32] = 960.0                           # 1.875 * 2^9: saturates under the MX rule
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("mode", ALL_MODES)
def test_quantize_rows_bit_exact(B, mode):
    rows, K = 300, 1024
    _say(f"case quantize_rows mode={mode} rows={rows} K={K}")
    x = _awkward_rows(rows, K, 20)
    shape = B.make_shape(1, 256, 128, 1, 1, mode)
    codes = torch.empty(rows, K, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device=DEV)
    B.moe_quantize_rows(shape, x.to(DEV), rows, K, codes, scales)
    torch.cuda.synchronize()
    if mode in F32_MODES:  # codes and the float scales [rows, K/128] bit for bit
        rc, rs, _ = f8.quantize_along_last_f32(orc.as_f64(x), 128)
        gc, gs = _np(codes), _np(scales).view(np.float32)
        bad = np.argwhere(gc != rc)
        assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[:5].tolist()}"
        assert np.array_equal(gs.view(np.uint32), rs.astype(np.float32).view(np.uint32))
        return
    block, rule = _rule(mode)
    rc, re, _ = f8.quantize_along_last(orc.as_f64(x), block, rule)
    rs = np.repeat(re + 127, block // 32, axis=-1).astype(np.uint8)
    gc, gs = _np(codes), _np(scales)
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, f"{len(bad)} code mismatches, first {bad[:5].tolist()}"
    assert np.array_equal(gs, rs)


def _tile_bytes(e, transpose):
    """Per-(row, 32-block) scale bytes of 128x128 tile exponents e [E, RB, CB]."""
    if transpose:
        e = np.swapaxes(e, -1, -2)
    return np.repeat(np.repeat(e + 127, 128, axis=1), 4, axis=2).astype(np.uint8)


@pytest.mark.parametrize("mode", ALL_MODES)
def test_quantize_weights_bit_exact(B, mode):
    E, H, I = 3, 512, 384
    _say(f"case quantize_weights mode={mode} E={E} H={H} I={I}")
    g = torch.Generator().manual_seed(21)
    W13 = torch.randn(E, 2 * I, H, generator=g) * torch.tensor([1e-3, 1.0, 5e3]).view(E, 1, 1)
    W2 = torch.randn(E, H, I, generator=g) * torch.tensor([7.0, 2e-2, 1e-30]).view(E, 1, 1)
    W13[1, :128, :128] = 0.0                   # a zero tile
    W2[0, 128:256, 0:128] = 448.0              # a tile at exactly 448
    W13, W2 = W13.to(torch.bfloat16), W2.to(torch.bfloat16)
    shape = B.make_shape(1, H, I, E, 1, mode)
    L = B.moe_get_wq_layout(shape)
    wq = torch.zeros(L["total"], dtype=torch.uint8, device=DEV)
    B.moe_quantize_weights(shape, W13.to(DEV), W2.to(DEV), wq)
    torch.cuda.synchronize()
    wq = _np(wq)
    w13, w2 = orc.as_f64(W13), orc.as_f64(W2)

    def region(name, n):
        return wq[L[name]:L[name] + n]

    def expect(w, transpose):
        if mode == "mxfp8":
            src = np.swapaxes(w, -1, -2) if transpose else w
            c, e, _ = f8.quantize_along_last(src, 32, "mx_floor")
            return c, (e + 127).astype(np.uint8)
        if mode in F32_MODES:  # one float per (row, 128 codes): the tile's scale on each of its rows
            c, sc, _ = f8.quantize_tiles_f32(w, 128)
            sc = np.swapaxes(sc, -1, -2) if transpose else sc
            return (np.swapaxes(c, -1, -2) if transpose else c), \
                np.repeat(sc.astype(np.float32), 128, axis=1).view(np.uint8)
        c, e, _ = f8.quantize_tiles(w, 128, "pow2_ceil")
        return (np.swapaxes(c, -1, -2) if transpose else c), _tile_bytes(e, transpose)

    uses = [("w2t", w2, True), ("w13t", w13, True)]
    if mode not in ("fp8_bwd", "fp8_bwd_f32"):
        uses += [("w13", w13, False), ("w2", w2, False)]
    else:
        assert L["w13"] == 2 ** 64 - 1 and L["w2"] == 2 ** 64 - 1
    for name, w, tr in uses:
        c, s = expect(w, tr)
        got_c = region(name, c.size).reshape(c.shape)
        got_s = region(name + "_scale", s.size).reshape(s.shape)
        assert np.array_equal(got_c, c), (name, int(np.sum(got_c != c)))
        assert np.array_equal(got_s, s), name


def _token_matrix(rows, C, seed):
    """bf16 rows whose magnitudes differ by up to 2^40, so that blocks along
    the rows mix scales; zero, tie, saturation and subnormal columns."""
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(torch.empty(rows, 1).uniform_(-14, 14, generator=g))
    x = torch.randn(rows, C, generator=g) * mag
    x[:, 0] = 0.0                                              # an all-zero column
    mids = torch.tensor([1.0625, 1.1875, 3.25, 0.01171875, 240.0, 208.0, 448.0, -448.0])
    x[:, 1] = mids.repeat(rows // 8 + 1)[:rows]                # ties at scale 2^0
    x[:, 2] = 1.0
    x[::32, 2] = 960.0                                         # saturates under the MX rule
    x[:, 3] = torch.randn(rows, generator=g) * 1e-39           # bf16 subnormals
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("gather", [False, True])
def test_quantize_tokens_bit_exact(B, mode, gather):
    """The weight-gradient quantizer: per expert (rows in permuted order,
    from token rows when gathering), every column in 128-row (32 for MX)
    blocks; codes and scale bytes equal the oracle's."""
    T, k, E, C = 700, 2, 6, 384
    _say(f"case quantize_tokens mode={mode} gather={gather} T={T} k={k} E={E} C={C}")
    idx, _ = inputs.make_random_routing_only(T, E, k, 22, DEV, "zipf")
    idx[idx == 4] = 5                                          # expert 4 gets no rows
    shape = B.make_shape(T, 256, 128, E, k, mode)
    n = T * k
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_of = torch.empty(n, dtype=torch.int32, device=DEV)
    src_of = torch.empty(n, dtype=torch.int32, device=DEV)
    scratch = torch.zeros(B.moe_permute_scratch_bytes(shape), dtype=torch.uint8, device=DEV)
    B.moe_permute(shape, idx, counts, offsets, row_of, src_of, scratch)
    rows_in = T if gather else n
    x = _token_matrix(rows_in, C + 128, 23)                    # ld = C + 128: extra columns stay unread
    K = B.wgrad_rows_cap(shape)
    codes = torch.full((C * K,), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((C * K // 32,), 0xAB, dtype=torch.uint8, device=DEV)
    B.moe_quantize_tokens(shape, x.to(DEV), C + 128, C, counts, offsets, src_of if gather else None, codes, scales)
    torch.cuda.synchronize()
    gc, gs = _np(codes), _np(scales)
    block, rule = _rule(mode)
    xs = orc.as_f64(x)[:, :C]
    _, ro, _, rsrc = orc.permute(_np(idx), E)
    poff = 0
    for e in range(E):
        r0, r1 = int(ro[e]), int(ro[e + 1])
        kp = -(-(r1 - r0) // 128) * 128
        seg = xs[rsrc[r0:r1] // k] if gather else xs[r0:r1]
        pad = np.zeros((kp, C))
        pad[:r1 - r0] = seg
        rc, re, _ = f8.quantize_along_last(pad.T, block, rule)  # [C, kp], [C, kp / block]
        rs = np.repeat(re + 127, block // 32, axis=-1).astype(np.uint8)
        got_c = gc[C * poff:C * (poff + kp)].reshape(C, kp)
        got_s = gs[C * poff // 32:C * (poff + kp) // 32].reshape(C, kp // 32)
        assert np.array_equal(got_c, rc), (e, int(np.sum(got_c != rc)))
        assert np.array_equal(got_s, rs), e
        poff += kp


# --------------------------------------------------------------- layer

def run_layer(B, cfg, d, mode, wgrad="bf16"):
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, mode, wgrad=wgrad)
    buf = B.LayerBuffers.allocate(shape)
    buf.fwd_ws.fill_(0xFF)
    buf.bwd_ws.fill_(0xFF)
    buf.saved.fill_(0xFF)
    buf.wq.fill_(0xFF)
    B.quantize_weights(buf, d["W13"], d["W2"])
    y = B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    dx, dw, dW13, dW2 = B.backward(buf, d["dy"], d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    torch.cuda.synchronize()
    Tk = cfg.T * cfg.k
    return {
        "y": y, "dx": dx, "dw": dw, "dW13": dW13, "dW2": dW2,
        "counts": buf.saved_view("counts", torch.int32, cfg.E).clone(),
        "h13": buf.saved_view("h13", torch.bfloat16, Tk * 2 * cfg.I).view(Tk, 2 * cfg.I).clone(),
        "act": buf.saved_view("act", torch.bfloat16, Tk * cfg.I).view(Tk, cfg.I).clone(),
        "status": B.moe_read_status(buf.fwd_ws),
    }


SMALL = [
    inputs.CONFIGS["tiny"],
    inputs.LayerConfig("mid", 600, 512, 384, 7, 3, "uniform", "bf16", 10),
    inputs.LayerConfig("skew", 333, 256, 128, 16, 4, "zipf", "bf16", 11, zipf_s=1.2, zipf_cold=5),
    inputs.LayerConfig("top1", 257, 768, 128, 40, 1, "uniform", "bf16", 13),
]
# the maximum expert count under skew (MX only: the oracle's weight
# quantization of 1024 experts takes ~25 s, so it runs once per mode here)
MAXE = inputs.LayerConfig("max_experts_zipf", 700, 256, 128, 1024, 8, "zipf", "bf16", 16, zipf_s=1.1,
                          zipf_cold=100)
CASES = [(c, m) for c in SMALL for m in ALL_MODES] + [(MAXE, "mxfp8")]

_WQ = {}


def _oracle_wq(cfg, mode, d):
    """The oracle's quantized weights of a configuration's seeded weights
    (the same values in every test that makes this configuration's inputs),
    computed once per (configuration, mode)."""
    key = (cfg.name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.seed, mode)
    if key not in _WQ:
        _WQ[key] = f8.quantize_weights(d["W13"], d["W2"], mode)
    return _WQ[key]
# Hot experts whose weight-gradient tiles are split along the expert's rows
# (2813 rows into 4 ranges, 1179 into 4), under both row-block rules (128
# rows, power-of-two; 32 rows, MX).
HOT = inputs.LayerConfig("hot", 8192, 512, 384, 32, 1, "zipf", "bf16", 21, zipf_s=1.2, zipf_cold=8)
WGRAD_CASES = [(c, m) for c, m in CASES if m in MODES] + [(HOT, "fp8_block"), (HOT, "mxfp8")]


@pytest.mark.parametrize("cfg,mode", CASES, ids=[f"{c.name}-{m}" for c, m in CASES])
def test_fp8_layer_matches_oracle_elementwise(B, cfg, mode):
    cfg = cfg.scaled(precision=mode)
    _say(f"case {inputs.describe(cfg)}")
    _fp8_elementwise(B, cfg, mode, inputs.make_layer_inputs(cfg, DEV))


DUP = inputs.LayerConfig("dup", 500, 512, 384, 6, 3, "uniform", "bf16", 31)


@pytest.mark.parametrize("mode", ALL_MODES)
def test_fp8_duplicate_expert_in_one_token_elementwise(B, mode):
    """Every third token names one expert in two of its slots (two rows,
    summed)."""
    cfg = DUP.scaled(precision=mode)
    _say(f"case duplicate experts {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    idx = d["topk_idx"].clone()
    idx[::3, 1] = idx[::3, 0]
    d["topk_idx"] = idx
    _WQ.pop((cfg.name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.seed, mode), None)
    _fp8_elementwise(B, cfg, mode, d)


def _fp8_elementwise(B, cfg, mode, d):
    out = run_layer(B, cfg, d, mode)
    assert out["status"] == 0
    args = (d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    wq = _oracle_wq(cfg, mode, d)
    y_ref, pairs = f8.forward(*args, mode, return_pairs=True, wq=wq)
    dx_ref, dw_ref, dW13_ref, dW2_ref = f8.backward(d["dy"], *args, mode, wq=wq)
    errs = {
        "y": max_rel_err(orc.as_f64(out["y"]), y_ref),
        "dx": max_rel_err(orc.as_f64(out["dx"]), dx_ref),
        "d_topk_w": max_rel_err(orc.as_f64(out["dw"]), dw_ref),
        "dW13": max_rel_err(orc.as_f64(out["dW13"]), dW13_ref),
        "dW2": max_rel_err(orc.as_f64(out["dW2"]), dW2_ref),
    }
    _, _, _, src_of = orc.permute(d["topk_idx"], cfg.E)
    M, I = src_of.size, cfg.I
    h13 = orc.as_f64(out["h13"])[:M]
    errs["g"] = max_rel_err(h13[:, :I], pairs["g"][src_of])
    errs["u"] = max_rel_err(h13[:, I:], pairs["u"][src_of])
    wf = orc.as_f64(d["topk_w"]).reshape(-1)
    wa_ref = pairs["wa"] if "wa" in pairs else pairs["a"] * wf[:, None]
    errs["wa"] = max_rel_err(orc.as_f64(out["act"])[:M], wa_ref[src_of])
    _say(f"{cfg.name}/{mode}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL_FP8, (k, v)
    counts = _np(out["counts"])
    for e in np.nonzero(counts == 0)[0]:
        assert not out["dW13"][e].any() and not out["dW2"][e].any()


@pytest.mark.parametrize("cfg,mode", WGRAD_CASES, ids=[f"{c.name}-{m}" for c, m in WGRAD_CASES])
def test_fp8_weight_gradients_match_oracle_elementwise(B, cfg, mode):
    """MOE_FLAG_FP8_WGRAD: dW13 and dW2 from operands quantized along each
    expert's rows; the other outputs equal those of the default reading."""
    cfg = cfg.scaled(precision=mode)
    _say(f"case fp8 wgrad {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    out = run_layer(B, cfg, d, mode, wgrad="fp8")
    base = run_layer(B, cfg, d, mode)
    assert out["status"] == 0
    for k in ("y", "dx", "dw"):
        assert torch.equal(out[k], base[k]), k
    args = (d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    wq = _oracle_wq(cfg, mode, d)
    _, _, dW13_ref, dW2_ref = f8.backward(d["dy"], *args, mode, wq=wq, wgrad="fp8")
    errs = {"dW13": max_rel_err(orc.as_f64(out["dW13"]), dW13_ref),
            "dW2": max_rel_err(orc.as_f64(out["dW2"]), dW2_ref)}
    _say(f"{cfg.name}/{mode}/wgrad fp8: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL_FP8, (k, v)
    counts = _np(out["counts"])
    for e in np.nonzero(counts == 0)[0]:
        assert not out["dW13"][e].any() and not out["dW2"][e].any()


def test_fp8_layer_deterministic_bitwise(B):
    cfg = SMALL[1].scaled(precision="mxfp8")
    _say(f"case determinism {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    a = run_layer(B, cfg, d, "mxfp8")
    b = run_layer(B, cfg, d, "mxfp8")
    for k in ("y", "dx", "dw", "dW13", "dW2", "h13", "act"):
        assert torch.equal(a[k], b[k]), k


def test_fp8_zero_tokens(B):
    cfg = inputs.LayerConfig("empty", 0, 256, 128, 4, 2, "uniform", "fp8_block", 16)
    d = inputs.make_layer_inputs(cfg, DEV)
    out = run_layer(B, cfg, d, "fp8_block")
    assert not out["dW13"].any() and not out["dW2"].any()


# --------------------------------------------------------------- page-sized layers, sampled

_WQ_EXPERT = {}


def _expert_wq(cfg, mode, d, experts, keys):
    """The oracle's quantized weights of the given experts of a configuration
    (cached per configuration, mode and expert; the oracle's weight blocks
    never straddle experts, so an expert's quantization is its own). Experts
    not yet cached are quantized on a pool of threads: numpy releases the
    interpreter lock in the quantizer's array operations."""
    from concurrent.futures import ThreadPoolExecutor
    key = (cfg.name, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.seed, mode)
    for other in [k for k in _WQ_EXPERT if k != key]:  # one configuration's weights at a time
        del _WQ_EXPERT[other]
    cache = _WQ_EXPERT.setdefault(key, {})
    todo = sorted({int(e) for e in experts} - set(cache))
    if todo:
        W13, W2 = d["W13"].cpu(), d["W2"].cpu()
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            res = ex.map(lambda e: f8.quantize_weights(W13[e:e + 1], W2[e:e + 1], mode, keys), todo)
            for e, r in zip(todo, res):
                cache[e] = r
    return cache


def _check_experts(counts):
    """The hottest expert (the one split along its rows, under skew), the
    coldest non-empty one and two of median row count."""
    nz = np.nonzero(counts > 0)[0]
    order = nz[np.argsort(counts[nz], kind="stable")]
    picks = [int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(order[(len(order) - 1) // 2 - 1])]
    out = []
    for e in picks:
        if e not in out:
            out.append(e)
    return out


def _sampled_check(B, cfg, n_tokens=64, wgrad="bf16"):
    """The page-sized FP8 layer on `n_tokens` tokens drawn uniformly over
    [0, T) (seeded) and on four experts (hottest, coldest non-empty, two
    median), each computed by the oracle on its own: a token needs only its k
    experts' weights and an expert's weight gradients only its own rows."""
    mode = cfg.precision
    t0 = time.time()
    _say(f"case full-size {inputs.describe(cfg)} wgrad={wgrad} tokens={n_tokens}")
    d = inputs.make_layer_inputs(cfg, DEV)
    out = run_layer(B, cfg, d, mode, wgrad=wgrad)
    assert out["status"] == 0
    counts = _np(out["counts"])
    idx_h = _np(d["topk_idx"])
    assert np.array_equal(counts, np.bincount(idx_h.reshape(-1), minlength=cfg.E))
    _say(f"  gpu done {time.time() - t0:.1f}s")
    toks = np.sort(np.random.default_rng(1000 + cfg.seed).choice(cfg.T, n_tokens, replace=False))
    experts = _check_experts(counts)
    keys = ("W2b", "W13b") if mode in f8.BF16_FORWARD_MODES else ("W13q", "W2q", "W2b", "W13b")
    cache = _expert_wq(cfg, mode, d, set(idx_h[toks].reshape(-1).tolist()) | set(experts), keys)
    _say(f"  {len(cache)} experts' weights quantized by the oracle ({time.time() - t0:.1f}s)")

    def wq_of(ex):
        return {k: np.concatenate([cache[e][k] for e in ex]) for k in cache[ex[0]]}

    ys, yr, dxs, dxr, dws, dwr = [], [], [], [], [], []
    for t in toks:
        ex = [int(e) for e in idx_h[t]]
        wq = wq_of(ex)
        sub = (d["x"][t:t + 1], np.arange(cfg.k).reshape(1, -1), d["topk_w"][t:t + 1], d["W13"][ex], d["W2"][ex])
        yr.append(f8.forward(*sub, mode, wq=wq)[0])
        gx, gw, _, _ = f8.backward(d["dy"][t:t + 1], *sub, mode, wq=wq)
        dxr.append(gx[0])
        dwr.append(gw[0])
        ys.append(orc.as_f64(out["y"][t]))
        dxs.append(orc.as_f64(out["dx"][t]))
        dws.append(orc.as_f64(out["dw"][t]))
    errs = {"y": max_rel_err(np.array(ys), np.array(yr)),
            "dx": max_rel_err(np.array(dxs), np.array(dxr)),
            "d_topk_w": max_rel_err(np.array(dws), np.array(dwr))}
    # and per token row
    errs["y_row"] = max(max_rel_err(a, b) for a, b in zip(ys, yr))
    errs["dx_row"] = max(max_rel_err(a, b) for a, b in zip(dxs, dxr))
    _say(f"  {n_tokens} tokens (first {toks[:4].tolist()}, last {toks[-1]}) done {time.time() - t0:.1f}s")
    for e in experts:
        f, xe, ie, we, dye = orc.restrict_to_expert(d["x"], d["topk_idx"], d["topk_w"], d["dy"], e)
        _, _, r13, r2 = f8.backward(dye, xe, ie, we, d["W13"][e:e + 1], d["W2"][e:e + 1], mode, wq=wq_of([e]),
                                    wgrad=wgrad)
        errs[f"dW13[{e}:{counts[e]}]"] = max_rel_err(orc.as_f64(out["dW13"][e]), r13[0])
        errs[f"dW2[{e}:{counts[e]}]"] = max_rel_err(orc.as_f64(out["dW2"][e]), r2[0])
    for e in np.nonzero(counts == 0)[0]:
        assert not out["dW13"][e].any() and not out["dW2"][e].any(), e
    _say(f"{cfg.name}/{mode}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items())
         + f" ({time.time() - t0:.1f}s)")
    for k, v in errs.items():
        assert v <= TOL_FP8, (k, v)
    for k in ("y", "dx", "dW13", "dW2"):
        assert torch.isfinite(out[k].float()).all(), k


def test_ep8_share_fp8_block_f32_sampled(B):
    cfg = inputs.CONFIGS["ep8_share"]
    assert cfg.precision == "fp8_block_f32"      # the workload's stated fp32 block scales
    _sampled_check(B, cfg)


def test_ep8_share_fp8_block_pow2_sampled(B):
    _sampled_check(B, inputs.CONFIGS["ep8_share"].scaled(precision="fp8_block"))


def test_ep8_share_fp8_block_pow2_fp8_wgrad_sampled(B):
    _sampled_check(B, inputs.CONFIGS["ep8_share"].scaled(precision="fp8_block"), wgrad="fp8")


def test_qwen3_235b_fp8_bwd_f32_sampled(B):
    cfg = inputs.CONFIGS["qwen3_235b"]
    assert cfg.precision == "fp8_bwd_f32"
    _sampled_check(B, cfg)


def test_qwen3_235b_fp8_bwd_pow2_sampled(B):
    _sampled_check(B, inputs.CONFIGS["qwen3_235b"].scaled(precision="fp8_bwd"))


def test_qwen3_235b_fp8_bwd_pow2_fp8_wgrad_sampled(B):
    _sampled_check(B, inputs.CONFIGS["qwen3_235b"].scaled(precision="fp8_bwd"), wgrad="fp8")


def test_qwen3_30b_zipf_mxfp8_sampled(B):
    _sampled_check(B, inputs.CONFIGS["zipf"])


def test_qwen3_30b_zipf_mxfp8_fp8_wgrad_sampled(B):
    _sampled_check(B, inputs.CONFIGS["zipf"], wgrad="fp8")


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8", "fp8_block_f32", "fp8_bwd_f32"])
def test_fp8_steps_run_without_bf16_weights(B, mode):
    """Where a step reads only the quantized weights (every FP8 backward; the
    FP8 forwards except fp8_bwd's bf16 one), W13 and W2 may be NULL: the
    results equal those of a call that passes them."""
    cfg = SMALL[1].scaled(precision=mode)
    _say(f"case no bf16 weights {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    ref = run_layer(B, cfg, d, mode)
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, mode)
    buf = B.LayerBuffers.allocate(shape)
    B.quantize_weights(buf, d["W13"], d["W2"])
    fwd_w = (d["W13"], d["W2"]) if mode in f8.BF16_FORWARD_MODES else (None, None)
    y = B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], *fwd_w)
    got = B.backward(buf, d["dy"], d["x"], d["topk_idx"], d["topk_w"], None, None)
    torch.cuda.synchronize()
    assert torch.equal(y, ref["y"])
    for k, g in zip(("dx", "dw", "dW13", "dW2"), got):
        assert torch.equal(g, ref[k]), k
