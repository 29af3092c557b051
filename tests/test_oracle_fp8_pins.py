"""Pins for the oracle's FP8 emulation (oracle/moe_fp8.py).

Independent references: E4M3 values fixed by the format's bit fields (OCP
8-bit floating point, E4M3 with exponent bias 7: code 0x38 is 1.0, 0x40 is
2.0, 0x7E is 448; an E8M0 scale byte b is 2^(b - 127)), the defining
properties of the scale rules and of round-to-nearest-even, and a per-token
loop implementation of the quantized layer with its own scalar rounding
(math.frexp based) on tiny inputs.
"""
import math
import struct

import numpy as np
import pytest

from oracle import moe_fp8 as f8
from oracle import moe_oracle as orc


def test_e4m3_anchor_values():
    t = f8.e4m3_decode_table()
    assert t[0x38] == 1.0 and t[0x40] == 2.0          # exponent field 7 and 8, bias 7
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0     # largest finite magnitude
    assert t[0x08] == 2.0 ** -6                       # smallest normal
    assert t[0x01] == 2.0 ** -9                       # smallest subnormal
    assert t[0x00] == 0.0 and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t[np.r_[0:0x7F, 0x80:0xFF]]).all()


def test_e4m3_monotone_and_round_trip():
    t = f8.e4m3_decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    codes = np.r_[0:0x7F, 0x81:0xFF].astype(np.uint8)
    assert np.array_equal(f8.e4m3_encode(t[codes]), codes)


def test_e4m3_ties_to_even_and_saturation():
    t = f8.e4m3_decode_table()
    for c in range(0, 0x7E):
        lo, hi = t[c], t[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert f8.e4m3_encode(mid) == even, c
        assert f8.e4m3_encode(np.nextafter(mid, hi)) == c + 1
        assert f8.e4m3_encode(np.nextafter(mid, lo)) == c
        assert f8.e4m3_encode(-mid) == (even | 0x80 if even else 0)
    assert f8.e4m3_encode(1e9) == 0x7E and f8.e4m3_encode(-1e9) == 0xFE
    assert f8.e4m3_encode(460.0) == 0x7E


def test_scale_exponent_rules():
    rng = np.random.default_rng(0)
    amax = np.exp(rng.uniform(-40, 40, size=20000))
    amax = np.concatenate([amax, [448.0, 449.0, 224.0, 1.0, 2.0 ** -30, 256.0, 512.0]])
    e = f8.scale_exponent(amax, "pow2_ceil")
    assert np.all(448.0 * np.ldexp(1.0, e) >= amax)
    assert np.all(448.0 * np.ldexp(1.0, e - 1) < amax)
    e = f8.scale_exponent(amax, "mx_floor")
    assert np.all(np.ldexp(1.0, e + 8) <= amax)
    assert np.all(np.ldexp(1.0, e + 9) > amax)
    assert f8.scale_exponent(np.zeros(3), "pow2_ceil").tolist() == [0, 0, 0]
    assert f8.scale_exponent(np.zeros(3), "mx_floor").tolist() == [0, 0, 0]


def test_scale_exponent_stays_in_e8m0_range():
    """E8M0 holds exponents -127..127; tiny blocks clamp at -127 and still
    encode without saturating (bf16 reaches down to 2^-133)."""
    tiny = np.array([2.0 ** -133, 2.0 ** -126, 1e-38, 2.0 ** -119 * 1.5])
    for rule in ("pow2_ceil", "mx_floor"):
        e = f8.scale_exponent(tiny, rule)
        assert np.all(e >= -127) and np.all(e <= 127)
        assert e[0] == -127 and e[1] == -127
        codes, e2, deq = f8.quantize_along_last(tiny.reshape(1, -1).repeat(32, axis=1).reshape(4, 32), 32, rule)
        assert np.all(np.abs(f8.e4m3_decode(codes)) < 448.0)
    huge = np.array([3.0e38])
    assert f8.scale_exponent(huge, "pow2_ceil")[0] == 120  # 448 * 2^120 >= 3e38 > 224 * 2^120


@pytest.mark.parametrize("block,rule", [(128, "pow2_ceil"), (32, "mx_floor")])
def test_quantization_error_bounds(block, rule):
    rng = np.random.default_rng(1)
    v = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-6, 6, size=(64, 1)))
    v[3, :block] = 0.0                                 # an all-zero block
    codes, e, deq = f8.quantize_along_last(v, block, rule)
    sc = np.repeat(np.ldexp(1.0, e), block, axis=-1)
    q = deq / sc
    if rule == "pow2_ceil":
        assert np.all(np.abs(q) <= 448.0)
        bound = np.abs(v) * 2.0 ** -4 + sc * 2.0 ** -10
        assert np.all(np.abs(deq - v) <= bound)
    else:
        unsat = np.abs(v / sc) <= 448.0
        bound = np.abs(v) * 2.0 ** -4 + sc * 2.0 ** -10
        assert np.all(np.abs(deq - v)[unsat] <= bound[unsat])
        assert np.all(np.abs(q[~unsat]) == 448.0)
    assert not deq[3, :block].any()


def test_weight_tiles_share_one_scale():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((2, 256, 384)) * 0.02
    codes, e, deq = f8.quantize_tiles(w, 128, "pow2_ceil")
    assert e.shape == (2, 2, 3)
    blk = np.abs(w[1, 128:256, 256:384]).max()
    assert 448 * 2.0 ** e[1, 1, 2] >= blk > 224 * 2.0 ** e[1, 1, 2]


# ----------------------------------------------------- loop reference, tiny layer

def _q_scalar(v, e):
    """Round v / 2^e to E4M3 (ties to even, saturating) with math.frexp and
    return the dequantized value."""
    a = abs(v) / 2.0 ** e
    s = -1.0 if v < 0 else 1.0
    if a >= 448.0:
        return s * 448.0 * 2.0 ** e
    if a == 0.0:
        return 0.0
    m, ex = math.frexp(a)            # a = m * 2^ex, m in [0.5, 1)
    lsb = 2.0 ** (max(ex - 1, -6) - 3)   # spacing of representable values here
    n = a / lsb
    r = math.floor(n)
    frac = n - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    return s * min(r * lsb, 448.0) * 2.0 ** e


def _bf(v):
    """Round a float to bf16 (8 significant bits, ties to even) with
    math.frexp and Python's round (which rounds halves to even); applied
    element by element to arrays. Magnitudes here stay far from the bf16
    subnormal range."""
    def one(x):
        if x == 0.0:
            return 0.0
        m, ex = math.frexp(x)            # x = m * 2^ex, |m| in [0.5, 1)
        return math.ldexp(round(m * 256.0), ex - 8)
    return np.vectorize(one, otypes=[np.float64])(np.asarray(v, dtype=np.float64))


def _fl32(x):
    """Round a Python float to float32 (the C conversion: nearest, ties to
    even) through struct."""
    return struct.unpack("f", struct.pack("f", x))[0]


def _q_block_f32(vals):
    """The fp32-scale rule, scalar: inv = 448 / amax and the products v * inv
    each rounded once to float32 (a quotient or product of float32 values is
    exact or correctly rounded in double first, so rounding that double to
    float32 is the float32 operation), then the nearest E4M3 value with the
    scalar rounding above; the stored value is code * fl32(amax / 448)."""
    amax = max(abs(v) for v in vals)
    if amax == 0.0 or 448.0 / amax > 3.4028234663852886e38:
        return [0.0 for _ in vals]
    inv = _fl32(448.0 / amax)
    s = _fl32(amax / 448.0)
    return [_q_scalar(_fl32(v * inv), 0) * s for v in vals]


def _q_block(vals, rule):
    if rule == "f32":
        return _q_block_f32(vals)
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        e = 0
    elif rule == "pow2_ceil":
        e = 0
        while 448.0 * 2.0 ** e < amax:
            e += 1
        while 448.0 * 2.0 ** (e - 1) >= amax:
            e -= 1
    else:
        e = math.floor(math.log2(amax)) - 8
        if 2.0 ** (e + 8) > amax:
            e -= 1
        if 2.0 ** (e + 9) <= amax:
            e += 1
    return [_q_scalar(v, e) for v in vals]


def _q_rows(M, block, rule):
    out = []
    for row in M:
        r = []
        for s in range(0, len(row), block):
            r += _q_block(list(row[s:s + block]), rule)
        out.append(r)
    return np.array(out)


def _mode_rule(mode):
    """(activation block, scale rule) of an FP8 mode."""
    if mode == "mxfp8":
        return 32, "mx_floor"
    return 128, ("f32" if mode.endswith("_f32") else "pow2_ceil")


def _q_weight(W, mode, reduce_last):
    if mode == "mxfp8":
        if reduce_last:
            return np.array([_q_rows(W[e], 32, "mx_floor") for e in range(W.shape[0])])
        return np.array([_q_rows(W[e].T, 32, "mx_floor").T for e in range(W.shape[0])])
    out = np.zeros_like(W)
    for e in range(W.shape[0]):
        for r in range(0, W.shape[1], 128):
            for c in range(0, W.shape[2], 128):
                blk = W[e, r:r + 128, c:c + 128]
                out[e, r:r + 128, c:c + 128] = np.array(_q_block(list(blk.reshape(-1)), _mode_rule(mode)[1])).reshape(
                    blk.shape)
    return out


def _layer_loops(x, idx, w, W13, W2, dy, mode):
    """Forward and dx/d_topk_w of the quantized layer, token by token."""
    blk, rule = _mode_rule(mode)
    T, H = x.shape
    I = W13.shape[1] // 2
    k = idx.shape[1]
    qa = lambda M: _q_rows(M, blk, rule)  # noqa: E731
    bf16_fwd = mode in ("fp8_bwd", "fp8_bwd_f32")
    if bf16_fwd:
        xq, W13q, W2q = x, W13, W2
        fwd_q = lambda M: M  # noqa: E731
    else:
        xq, W13q, W2q = qa(x), _q_weight(W13, mode, True), _q_weight(W2, mode, True)
        fwd_q = qa
    W2b = _q_weight(W2, mode, False)
    W13b = _q_weight(W13, mode, False)
    dyq = qa(dy)
    y = np.zeros((T, H))
    dx = np.zeros((T, H))
    dw = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = W13q[e, :I] @ xq[t]
            u = W13q[e, I:] @ xq[t]
            sg = 1.0 / (1.0 + np.exp(-g))
            a = g * sg * u
            # the stored (bf16) activation is what gets quantized
            wa = w[t, j] * a if bf16_fwd else fwd_q(_bf(w[t, j] * a)[None, :])[0]
            y[t] += W2q[e] @ wa
            # the backward reads the saved bf16 g and u
            g, u = _bf(g), _bf(u)
            sg = 1.0 / (1.0 + np.exp(-g))
            a = g * sg * u
            dau = W2b[e].T @ dyq[t]
            dw[t, j] = float(dau @ a)
            da = w[t, j] * dau
            dh = np.concatenate([da * u * sg * (1 + g * (1 - sg)), da * g * sg])
            dx[t] += W13b[e].T @ qa(_bf(dh)[None, :])[0]
    return y, dx, dw


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8", "fp8_bwd", "fp8_block_f32", "fp8_bwd_f32"])
def test_quantized_layer_matches_per_token_loops(mode):
    rng = np.random.default_rng(3)
    T, H, I, E, k = 6, 256, 128, 3, 2
    # bf16-valued inputs, as the layer's are (the fp32-scale rule reads its
    # block maxima as float32 values)
    x = torch_bf16(rng.standard_normal((T, H)))
    W13 = torch_bf16(rng.standard_normal((E, 2 * I, H)) * 0.05)
    W2 = torch_bf16(rng.standard_normal((E, H, I)) * 0.05)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k))
    dy = torch_bf16(rng.standard_normal((T, H)))
    y = f8.forward(x, idx, w, W13, W2, mode)
    dx, dw, _, _ = f8.backward(dy, x, idx, w, W13, W2, mode)
    ry, rdx, rdw = _layer_loops(x, idx, w, W13, W2, dy, mode)
    np.testing.assert_allclose(y, ry, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(dx, rdx, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(dw, rdw, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8"])
def test_quantized_layer_close_to_exact_layer(mode):
    """Sanity scale of the quantization error (a few percent), not a pin."""
    from grouped_gemm_02_amd import inputs
    d = inputs.make_layer_inputs(inputs.CONFIGS["tiny"], "cpu")
    y = f8.forward(d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"], mode)
    ref = orc.forward(d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    err = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert err < 0.15, err


def test_weight_gradients_use_unquantized_operands():
    """With a full-precision forward, dW2 = dY^T (w a) involves no quantized
    operand: it equals the exact gradient up to the bf16 storage of w a
    (relative 2^-9 per element); dW13 inherits the quantized dH product
    through [dg | du] only."""
    from grouped_gemm_02_amd import inputs
    d = inputs.make_layer_inputs(inputs.CONFIGS["tiny"], "cpu")
    args = (d["dy"], d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    _, _, dW13, dW2 = f8.backward(*args, mode="fp8_bwd")
    _, _, rW13, rW2 = orc.backward(*args)
    assert 0 < np.max(np.abs(dW2 - rW2)) / np.max(np.abs(rW2)) < 2.0 ** -8
    assert np.max(np.abs(dW13 - rW13)) / np.max(np.abs(rW13)) < 0.15


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8"])
def test_weight_quantization_is_per_expert(mode):
    """Blocks never straddle experts: quantizing a stack equals stacking the
    per-expert quantizations (what the sampled full-size checks rely on)."""
    rng = np.random.default_rng(5)
    W13 = rng.standard_normal((3, 256, 256)) * np.array([0.01, 1.0, 100.0])[:, None, None]
    W2 = rng.standard_normal((3, 256, 128)) * np.array([5.0, 0.02, 1.0])[:, None, None]
    full = f8.quantize_weights(W13, W2, mode)
    for e in range(3):
        one = f8.quantize_weights(W13[e:e + 1], W2[e:e + 1], mode)
        for key in full:
            assert np.array_equal(full[key][e:e + 1], one[key]), (key, e)


def test_prequantized_weights_give_identical_layer():
    from grouped_gemm_02_amd import inputs
    d = inputs.make_layer_inputs(inputs.CONFIGS["tiny"], "cpu")
    args = (d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    for mode in ("fp8_block", "mxfp8", "fp8_bwd"):
        wq = f8.quantize_weights(d["W13"], d["W2"], mode)
        assert np.array_equal(f8.forward(*args, mode), f8.forward(*args, mode, wq=wq))
        a = f8.backward(d["dy"], *args, mode)
        b = f8.backward(d["dy"], *args, mode, wq=wq)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


# ----------------------------------------------------- FP8 weight gradients

def _wgrad_loops(x, idx, w, W13, W2, dy, mode):
    """dW13, dW2 of the fp8 weight-gradient reading, pair by pair: each
    expert's rows in ascending pair order, every column quantized in blocks
    of 128 (32 for mxfp8) consecutive rows with the scalar helpers above."""
    blk, rule = (32, "mx_floor") if mode == "mxfp8" else (128, "pow2_ceil")
    T, H = x.shape
    E = W13.shape[0]
    I = W13.shape[1] // 2
    k = idx.shape[1]
    qa = lambda M: _q_rows(M, 32 if mode == "mxfp8" else 128, rule)  # noqa: E731
    if mode == "fp8_bwd":
        xq, W13q = x, W13
    else:
        xq, W13q = qa(x), _q_weight(W13, mode, True)
    W2b = _q_weight(W2, mode, False)
    dyq = qa(dy)
    rows = {e: {"dh": [], "x": [], "dy": [], "wa": []} for e in range(E)}
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = W13q[e, :I] @ xq[t]
            u = W13q[e, I:] @ xq[t]
            wa = _bf(w[t, j] * g / (1.0 + np.exp(-g)) * u)   # the saved activation
            g, u = _bf(g), _bf(u)                             # the saved g, u
            sg = 1.0 / (1.0 + np.exp(-g))
            dau = W2b[e].T @ dyq[t]
            da = w[t, j] * dau
            rows[e]["dh"].append(_bf(np.concatenate([da * u * sg * (1 + g * (1 - sg)), da * g * sg])))
            rows[e]["x"].append(x[t])
            rows[e]["dy"].append(dy[t])
            rows[e]["wa"].append(wa)

    def qcols(R):  # quantize each column of R [n, C] in row blocks
        R = np.array(R)
        out = np.zeros_like(R)
        for c in range(R.shape[1]):
            for s in range(0, R.shape[0], blk):
                out[s:s + blk, c] = _q_block(list(R[s:s + blk, c]), rule)
        return out
    dW13 = np.zeros((E, 2 * I, H))
    dW2 = np.zeros((E, H, I))
    for e in range(E):
        if not rows[e]["x"]:
            continue
        dW13[e] = qcols(rows[e]["dh"]).T @ qcols(rows[e]["x"])
        dW2[e] = qcols(rows[e]["dy"]).T @ qcols(rows[e]["wa"])
    return dW13, dW2


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8", "fp8_bwd"])
def test_fp8_weight_gradients_match_pair_loops(mode):
    """Expert segments of ~200 rows: one full and one partial 128-row block
    (blockwise), several 32-row blocks (MX)."""
    rng = np.random.default_rng(8)
    T, H, I, E, k = 300, 256, 128, 3, 2
    x = rng.standard_normal((T, H))
    W13 = rng.standard_normal((E, 2 * I, H)) * 0.05
    W2 = rng.standard_normal((E, H, I)) * 0.05
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k))
    dy = rng.standard_normal((T, H)) * np.exp(rng.standard_normal((T, 1)))  # rows of different scale
    _, _, dW13, dW2 = f8.backward(dy, x, idx, w, W13, W2, mode, wgrad="fp8")
    r13, r2 = _wgrad_loops(x, idx, w, W13, W2, dy, mode)
    np.testing.assert_allclose(dW13, r13, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(dW2, r2, rtol=1e-9, atol=1e-9)
    # sanity scale, not a pin: quantizing along rows of mixed magnitude costs
    # percents (more under the MX rule, which saturates the block maximum)
    _, _, b13, b2 = f8.backward(dy, x, idx, w, W13, W2, mode, wgrad="bf16")
    for q, b in ((dW13, b13), (dW2, b2)):
        err = np.max(np.abs(q - b)) / np.max(np.abs(b))
        assert 0 < err < 0.3, err


def test_token_blocks_restart_and_stand_alone():
    """Row blocks start at the segment's first row: the first 128 rows
    quantize the same whatever follows, and the partial last block on its
    own rows; values exactly representable at their block's scale come back
    unchanged."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal((200, 64))
    v[150, 3] = 1e6                       # only block 1 of column 3 sees it
    q = f8._tok(v, "fp8_block")
    assert np.array_equal(q[:128], f8._tok(v[:128], "fp8_block"))
    assert np.array_equal(q[128:], f8._tok(v[128:], "fp8_block"))
    qm = f8._tok(v, "mxfp8")
    for s in range(0, 200, 32):
        assert np.array_equal(qm[s:s + 32], f8._tok(v[s:s + 32], "mxfp8"))
    exact = rng.choice([-256.0, -3.0, -0.5, 0.0, 0.25, 1.0, 7.0, 448.0], size=(160, 8))
    exact[0] = 448.0                      # block maxima 448: scale 2^0
    exact[128] = 448.0
    assert np.array_equal(f8._tok(exact, "fp8_block"), exact)


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8"])
def test_fp8_weight_gradients_are_per_expert(mode):
    """An expert's weight gradients depend only on its own pairs (what the
    sampled full-size GPU checks rely on): restricting the problem to one
    expert's pairs, in order, gives the same bits."""
    rng = np.random.default_rng(10)
    T, H, I, E, k = 150, 256, 128, 4, 2
    x = rng.standard_normal((T, H))
    W13 = rng.standard_normal((E, 2 * I, H)) * 0.05
    W2 = rng.standard_normal((E, H, I)) * 0.05
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k))
    dy = rng.standard_normal((T, H))
    _, _, dW13, dW2 = f8.backward(dy, x, idx, w, W13, W2, mode, wgrad="fp8")
    for e in range(E):
        f, xe, ie, we, dye = orc.restrict_to_expert(x, idx, w, dy, e)
        _, _, s13, s2 = f8.backward(dye, xe, ie, we, W13[e:e + 1], W2[e:e + 1], mode, wgrad="fp8")
        assert np.array_equal(dW13[e], s13[0]) and np.array_equal(dW2[e], s2[0]), e


# ----------------------------------------------------- default (bf16) weight gradients of the FP8 modes

def _bf16_wgrad_loops(x, idx, w, W13, W2, dy, mode, slip=None):
    """dW13, dW2 under the default reading (weight-gradient GEMMs on the
    unquantized operands) of an FP8 mode, accumulated pair by pair as outer
    products: dW13[e] += [dg | du] x[t]^T and dW2[e] += dY[t] (w a)^T, where
    g, u and w a are the forward's saved bf16 values (quantized x and W13 in
    fp8_block and mxfp8, exact in fp8_bwd) and [dg | du] comes from the
    quantized dH product. `slip` plants a mistake on purpose: "xq" multiplies the
    quantized x in dW13, "exact_a" takes a from the unquantized forward."""
    blk, rule = _mode_rule(mode)
    T, H = x.shape
    E = W13.shape[0]
    I = W13.shape[1] // 2
    k = idx.shape[1]
    qa = lambda M: _q_rows(M, blk, rule)  # noqa: E731
    if mode in ("fp8_bwd", "fp8_bwd_f32"):
        xq, W13q = x, W13
    else:
        xq, W13q = qa(x), _q_weight(W13, mode, True)
    W2b = _q_weight(W2, mode, False)
    dyq = qa(dy)
    dW13 = np.zeros((E, 2 * I, H))
    dW2 = np.zeros((E, H, I))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = W13q[e, :I] @ xq[t]
            u = W13q[e, I:] @ xq[t]
            wa = _bf(w[t, j] * g / (1.0 + np.exp(-g)) * u)   # the saved activation
            if slip == "exact_a":
                ge, ue = W13[e, :I] @ x[t], W13[e, I:] @ x[t]
                wa = _bf(w[t, j] * ge / (1.0 + np.exp(-ge)) * ue)
            g, u = _bf(g), _bf(u)                             # the saved g, u
            sg = 1.0 / (1.0 + np.exp(-g))
            dau = W2b[e].T @ dyq[t]
            da = w[t, j] * dau
            dh = np.concatenate([da * u * sg * (1 + g * (1 - sg)), da * g * sg])
            dW13[e] += np.outer(dh, xq[t] if slip == "xq" else x[t])
            dW2[e] += np.outer(dy[t], wa)
    return dW13, dW2


@pytest.mark.parametrize("mode", ["fp8_block", "mxfp8", "fp8_bwd", "fp8_block_f32", "fp8_bwd_f32"])
def test_default_weight_gradients_match_pair_loops(mode):
    """The default weight-gradient reading of every FP8 mode against outer
    products summed pair by pair, with the scalar rounding helpers above for
    every quantization point of the forward and the dH product. The planted
    slips (the quantized x in dW13; a from the unquantized forward in dW2)
    are far outside the pin's tolerance, so the pin would catch them."""
    rng = np.random.default_rng(11)
    T, H, I, E, k = 7, 256, 128, 3, 2
    x = torch_bf16(rng.standard_normal((T, H)) * np.exp(rng.standard_normal((T, 1))))
    W13 = torch_bf16(rng.standard_normal((E, 2 * I, H)) * 0.05)
    W2 = torch_bf16(rng.standard_normal((E, H, I)) * 0.05)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k))
    dy = torch_bf16(rng.standard_normal((T, H)))
    _, _, dW13, dW2 = f8.backward(dy, x, idx, w, W13, W2, mode)
    r13, r2 = _bf16_wgrad_loops(x, idx, w, W13, W2, dy, mode)
    np.testing.assert_allclose(dW13, r13, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(dW2, r2, rtol=1e-9, atol=1e-9)
    if mode not in ("fp8_bwd", "fp8_bwd_f32"):  # (a bf16 forward is exact: both slips are no-ops there)
        s13, _ = _bf16_wgrad_loops(x, idx, w, W13, W2, dy, mode, slip="xq")
        _, s2 = _bf16_wgrad_loops(x, idx, w, W13, W2, dy, mode, slip="exact_a")
        assert np.max(np.abs(s13 - dW13)) / np.max(np.abs(dW13)) > 1e-4
        assert np.max(np.abs(s2 - dW2)) / np.max(np.abs(dW2)) > 1e-4


def test_bf16_round_matches_library_and_scalar_rounding():
    """The oracle's bf16 rounding against torch's float32 -> bfloat16
    conversion (on float32 values, where that conversion rounds once),
    against the scalar math.frexp rounding above on float64 values, and on
    hand-made ties (halfway values go to the even neighbour)."""
    import torch
    rng = np.random.default_rng(12)
    v32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    lib = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(f8.bf16_round(v32.astype(np.float64)), lib)
    v64 = rng.standard_normal(5000) * np.exp(rng.uniform(-20, 20, 5000))
    assert np.array_equal(f8.bf16_round(v64), _bf(v64))
    one = 1.0 + 2.0 ** -8                      # halfway between 1 and 1 + 2^-7: to 1 (even)
    three = 1.0 + 3 * 2.0 ** -8                # halfway between 1 + 2^-7 and 1 + 2^-6: to 1 + 2^-6
    assert f8.bf16_round(np.array([one, -one, three, np.nextafter(one, 2.0), 0.0])).tolist() == \
        [1.0, -1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, 0.0]
    assert f8.bf16_round(np.array([2.0 ** -133, 2.0 ** -134 * 3, 2.0 ** -135])).tolist() == \
        [2.0 ** -133, 2.0 ** -132, 0.0]         # subnormals: spacing 2^-133, ties to even


# ----------------------------------------------------- fp32-scale blockwise rule

def test_f32_rule_block_maximum_maps_to_448_and_scale_is_amax_over_448():
    """Every block's largest magnitude gets the code of +-448, the stored
    scale is amax / 448 in float32, and so the dequantized maximum is amax
    to within a float32 rounding; blocks of every magnitude, both signs."""
    rng = np.random.default_rng(13)
    v = rng.standard_normal((400, 256)) * np.exp(rng.uniform(-60, 60, size=(400, 1)))
    v = torch_bf16(v)
    codes, s, deq = f8.quantize_along_last_f32(v, 128)
    vb = v.reshape(400, 2, 128)
    cb = codes.reshape(400, 2, 128)
    arg = np.argmax(np.abs(vb), axis=-1)
    top = np.take_along_axis(cb, arg[..., None], axis=-1)[..., 0]
    sign = np.take_along_axis(vb, arg[..., None], axis=-1)[..., 0] < 0
    assert np.array_equal(top, np.where(sign, 0xFE, 0x7E))
    amax = np.max(np.abs(vb), axis=-1)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32))
    dmax = np.max(np.abs(deq.reshape(400, 2, 128)), axis=-1)
    assert np.all(np.abs(dmax - amax) <= amax * 2.0 ** -22)
    # zero and overflowing blocks: scale 1, zero codes
    z = np.zeros((2, 128))
    z[1, 5] = 1e-38                       # 448 / 1e-38 overflows float32
    c, sz, dz = f8.quantize_along_last_f32(z, 128)
    assert not c.any() and not dz.any() and sz.reshape(-1).tolist() == [1.0, 1.0]


def torch_bf16(v):
    import torch
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).float().bfloat16().double().numpy()


def test_f32_rule_matches_scalar_rounding():
    """Rows and 128 x 128 tiles against the scalar rule written with Python
    floats and struct's float32 rounding."""
    rng = np.random.default_rng(14)
    v = torch_bf16(rng.standard_normal((12, 384)) * np.exp(rng.uniform(-8, 8, size=(12, 1))))
    v[3, :128] = 0.0
    v[4, 130] = 448.0 * 3                  # a block whose maximum is an exact multiple of 448
    _, _, deq = f8.quantize_along_last_f32(v, 128)
    assert np.array_equal(deq, _q_rows(v, 128, "f32"))
    w = torch_bf16(rng.standard_normal((1, 256, 128)) * 0.02)
    _, s, dw = f8.quantize_tiles_f32(w, 128)
    assert s.shape == (1, 2, 1)
    assert np.array_equal(dw, _q_weight(w, "fp8_block_f32", True))


def test_f32_rule_error_bound():
    """Within a block the error is at most half an E4M3 step of the value
    (relative 2^-4 for normal codes) plus half the subnormal step times the
    scale, and the rule never saturates a value other than the maximum."""
    rng = np.random.default_rng(15)
    v = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-6, 6, size=(64, 1)))
    codes, s, deq = f8.quantize_along_last_f32(v, 128)
    sc = np.repeat(s.astype(np.float64), 128, axis=-1)
    bound = np.abs(v) * 2.0 ** -4 + sc * 2.0 ** -10 + np.abs(v) * 2.0 ** -22
    assert np.all(np.abs(deq - v) <= bound)
