"""FP8 emulation for the CPU oracle: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module. It shares no code with the HIP
path.

The pages name the precisions (ic.work analysis, section on hardware
constraints: BF16, MXFP8 and blockwise FP8; MarkTechPost article, "How do
developers use it?": bf16, mxfp8, fp8 and fp8_bwd = BF16 forward with FP8
backward) but not the number format, block shapes, scale rule or which
tensors are quantized. The readings used here:

* FP8 is OCP E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals, no infinities, largest finite value 448.
  Values are rounded to nearest, ties to the even code, and saturate at +-448.
* Every block has one power-of-two scale 2^e (stored as an E8M0 exponent
  byte e + 127); a value v is stored as code(v / 2^e).
  - "fp8_block" (blockwise): activations in 1x128 blocks along the GEMM's
    reduction axis, weights in 128x128 blocks; e is the smallest integer with
    448 * 2^e >= amax (no value saturates).
  - "mxfp8": 1x32 blocks along the reduction axis for every operand, weights
    included; e = floor(log2 amax) - 8 (the OCP MX rule; values up to just
    under 2 * 2^(e+8) saturate at 448).
  - an all-zero block gets e = 0.
* "fp8_block_f32" and "fp8_bwd_f32" (blockwise with fp32 scales): the same
  blocks as "fp8_block" (1x128 activations, 128x128 weights), each with an
  fp32 scale s = amax / 448 rounded to fp32; a value v becomes
  code(v * inv), with inv = 448 / amax rounded to fp32 and the product
  rounded to fp32, so the block maximum lands on +-448 (the product is within
  an fp32 rounding of 448, and the E4M3 grid there is 32 apart). An all-zero
  block, or one so small that 448 / amax overflows fp32 (amax below about
  1.3e-36), gets s = 1 and zero codes. The value stored is code * s.
  "fp8_bwd_f32" runs the bf16 forward and the "fp8_block_f32" backward.
  - e is clamped to [-127, 127], the exponents an E8M0 byte can hold (the
    byte 255 is NaN); only blocks with amax below about 2^-119 reach the
    lower clamp, and there the larger scale leaves every value in range.
* Quantization points: forward x (along H) and the weighted activation
  w * silu(g) * u (along I), gate/up and down weights; backward dY (along H)
  and [dg | du] (along 2I), and the weights again for the transposed use
  (blockwise: the same 128x128 blocks; mxfp8: re-blocked along the new
  reduction axis).
* The two weight-gradient GEMMs (reduction over an expert's rows) have two
  readings, chosen by `wgrad`: "bf16" runs them on the unquantized operands;
  "fp8" quantizes all four operands (x, [dg | du], dY, w * silu(g) * u)
  along the expert's rows, column by column, in blocks of 128 rows
  (blockwise and fp8_bwd, pow2 rule) or 32 rows (mxfp8, MX rule) counted from
  the expert's first row in permuted order (pairs in ascending flat index);
  a last partial block is quantized on its own rows.
* The layer keeps what it passes between its GEMMs in bf16 (round to
  nearest even): g and u and the weighted activation w * silu(g) * u, which
  the forward saves for the backward, and [dg | du], which the dH product
  hands to the dX and dW13 products. A quantized code is an integer decided
  by a floating-point value, so it is taken on that stored bf16 value: the
  activation and [dg | du] are rounded to bf16, then quantized. The
  backward reads the saved bf16 g, u and w * silu(g) * u. Inputs (x, dY and
  the weights) are bf16 already; every other step stays exact.
* Quantization is applied to the (float64) value at each point; the result
  is dequantized (code * 2^e) and the math continues exactly.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as base

E4M3_MAX = 448.0
MODES = ("fp8_block", "mxfp8", "fp8_bwd", "fp8_block_f32", "fp8_bwd_f32")
F32_MODES = ("fp8_block_f32", "fp8_bwd_f32")
BF16_FORWARD_MODES = ("fp8_bwd", "fp8_bwd_f32")


# --------------------------------------------------------------- E4M3 codes

def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for the two NaN codes)."""
    vals = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ex = (c >> 3) & 0xF
        m = c & 0x7
        if ex == 0xF and m == 0x7:
            vals[c] = np.nan
        elif ex == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (ex - 7)
    return vals


_TABLE = e4m3_decode_table()
_POS = _TABLE[:0x7F]                    # codes 0x00..0x7E: 0 .. 448, increasing


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code (ties to the even code), saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS[hi], hi, code).astype(np.uint8)
    neg = (v < 0) & (code != 0)
    return (code | (neg.astype(np.uint8) << 7)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------- bf16 storage

def bf16_round(v) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits, the float32
    exponent range), ties to the even value: v = m * 2^ex with m in [0.5, 1)
    keeps round(m * 2^8) / 2^8, and below the smallest normal (2^-126) the
    spacing stays 2^-133. Used where the layer stores a value in bf16."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)
    ex = np.maximum(ex, -125)            # the subnormal range keeps the spacing of 2^-126's binade
    return np.ldexp(np.rint(np.ldexp(v, 8 - ex)), ex - 8)


# --------------------------------------------------------------- block scales

def scale_exponent(amax, rule: str) -> np.ndarray:
    """Integer e of the block scale 2^e for block maxima `amax` (float64)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    if rule == "pow2_ceil":
        # smallest e with 448 * 2^e >= amax, found exactly (448 * 2^e is exact)
        e = np.ceil(np.log2(amax[nz] / E4M3_MAX)).astype(np.int64)
        e = np.where(np.ldexp(E4M3_MAX, e) < amax[nz], e + 1, e)
        e = np.where(np.ldexp(E4M3_MAX, e - 1) >= amax[nz], e - 1, e)
        out[nz] = e
    elif rule == "mx_floor":
        _, ex = np.frexp(amax[nz])            # amax = f * 2^ex, f in [0.5, 1)
        out[nz] = (ex - 1) - 8                # floor(log2 amax) - emax(E4M3)
    else:
        raise ValueError(rule)
    return np.clip(out, -127, 127)


def quantize_along_last(v, block: int, rule: str):
    """Blocks of `block` consecutive values along the last axis. Returns
    (codes uint8, e int64 per block, dequantized float64)."""
    v = np.asarray(v, dtype=np.float64)
    *lead, n = v.shape
    assert n % block == 0
    vb = v.reshape(*lead, n // block, block)
    e = scale_exponent(np.max(np.abs(vb), axis=-1), rule)
    codes = e4m3_encode(vb / np.ldexp(1.0, e)[..., None])
    deq = e4m3_decode(codes) * np.ldexp(1.0, e)[..., None]
    return codes.reshape(v.shape), e, deq.reshape(v.shape)


def f32_block_scale(amax):
    """(inv, s) of the fp32-scale rule for block maxima `amax`: inv = 448 /
    amax and s = amax / 448, each one float32 division (correctly rounded);
    zero blocks and blocks whose inv overflows get inv = 0 and s = 1."""
    a = np.asarray(amax, dtype=np.float64).astype(np.float32)   # block maxima of bf16 values: exact
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.float32(E4M3_MAX) / a
        s = a / np.float32(E4M3_MAX)
    flat = ~np.isfinite(inv) | (a == 0)
    inv = np.where(flat, np.float32(0.0), inv).astype(np.float32)
    s = np.where(flat, np.float32(1.0), s).astype(np.float32)
    return inv, s


def _f32_codes(vb, inv):
    """E4M3 codes of fl32(v * inv) for float32-exact values vb."""
    y = vb.astype(np.float32) * inv              # one float32 rounding
    return e4m3_encode(y.astype(np.float64))


def quantize_along_last_f32(v, block: int = 128):
    """fp32-scale blocks of `block` along the last axis. Returns (codes,
    float32 scales per block, dequantized float64)."""
    v = np.asarray(v, dtype=np.float64)
    *lead, n = v.shape
    assert n % block == 0
    vb = v.reshape(*lead, n // block, block)
    inv, s = f32_block_scale(np.max(np.abs(vb), axis=-1))
    codes = _f32_codes(vb, inv[..., None])
    deq = e4m3_decode(codes) * s.astype(np.float64)[..., None]
    return codes.reshape(v.shape), s, deq.reshape(v.shape)


def quantize_tiles_f32(w, tile: int = 128):
    """fp32-scale tile x tile blocks over the last two axes. Returns (codes,
    float32 scales per tile, dequantized float64)."""
    w = np.asarray(w, dtype=np.float64)
    *lead, r, c = w.shape
    assert r % tile == 0 and c % tile == 0
    wb = w.reshape(*lead, r // tile, tile, c // tile, tile)
    inv, s = f32_block_scale(np.max(np.abs(wb), axis=(-3, -1)))
    codes = _f32_codes(wb, inv[..., :, None, :, None])
    deq = e4m3_decode(codes) * s.astype(np.float64)[..., :, None, :, None]
    return codes.reshape(w.shape), s, deq.reshape(w.shape)


def quantize_tiles(w, tile: int, rule: str):
    """tile x tile blocks over the last two axes. Returns (codes, e, deq)."""
    w = np.asarray(w, dtype=np.float64)
    *lead, r, c = w.shape
    assert r % tile == 0 and c % tile == 0
    wb = w.reshape(*lead, r // tile, tile, c // tile, tile)
    e = scale_exponent(np.max(np.abs(wb), axis=(-3, -1)), rule)
    sc = np.ldexp(1.0, e)[..., :, None, :, None]
    codes = e4m3_encode(wb / sc)
    deq = e4m3_decode(codes) * sc
    return codes.reshape(w.shape), e, deq.reshape(w.shape)


def _act(v, mode):
    """Quantize-dequantize an activation along its last (reduction) axis."""
    if mode == "mxfp8":
        return quantize_along_last(v, 32, "mx_floor")[2]
    if mode in F32_MODES:
        return quantize_along_last_f32(v, 128)[2]
    return quantize_along_last(v, 128, "pow2_ceil")[2]


def _tok(v, mode):
    """Quantize-dequantize one expert's operand [n, C] along its rows (the
    weight-gradient GEMM's reduction axis): each column in blocks of 128
    (32 for mxfp8) consecutive rows from row 0; zero rows pad the last block,
    which leaves its maximum and its other values unchanged."""
    if mode in F32_MODES:
        raise ValueError("the fp32-scale modes have no FP8 weight-gradient reading")
    block, rule = (32, "mx_floor") if mode == "mxfp8" else (128, "pow2_ceil")
    v = np.asarray(v, dtype=np.float64)
    n, c = v.shape
    vp = np.zeros((-(-n // block) * block, c))
    vp[:n] = v
    return quantize_along_last(vp.T, block, rule)[2].T[:n]


def _weight(w, mode, reduce_axis_last: bool):
    """Quantize-dequantize a weight matrix stack [E, R, C]; the GEMM reduces
    over its last axis (reduce_axis_last) or over the middle axis."""
    if mode == "mxfp8":
        if reduce_axis_last:
            return quantize_along_last(w, 32, "mx_floor")[2]
        return np.swapaxes(quantize_along_last(np.swapaxes(w, -1, -2), 32, "mx_floor")[2], -1, -2)
    if mode in F32_MODES:
        return quantize_tiles_f32(w, 128)[2]
    return quantize_tiles(w, 128, "pow2_ceil")[2]


# --------------------------------------------------------------- layer

_WEIGHT_USES = {
    "W13q": ("W13", True),    # forward gate/up product reduces over H (W13's columns)
    "W2q": ("W2", True),      # forward down product reduces over I (W2's columns)
    "W2b": ("W2", False),     # dH product reduces over H = W2's rows
    "W13b": ("W13", False),   # dX product reduces over 2I = W13's rows
}


def quantize_weights(W13, W2, mode: str, keys=("W13q", "W2q", "W2b", "W13b")) -> dict:
    """Dequantized weight stacks for the uses in `keys`. Every block lies
    inside one expert, so the result for a stack equals the stack of the
    per-expert results."""
    src = {"W13": base.as_f64(W13), "W2": base.as_f64(W2)}
    return {k: _weight(src[_WEIGHT_USES[k][0]], mode, _WEIGHT_USES[k][1]) for k in keys}


def _need(wq, W13, W2, mode, keys):
    wq = dict(wq or {})
    missing = [k for k in keys if k not in wq]
    if missing:
        wq.update(quantize_weights(W13, W2, mode, missing))
    return wq


def forward(x, topk_idx, topk_w, W13, W2, mode: str, return_pairs: bool = False, wq: dict | None = None):
    """Forward with the quantization points of `mode` ("fp8_bwd" runs the
    forward in full precision). `wq` may carry quantize_weights() results
    for these W13, W2."""
    if mode in BF16_FORWARD_MODES:
        return base.forward(x, topk_idx, topk_w, W13, W2, return_pairs=return_pairs)
    x = base.as_f64(x)
    w = base.as_f64(topk_w)
    idx = base.as_i64(topk_idx)
    T, H = x.shape
    wq = _need(wq, W13, W2, mode, ("W13q", "W2q"))
    W13q, W2q = wq["W13q"], wq["W2q"]
    E, I2, _ = W13q.shape
    I = I2 // 2
    k = idx.shape[1]
    wf = w.reshape(-1)
    xq = _act(x, mode)
    y = np.zeros((T, H))
    pairs = {"g": np.zeros((T * k, I)), "u": np.zeros((T * k, I)), "wa": np.zeros((T * k, I))} \
        if return_pairs else None
    for e in range(E):
        f = base.expert_pairs(idx, e)
        if f.size == 0:
            continue
        t = f // k
        X = xq[t]
        G = X @ W13q[e, :I].T
        U = X @ W13q[e, I:].T
        WA = wf[f][:, None] * (base.silu(G) * U)
        O = _act(bf16_round(WA), mode) @ W2q[e].T
        np.add.at(y, t, O)
        if return_pairs:
            pairs["g"][f] = G
            pairs["u"][f] = U
            pairs["wa"][f] = WA
    if return_pairs:
        return y, pairs
    return y


def backward(dy, x, topk_idx, topk_w, W13, W2, mode: str, wq: dict | None = None, wgrad: str = "bf16"):
    """Gradients of L = <dY, y> with the backward quantization points of
    `mode`: dY and W2 quantized for the dH product, [dg | du] and W13 for the
    dX product; the weight gradients use unquantized operands (wgrad="bf16")
    or operands quantized along the expert's rows (wgrad="fp8"). g and u come
    from the forward of the same mode."""
    if wgrad not in ("bf16", "fp8"):
        raise ValueError(wgrad)
    dy = base.as_f64(dy)
    x = base.as_f64(x)
    W13 = base.as_f64(W13)
    W2 = base.as_f64(W2)
    w = base.as_f64(topk_w)
    idx = base.as_i64(topk_idx)
    T, H = x.shape
    E, I2, _ = W13.shape
    I = I2 // 2
    k = idx.shape[1]
    wf = w.reshape(-1)
    if mode in BF16_FORWARD_MODES:
        wq = _need(wq, W13, W2, mode, ("W2b", "W13b"))
        xf, W13f = x, W13
    else:
        wq = _need(wq, W13, W2, mode, ("W13q", "W2b", "W13b"))
        xf, W13f = _act(x, mode), wq["W13q"]
    dyq = _act(dy, mode)
    W2b, W13b = wq["W2b"], wq["W13b"]
    dx = np.zeros((T, H))
    dwf = np.zeros(T * k)
    dW13 = np.zeros((E, I2, H))
    dW2 = np.zeros((E, H, I))
    for e in range(E):
        f = base.expert_pairs(idx, e)
        if f.size == 0:
            continue
        t = f // k
        # what the forward saved, in bf16: g, u and w * silu(g) * u
        G0 = xf[t] @ W13f[e, :I].T
        U0 = xf[t] @ W13f[e, I:].T
        WA = bf16_round(wf[f][:, None] * (base.silu(G0) * U0))
        G, U = bf16_round(G0), bf16_round(U0)
        S = base.sigmoid(G)
        A = G * S * U
        dAu = dyq[t] @ W2b[e]
        dwf[f] = np.sum(dAu * A, axis=1)
        dA = wf[f][:, None] * dAu
        dG = dA * U * S * (1.0 + G * (1.0 - S))
        dU = dA * G * S
        dHm = np.concatenate([dG, dU], axis=1)
        dHs = bf16_round(dHm)                 # [dg | du] as handed to the next products
        np.add.at(dx, t, _act(dHs, mode) @ W13b[e])
        if wgrad == "fp8":
            dW13[e] = _tok(dHs, mode).T @ _tok(x[t], mode)
            dW2[e] = _tok(dy[t], mode).T @ _tok(WA, mode)
        else:
            dW13[e] = dHm.T @ x[t]
            dW2[e] = dy[t].T @ WA
    return dx, dwf.reshape(T, k), dW13, dW2


__all__ = ["MODES", "F32_MODES", "BF16_FORWARD_MODES", "E4M3_MAX", "bf16_round", "f32_block_scale",
           "quantize_along_last_f32", "quantize_tiles_f32", "e4m3_decode_table", "e4m3_encode", "e4m3_decode", "scale_exponent",
           "quantize_along_last", "quantize_tiles", "quantize_weights", "forward", "backward"]
