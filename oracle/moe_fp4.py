"""CPU oracle of the FP8 x FP4 forward: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module; it shares no code with the HIP
path.

The pages list FP8 x FP4 among the data types of DeepGEMM's Mega MoE, a
forward-only fused MoE kernel (MarkTechPost article, comparison table of
fused MoE options: data-type and backward-pass rows), and give no recipe for
it. The reading used here, an inference forward of the
layer:

* expert weights in FP4 E2M1 (OCP MX: sign, 2 exponent bits with bias 1, one
  mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity or NaN),
  in blocks of 32 consecutive values along the GEMM's reduction axis (W13
  along H, W2 along I), each block with a power-of-two scale 2^e,
  e = floor(log2 amax) - 2 (the OCP MX rule: 2 is E2M1's largest exponent),
  so that block values reach just under 8 * 2^e and those above 6 * 2^e
  saturate at 6; an all-zero block gets e = 0, e is clamped to [-127, 127];
* a value v becomes the E2M1 magnitude nearest to |v| / 2^e, ties to the
  even code, with the sign of v (a zero result is +0);
* activations (x along H, w * silu(g) * u along I) in MXFP8 exactly as the
  mxfp8 mode of moe_fp8 (E4M3, 1x32 blocks, MX rule), the activation taken,
  as there, at its stored bf16 value;
* everything after quantization is exact (float64), as in moe_fp8.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_fp8 as f8
from oracle import moe_oracle as base

E2M1_MAX = 6.0
BLOCK = 32

# magnitude of codes 0..7 (code | 8 is the negative value)
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    v = _MAG[c & 7]
    return np.where(c & 8, -v, v)


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code (ties to the even code), saturating at +-6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    hi = np.minimum(np.searchsorted(_MAG, a, side="left"), 7)   # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAG[lo]
    d_hi = _MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _MAG[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = (v < 0) & (code != 0)
    return (code | (neg.astype(np.uint8) << 3)).astype(np.uint8)


def fp4_scale_exponent(amax) -> np.ndarray:
    """e of the block scale 2^e: floor(log2 amax) - 2, 0 for a zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])            # amax = f * 2^ex, f in [0.5, 1)
    out[nz] = (ex - 1) - 2
    return np.clip(out, -127, 127)


def quantize_fp4_along_last(v):
    """Blocks of 32 along the last axis. Returns (codes uint8 0..15, e per
    block, dequantized float64)."""
    v = np.asarray(v, dtype=np.float64)
    *lead, n = v.shape
    assert n % BLOCK == 0
    vb = v.reshape(*lead, n // BLOCK, BLOCK)
    e = fp4_scale_exponent(np.max(np.abs(vb), axis=-1))
    codes = e2m1_encode(vb / np.ldexp(1.0, e)[..., None])
    deq = e2m1_decode(codes) * np.ldexp(1.0, e)[..., None]
    return codes.reshape(v.shape), e, deq.reshape(v.shape)


def quantize_weights(W13, W2) -> dict:
    """Dequantized FP4 weight stacks: W13q along H, W2q along I (the forward
    products' reduction axes; every block lies inside one expert)."""
    return {"W13q": quantize_fp4_along_last(base.as_f64(W13))[2],
            "W2q": quantize_fp4_along_last(base.as_f64(W2))[2]}


def _act(v):
    return f8.quantize_along_last(v, 32, "mx_floor")[2]


def forward(x, topk_idx, topk_w, W13, W2, return_pairs: bool = False, wq: dict | None = None):
    """Forward with MXFP8 activations and FP4 weights. `wq` may carry
    quantize_weights() of these W13, W2."""
    x = base.as_f64(x)
    w = base.as_f64(topk_w)
    idx = base.as_i64(topk_idx)
    T, H = x.shape
    if wq is None:
        wq = quantize_weights(W13, W2)
    W13q, W2q = wq["W13q"], wq["W2q"]
    E, I2, _ = W13q.shape
    I = I2 // 2
    k = idx.shape[1]
    wf = w.reshape(-1)
    xq = _act(x)
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
        O = _act(f8.bf16_round(WA)) @ W2q[e].T   # quantized as stored: in bf16
        np.add.at(y, t, O)
        if return_pairs:
            pairs["g"][f] = G
            pairs["u"][f] = U
            pairs["wa"][f] = WA
    if return_pairs:
        return y, pairs
    return y


__all__ = ["E2M1_MAX", "BLOCK", "e2m1_encode", "e2m1_decode", "fp4_scale_exponent", "quantize_fp4_along_last",
           "quantize_weights", "forward"]
