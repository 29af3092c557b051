"""Pins of the FP8 x FP4 forward oracle (oracle/moe_fp4.py) against what the
E2M1 format and the MX scale rule fix: the code table from its bit fields,
ties to the even code at every midpoint, saturation, the defining inequality
of the block exponent, exactness on representable values, and a token-by-token
loop of the quantized forward with its own scalar rounding."""
import math

import numpy as np
import pytest

from oracle import moe_fp4 as f4

pytestmark = pytest.mark.filterwarnings("ignore")


def _bits_value(c):
    """E2M1 value of code c from its fields: sign, 2 exponent bits (bias 1),
    1 mantissa bit; exponent 0 is subnormal (0 or 0.5)."""
    s = -1.0 if c & 8 else 1.0
    ex, m = (c >> 1) & 3, c & 1
    return s * (m * 0.5 if ex == 0 else (1.0 + 0.5 * m) * 2.0 ** (ex - 1))


def test_code_table_from_bit_fields():
    for c in range(16):
        assert f4.e2m1_decode(np.uint8(c)) == _bits_value(c), c
    assert f4.E2M1_MAX == max(_bits_value(c) for c in range(16))


def test_round_trip_and_ties_to_even():
    mags = [_bits_value(c) for c in range(8)]
    for c in range(16):
        v = _bits_value(c)
        got = int(f4.e2m1_encode(v))
        assert f4.e2m1_decode(np.uint8(got)) == v and (got == c or v == 0.0), (c, got)
    for c in range(7):
        lo, hi = mags[c], mags[c + 1]
        mid = 0.5 * (lo + hi)
        even = c if c % 2 == 0 else c + 1
        assert int(f4.e2m1_encode(mid)) == even, (lo, hi)
        assert int(f4.e2m1_encode(-mid)) == (even | 8 if even else 0)
        eps = (hi - lo) * 1e-6
        assert int(f4.e2m1_encode(mid - eps)) == c
        assert int(f4.e2m1_encode(mid + eps)) == c + 1


def test_saturation_and_signed_zero():
    for v in (6.0, 6.5, 7.99, 1e6):
        assert int(f4.e2m1_encode(v)) == 7 and int(f4.e2m1_encode(-v)) == 15
    assert int(f4.e2m1_encode(-0.0)) == 0
    assert int(f4.e2m1_encode(-0.2)) == 0    # rounds to zero: stored as +0


def test_scale_exponent_rule():
    rng = np.random.default_rng(0)
    amax = np.concatenate([np.exp(rng.uniform(-60, 60, 20000)), 2.0 ** np.arange(-40, 40),
                           np.nextafter(2.0 ** np.arange(-40, 40), 0)])
    e = f4.fp4_scale_exponent(amax)
    r = amax / np.ldexp(1.0, e)
    assert np.all(r >= 4.0) and np.all(r < 8.0)
    assert f4.fp4_scale_exponent(np.array([0.0]))[0] == 0


def test_representable_blocks_are_exact():
    """Blocks whose values are E2M1 values times 2^e, with a block maximum of
    6 * 2^e or 4 * 2^e, come back unchanged."""
    rng = np.random.default_rng(1)
    mags = np.array([_bits_value(c) for c in range(16)])
    v = rng.choice(mags, size=(5, 8, 64))
    v[..., 0] = 6.0
    v[..., 32] = -4.0
    v = v * np.ldexp(1.0, rng.integers(-20, 20, size=(5, 8, 1)))
    _, _, deq = f4.quantize_fp4_along_last(v)
    np.testing.assert_array_equal(deq, v)


def test_quantization_error_bound():
    """|q(v) - v| is at most half the spacing at |v| (0.25 * 2^e below 2 * 2^e,
    0.5 * 2^e up to 4 * 2^e, 1 * 2^e up to 6 * 2^e) or the saturation gap."""
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-5, 5, (64, 1)))
    _, e, deq = f4.quantize_fp4_along_last(v)
    sc = np.repeat(np.ldexp(1.0, e), 32, axis=-1)
    a = np.abs(v) / sc
    half_gap = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = np.where(a > 6, a - 6, half_gap) * sc
    assert np.all(np.abs(deq - v) <= bound * (1 + 1e-12))


# ----------------------------------------------------- loop reference, tiny layer

def _fp4_scalar(v, e):
    """Nearest E2M1 magnitude of |v| / 2^e by search over the 8 magnitudes
    (ties to the even code), saturating at 6; dequantized."""
    a = min(abs(v) / 2.0 ** e, 6.0)
    mags = [_bits_value(c) for c in range(8)]
    best = min(range(8), key=lambda c: (abs(a - mags[c]), c % 2))
    return math.copysign(mags[best], v) * 2.0 ** e if mags[best] else 0.0


def _fp4_block(vals):
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        return [0.0 for _ in vals]
    m, ex = math.frexp(amax)       # amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
    e = (ex - 1) - 2
    return [_fp4_scalar(v, e) for v in vals]


def _e4m3_scalar(v, e):
    a = abs(v) / 2.0 ** e
    if a == 0.0:
        return 0.0
    if a >= 448.0:
        return math.copysign(448.0 * 2.0 ** e, v)
    m, ex = math.frexp(a)
    lsb = 2.0 ** (max(ex - 1, -6) - 3)
    n = a / lsb
    r = math.floor(n)
    frac = n - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    return math.copysign(min(r * lsb, 448.0), v) * 2.0 ** e


def _mx8_block(vals):
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        return [0.0 for _ in vals]
    m, ex = math.frexp(amax)
    e = (ex - 1) - 8
    return [_e4m3_scalar(v, e) for v in vals]


def _bf(v):
    """bf16 rounding of each element (8 significant bits, halves to even via
    Python's round), written with math.frexp."""
    def one(x):
        if x == 0.0:
            return 0.0
        m, ex = math.frexp(x)
        return math.ldexp(round(m * 256.0), ex - 8)
    return np.vectorize(one, otypes=[np.float64])(np.asarray(v, dtype=np.float64))


def _rows(M, fn):
    return np.array([[q for s in range(0, len(row), 32) for q in fn(list(row[s:s + 32]))] for row in M])


def test_forward_matches_per_token_loops():
    rng = np.random.default_rng(3)
    T, H, I, E, k = 5, 128, 64, 3, 2
    x = rng.standard_normal((T, H))
    W13 = rng.standard_normal((E, 2 * I, H)) * 0.05
    W2 = rng.standard_normal((E, H, I)) * 0.05
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, size=(T, k))
    y = f4.forward(x, idx, w, W13, W2)
    W13q = np.array([_rows(W13[e], _fp4_block) for e in range(E)])
    W2q = np.array([_rows(W2[e], _fp4_block) for e in range(E)])
    xq = _rows(x, _mx8_block)
    ry = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = W13q[e, :I] @ xq[t]
            u = W13q[e, I:] @ xq[t]
            a = g / (1.0 + np.exp(-g)) * u
            # the activation is quantized at its stored bf16 value
            ry[t] += W2q[e] @ _rows(_bf(w[t, j] * a)[None, :], _mx8_block)[0]
    np.testing.assert_allclose(y, ry, rtol=1e-9, atol=1e-9)


def test_forward_close_to_exact_layer():
    """Sanity scale of the quantization error (FP4 weights: ~10 %), not a pin."""
    from grouped_gemm_02_amd import inputs
    from oracle import moe_oracle as base
    cfg = inputs.CONFIGS["tiny"]
    d = inputs.make_layer_inputs(cfg, "cpu")
    ref = base.forward(d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    y = f4.forward(d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    assert np.abs(y - ref).max() / np.abs(ref).max() < 0.3
