"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Indices (counts, offsets, row_of, src_of) must match bit-exactly; floating
outputs and gradients must be within the bf16 max-relative-error bound
(normwise by the reference maximum). Small layers are compared element by
element, and so is the Qwen3-30B-A3B-shaped layer (uniform and Zipf
routing), whose every token row and every expert is also held to the bound
on its own.
"""
import os
import sys

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs
from oracle import moe_oracle as orc
from tests.helpers import TOL_BF16, max_rel_err

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


def run_layer(B, cfg, d, num_cus=0):
    """Forward + backward through the C ABI. Returns host tensors."""
    shape = B.make_shape(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, "bf16", num_cus)
    buf = B.LayerBuffers.allocate(shape)
    buf.fwd_ws.fill_(0xFF)   # poison scratch: reads of unwritten memory show up
    buf.bwd_ws.fill_(0xFF)
    buf.saved.fill_(0xFF)
    y = B.forward(buf, d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    dx, dw, dW13, dW2 = B.backward(buf, d["dy"], d["x"], d["topk_idx"], d["topk_w"], d["W13"], d["W2"])
    torch.cuda.synchronize()
    Tk = cfg.T * cfg.k
    out = {
        "y": y, "dx": dx, "dw": dw, "dW13": dW13, "dW2": dW2,
        "counts": buf.saved_view("counts", torch.int32, cfg.E).clone(),
        "offsets": buf.saved_view("offsets", torch.int32, cfg.E + 1).clone(),
        "row_of": buf.saved_view("row_of", torch.int32, Tk).clone(),
        "src_of": buf.saved_view("src_of", torch.int32, Tk).clone(),
        "h13": buf.saved_view("h13", torch.bfloat16, Tk * 2 * cfg.I).view(Tk, 2 * cfg.I).clone(),
        "act": buf.saved_view("act", torch.bfloat16, Tk * cfg.I).view(Tk, cfg.I).clone(),
        "status": B.moe_read_status(buf.fwd_ws),
    }
    return out


def check_permutation(out, idx, E):
    counts, offsets, row_of, src_of = orc.permute(idx, E)
    M = int(offsets[E])
    assert np.array_equal(out["counts"].cpu().numpy(), counts)
    assert np.array_equal(out["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(out["row_of"].cpu().numpy(), row_of)
    assert np.array_equal(out["src_of"].cpu().numpy()[:M], src_of)


def check_full(out, cfg, d, tol=TOL_BF16):
    """Element-by-element comparison of every output against the oracle."""
    idx = d["topk_idx"]
    check_permutation(out, idx, cfg.E)
    y_ref, pairs = orc.forward(d["x"], idx, d["topk_w"], d["W13"], d["W2"], return_pairs=True)
    dx_ref, dw_ref, dW13_ref, dW2_ref = orc.backward(d["dy"], d["x"], idx, d["topk_w"], d["W13"], d["W2"])
    errs = {
        "y": max_rel_err(orc.as_f64(out["y"]), y_ref),
        "dx": max_rel_err(orc.as_f64(out["dx"]), dx_ref),
        "d_topk_w": max_rel_err(orc.as_f64(out["dw"]), dw_ref),
        "dW13": max_rel_err(orc.as_f64(out["dW13"]), dW13_ref),
        "dW2": max_rel_err(orc.as_f64(out["dW2"]), dW2_ref),
    }
    # saved intermediates, per permuted row
    _, _, row_of, src_of = orc.permute(idx, cfg.E)
    M = src_of.size
    I = cfg.I
    h13 = orc.as_f64(out["h13"])[:M]
    errs["g"] = max_rel_err(h13[:, :I], pairs["g"][src_of])
    errs["u"] = max_rel_err(h13[:, I:], pairs["u"][src_of])
    # the saved activation carries the routing weight: w * silu(g) * u
    wf = orc.as_f64(d["topk_w"]).reshape(-1)
    errs["wa"] = max_rel_err(orc.as_f64(out["act"])[:M], pairs["a"][src_of] * wf[src_of][:, None])
    _say(f"{cfg.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)
    # empty experts: exactly zero weight gradients
    counts = orc.permute(idx, cfg.E)[0]
    for e in np.nonzero(counts == 0)[0]:
        assert not out["dW13"][e].any() and not out["dW2"][e].any()
    assert np.all(np.isfinite(orc.as_f64(out["dx"])))
    return {"y": y_ref, "dx": dx_ref, "dW13": dW13_ref, "dW2": dW2_ref}


SMALL = [
    inputs.CONFIGS["tiny"],
    # several m-tiles per expert with a ragged tail, several n-tiles, K loop > 1
    inputs.LayerConfig("mid", 600, 512, 384, 7, 3, "uniform", "bf16", 10),
    # skewed: empty experts and one hot expert; ragged everything
    inputs.LayerConfig("skew", 333, 256, 128, 16, 4, "zipf", "bf16", 11, zipf_s=1.2, zipf_cold=5),
    # one expert, top-1: a dense GEMM pair through the grouped path
    inputs.LayerConfig("one_expert", 300, 256, 256, 1, 1, "uniform", "bf16", 12),
    # top-1 routing over many experts with short segments
    inputs.LayerConfig("top1", 257, 768, 128, 40, 1, "uniform", "bf16", 13),
    # a single token
    inputs.LayerConfig("one_token", 1, 256, 128, 8, 8, "uniform", "bf16", 14),
    # the maximum expert count: ~5 rows per expert, many experts empty
    inputs.LayerConfig("max_experts", 600, 256, 128, 1024, 8, "uniform", "bf16", 15),
    # the maximum expert count under skew (the weight gradients' queue schedule)
    inputs.LayerConfig("max_experts_zipf", 700, 256, 384, 1024, 8, "zipf", "bf16", 16, zipf_s=1.1, zipf_cold=100),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_layer_matches_oracle_elementwise(B, cfg):
    _say(f"case {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    out = run_layer(B, cfg, d)
    assert out["status"] == 0
    check_full(out, cfg, d)


# Skewed routing with experts hot enough that their weight-gradient tiles are
# cut along the expert's rows (at least 1024 rows and over 3/4 of one
# workgroup's nominal share, under a max * E > 2 * total skew): the hottest
# expert (2813 rows) into 4 row ranges of 768, the next (1179 rows) into 4 of
# 384, both with a ragged last range.
HOT = inputs.LayerConfig("hot", 8192, 512, 384, 32, 1, "zipf", "bf16", 21, zipf_s=1.2, zipf_cold=8)


def _assert_split_routing(d, cfg):
    c = np.bincount(d["topk_idx"].cpu().numpy().ravel(), minlength=cfg.E)
    assert int(c.max()) * cfg.E > 2 * int(c.sum()) and np.sort(c)[-2] >= 1024, np.sort(c)[-4:]


def test_split_weight_gradients_match_oracle_elementwise(B):
    cfg = HOT
    _say(f"case split dW {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    _assert_split_routing(d, cfg)
    out = run_layer(B, cfg, d)
    assert out["status"] == 0
    check_full(out, cfg, d)


def test_split_weight_gradients_deterministic_bitwise(B):
    cfg = HOT
    _say(f"case split dW determinism {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    a = run_layer(B, cfg, d)
    b = run_layer(B, cfg, d, num_cus=37)
    for k in ("dW13", "dW2"):
        assert torch.equal(a[k], b[k]), k


# Balanced routing whose weight-gradient tiles leave the last round of the
# nominal 256 workgroups partly empty: dW2 has 10 * 8 * 4 = 320 tiles (one
# round and a quarter), dW13 640 (two and a half); the tiles of the two
# heaviest experts (about 2000 rows each) are cut into two row ranges of 1024
# and the rest, and the whole tiles run first.
TAIL = inputs.LayerConfig("tail", 10000, 2048, 1024, 10, 2, "uniform", "bf16", 23)


def _assert_tail_routing(d, cfg):
    c = np.bincount(d["topk_idx"].cpu().numpy().ravel(), minlength=cfg.E)
    assert int(c.max()) * cfg.E <= 2 * int(c.sum()), "balanced (no skew split)"
    assert np.sort(c)[-2] > 1024, np.sort(c)[-4:]
    for per_expert in ((cfg.H // 256) * ((cfg.I + 255) // 256), (2 * cfg.I // 256) * (cfg.H // 256)):
        n = cfg.E * per_expert
        assert 1 <= n // 256 <= 3 and 0 < 2 * (n % 256) <= 256, n


def test_tail_split_weight_gradients_elementwise(B):
    d = inputs.make_layer_inputs(TAIL, "cpu")
    _assert_tail_routing(d, TAIL)
    del d
    _full_size_check(B, TAIL)


def test_tail_split_weight_gradients_deterministic_bitwise(B):
    cfg = TAIL
    _say(f"case tail-split dW determinism {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    a = run_layer(B, cfg, d)
    for cus in (37, 3):  # 3 workgroups: most XCD shares are taken over by other workgroups
        b = run_layer(B, cfg, d, num_cus=cus)
        for k in ("dW13", "dW2"):
            assert torch.equal(a[k], b[k]), (k, cus)


def test_layer_deterministic_bitwise(B):
    cfg = SMALL[1]
    _say(f"case determinism {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    a = run_layer(B, cfg, d)
    b = run_layer(B, cfg, d)
    for k in ("y", "dx", "dw", "dW13", "dW2", "h13", "act"):
        assert torch.equal(a[k], b[k]), k


def test_invalid_expert_ids_are_dropped_and_reported(B):
    cfg = inputs.LayerConfig("invalid_ids", 200, 256, 128, 8, 2, "uniform", "bf16", 15)
    _say(f"case {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    idx = d["topk_idx"].clone()
    idx[3, 1] = 8
    idx[17, 0] = -1
    idx[199, 1] = 1 << 20
    d["topk_idx"] = idx
    out = run_layer(B, cfg, d)
    assert out["status"] == 8  # MOE_ERR_ROUTING
    check_full(out, cfg, d)
    dw = out["dw"].cpu()
    assert dw[3, 1] == 0 and dw[17, 0] == 0 and dw[199, 1] == 0


def test_invalid_expert_ids_top1(B):
    """Top-1 rows are written straight to their tokens; dropped tokens must
    still come out as zero rows of y and dx."""
    cfg = inputs.LayerConfig("invalid_ids_top1", 300, 256, 128, 6, 1, "uniform", "bf16", 17)
    _say(f"case {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    idx = d["topk_idx"].clone()
    idx[0, 0] = 6
    idx[150, 0] = -3
    idx[299, 0] = 1 << 30
    d["topk_idx"] = idx
    out = run_layer(B, cfg, d)
    assert out["status"] == 8
    check_full(out, cfg, d)
    for t in (0, 150, 299):
        assert not out["y"][t].any() and not out["dx"][t].any() and out["dw"][t, 0] == 0


def test_zero_tokens_gives_zero_weight_grads(B):
    cfg = inputs.LayerConfig("empty", 0, 256, 128, 4, 2, "uniform", "bf16", 16)
    d = inputs.make_layer_inputs(cfg, DEV)
    out = run_layer(B, cfg, d)
    assert out["counts"].sum().item() == 0
    assert not out["dW13"].any() and not out["dW2"].any()


def test_num_cus_cap_gives_identical_results(B):
    cfg = SMALL[1]
    d = inputs.make_layer_inputs(cfg, DEV)
    a = run_layer(B, cfg, d)
    b = run_layer(B, cfg, d, num_cus=13)
    for k in ("y", "dx", "dw", "dW13", "dW2"):
        assert torch.equal(a[k], b[k]), k


# --------------------------------------------------------------- full size

def _row_errs(got, ref):
    """Per-row max-relative error (max |diff| over the row / max |ref| over
    the row); rows whose reference is all zero must come out all zero."""
    got = orc.as_f64(got)
    diff = np.max(np.abs(got - ref), axis=1)
    scale = np.max(np.abs(ref), axis=1)
    z = scale == 0
    assert not np.any(diff[z]), "rows with an all-zero reference must be zero"
    return diff[~z] / scale[~z]


def _full_size_check(B, cfg):
    """The page-sized layer compared element by element with the full oracle
    (every token, every pair, every expert): the stated per-tensor bound, and
    the same bound per token row of y and dx and per expert of dW13 and dW2,
    so that an error confined to some tiles (the XCD remap, the n-tile-major
    walk, the split plan under skew) cannot hide behind the largest values."""
    import time
    t0 = time.time()
    _say(f"case full-size elementwise {inputs.describe(cfg)}")
    d = inputs.make_layer_inputs(cfg, DEV)
    out = run_layer(B, cfg, d)
    assert out["status"] == 0
    _say(f"  gpu done {time.time() - t0:.1f}s")
    ref = check_full(out, cfg, d)
    _say(f"  oracle + per-tensor check done {time.time() - t0:.1f}s")
    y_ref, dx_ref, dW13_ref, dW2_ref = ref["y"], ref["dx"], ref["dW13"], ref["dW2"]
    del ref
    worst = {"y_row": float(np.max(_row_errs(out["y"], y_ref))),
             "dx_row": float(np.max(_row_errs(out["dx"], dx_ref)))}
    del y_ref, dx_ref
    counts = out["counts"].cpu().numpy()
    e13, e2 = [], []
    for e in range(cfg.E):
        if counts[e] == 0:
            continue
        e13.append(max_rel_err(orc.as_f64(out["dW13"][e]), dW13_ref[e]))
        e2.append(max_rel_err(orc.as_f64(out["dW2"][e]), dW2_ref[e]))
    worst["dW13_expert"] = max(e13)
    worst["dW2_expert"] = max(e2)
    _say(f"{cfg.name}: worst " + " ".join(f"{k}={v:.2e}" for k, v in worst.items())
         + f" over {cfg.T} tokens, {len(e13)} non-empty experts ({time.time() - t0:.1f}s)")
    for k, v in worst.items():
        assert v <= TOL_BF16, (k, v)


def test_qwen3_30b_shape_elementwise(B):
    _full_size_check(B, inputs.CONFIGS["qwen3_30b"])


def test_qwen3_30b_shape_zipf_routing_bf16_elementwise(B):
    cfg = inputs.CONFIGS["zipf"].scaled(name="zipf_bf16", precision="bf16")
    _full_size_check(B, cfg)


def test_ep8_share_bf16_elementwise(B):
    """One EP=8 rank's share in bf16 (131,072 rows, 16 experts, top-1): the
    down and dX GEMMs write rows straight to their tokens, and dW2's 384
    tiles take the last-round split."""
    cfg = inputs.CONFIGS["ep8_share"].scaled(name="ep8_share_bf16", precision="bf16")
    _full_size_check(B, cfg)


# --------------------------------------------------------------- duplicate experts

def _with_duplicates(d, every=3):
    """Every `every`-th token sends two of its slots to the same expert
    (slot 1 repeats slot 0): two rows of that expert, summed in y."""
    idx = d["topk_idx"].clone()
    idx[::every, 1] = idx[::every, 0]
    d["topk_idx"] = idx
    return d


DUPS = [inputs.LayerConfig("dup", 500, 512, 384, 6, 3, "uniform", "bf16", 31),
        inputs.LayerConfig("dup_top2", 300, 256, 128, 4, 2, "uniform", "bf16", 32)]


@pytest.mark.parametrize("cfg", DUPS, ids=[c.name for c in DUPS])
def test_duplicate_expert_in_one_token_elementwise(B, cfg):
    """A token may name one expert twice (the reading: two rows, summed):
    the permutation keeps both pairs in flat order and every output matches
    the oracle element by element."""
    _say(f"case duplicate experts {inputs.describe(cfg)}")
    d = _with_duplicates(inputs.make_layer_inputs(cfg, DEV))
    idx = d["topk_idx"].cpu().numpy()
    assert np.any(idx[:, 0] == idx[:, 1])
    out = run_layer(B, cfg, d)
    assert out["status"] == 0
    check_full(out, cfg, d)
