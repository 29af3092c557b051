"""GPU permutation through moe_permute: bit-exact against the oracle's stable
counting sort, including ids outside [0, E), chunk boundaries and empty
experts."""
import sys

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs
from oracle import moe_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from grouped_gemm_02_amd import binding
    binding.lib()
    return binding


def gpu_permute(B, idx, E):
    T, k = idx.shape
    shape = B.make_shape(T, 256, 128, E, k)
    n = T * k
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    row_of = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    src_of = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    scratch = torch.zeros(B.moe_permute_scratch_bytes(shape), dtype=torch.uint8, device="cuda")
    B.moe_permute(shape, idx, counts, offsets, row_of, src_of, scratch)
    torch.cuda.synchronize()
    return (counts.cpu().numpy(), offsets.cpu().numpy(), row_of.cpu().numpy()[:n], src_of.cpu().numpy(),
            B.moe_read_status(scratch))


CASES = [
    # (T, k, E, routing, seed)
    (1, 1, 1, "uniform", 0),
    (50, 2, 8, "uniform", 1),
    (512, 2, 8, "uniform", 2),       # exactly one chunk of 1024 pairs
    (1025, 1, 3, "uniform", 3),      # one pair past a chunk
    (4097, 1, 3, "uniform", 3),      # one pair past four chunks
    (12800, 4, 300, "uniform", 8),   # 50 chunks over 3 scan segments
    (16384, 8, 128, "uniform", 4),   # 30B shape
    (16384, 8, 128, "zipf", 5),      # empty experts, one hot expert
    (131072, 1, 16, "uniform", 6),   # EP=8 share shape
    (3000, 8, 1024, "uniform", 9),   # the maximum expert count, most experts nearly empty
    (3000, 8, 1024, "zipf", 10),     # the maximum expert count, skewed
    (3000, 4, 1024, "uniform", 7),   # the largest expert count
    (16384, 8, 1024, "zipf", 9),     # 128 chunks, one scan segment
]


@pytest.mark.parametrize("T,k,E,routing,seed", CASES)
def test_permute_bit_exact(B, T, k, E, routing, seed):
    print(f"case permute T={T} k={k} E={E} {routing}", flush=True)
    idx, _ = inputs.make_random_routing_only(T, E, k, seed, "cuda", routing)
    c, o, r, s, st = gpu_permute(B, idx, E)
    rc, ro, rr, rs = orc.permute(idx, E)
    M = int(ro[E])
    assert st == 0
    assert np.array_equal(c, rc)
    assert np.array_equal(o, ro)
    assert np.array_equal(r, rr)
    assert np.array_equal(s[:M], rs)
    assert c.sum() == T * k


def test_permute_invalid_ids(B):
    print("case permute invalid ids", flush=True)
    T, k, E = 5000, 3, 20
    g = torch.Generator().manual_seed(9)
    idx = torch.randint(-3, E + 3, (T, k), generator=g, dtype=torch.int32)
    idx[0, 0] = 2 ** 31 - 1
    idx[1, 1] = -(2 ** 31)
    c, o, r, s, st = gpu_permute(B, idx.cuda(), E)
    rc, ro, rr, rs = orc.permute(idx, E)
    M = int(ro[E])
    assert st == 8
    assert np.array_equal(c, rc) and np.array_equal(o, ro)
    assert np.array_equal(r, rr) and np.array_equal(s[:M], rs)
    assert M < T * k


def test_permute_no_tokens(B):
    shape = B.make_shape(0, 256, 128, 5, 2)
    counts = torch.full((5,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    scratch = torch.zeros(B.moe_permute_scratch_bytes(shape), dtype=torch.uint8, device="cuda")
    B.moe_permute(shape, None, counts, offsets, None, None, scratch)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 5 and offsets.cpu().tolist() == [0] * 6
    sys.stdout.flush()
