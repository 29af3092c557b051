"""The allocation-free permutation entry point (moe_permute_noalloc, whose
chunk table is a fixed device array of the library) against moe_permute
(scratch from the caller), bit for bit, on two calls in a row, the second
with a smaller input that also carries invalid expert ids."""
import sys

import numpy as np
import pytest
import torch

from grouped_gemm_02_amd import inputs

pytestmark = pytest.mark.gpu


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


def _outs(E, n, fill):
    mk = lambda m: torch.full((max(m, 1),), fill, dtype=torch.int32, device="cuda")  # noqa: E731
    return mk(E), mk(E + 1), mk(n), mk(n), mk(1)


def _both(B, idx, E):
    T, k = idx.shape
    shape = B.make_shape(T, 256, 128, E, k)
    n = T * k
    ref = _outs(E, n, -7)
    scratch = torch.zeros(B.moe_permute_scratch_bytes(shape), dtype=torch.uint8, device="cuda")
    B.moe_permute(shape, idx, *ref[:4], scratch)
    got = _outs(E, n, -9)
    B.moe_permute_noalloc(shape, idx, *got)
    torch.cuda.synchronize()
    ref_status = B.moe_read_status(scratch)
    M = int(ref[1][E].item())
    for name, a, b in (("counts", ref[0], got[0]), ("offsets", ref[1], got[1]), ("row_of", ref[2][:n], got[2][:n]),
                       ("src_of", ref[3][:M], got[3][:M])):
        assert torch.equal(a, b), name
    assert int(got[4].item()) == ref_status
    return ref_status, M


def test_noalloc_permute_matches_permute_twice(B):
    E, k = 128, 8
    _say("case noalloc permute: T=16384 k=8 E=128 uniform, then T=999 k=8 E=128 zipf with invalid ids")
    idx1, _ = inputs.make_random_routing_only(16384, E, k, 41, "cuda", "uniform")
    st, M = _both(B, idx1, E)
    assert st == 0 and M == 16384 * k
    idx2, _ = inputs.make_random_routing_only(999, E, k, 42, "cuda", "zipf")
    idx2 = idx2.clone()
    idx2[5, 3] = E
    idx2[998, 0] = -1
    st, M = _both(B, idx2, E)
    assert st == 8 and M == 999 * k - 2


def test_noalloc_permute_at_the_largest_expert_count(B):
    """E = 1024 with ~1M pairs: a chunk table near the array's limit."""
    E, k = 1024, 8
    T = (1 << 20) // k - 256
    _say(f"case noalloc permute: T={T} k={k} E={E} uniform")
    idx, _ = inputs.make_random_routing_only(T, E, k, 43, "cuda", "uniform")
    st, M = _both(B, idx, E)
    assert st == 0 and M == T * k


def test_noalloc_permute_refuses_tables_past_the_limit(B):
    E, k = 1024, 8
    T = (1 << 20) // k + 1024          # 1025 chunks of 1025 entries > 2^20
    shape = B.make_shape(T, 256, 128, E, k)
    o = _outs(E, 1, 0)
    P = 1 << 20    # an aligned stand-in address: the call is refused before any pointer is read
    with pytest.raises(B.MoEError) as ei:
        B.moe_permute_noalloc(shape, P, o[0], o[1], P, P, o[4])
    assert ei.value.status == 6
