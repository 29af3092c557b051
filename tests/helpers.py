"""Shared helpers of the test suite (no layer arithmetic lives here)."""
from __future__ import annotations

import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "grouped_gemm_02_amd", "libmoe.so")

# max-relative-error bounds (normwise by the reference's max magnitude)
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def max_rel_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are all-zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if scale == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return diff / scale


def header_symbols() -> list[str]:
    """Function names declared in include/moe.h."""
    import re
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))
