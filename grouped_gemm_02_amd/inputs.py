"""Seeded synthetic inputs for the MoE expert layer.

Shared by the oracle tests, the GPU parity tests and the benchmark. This module
only draws random numbers: it holds none of the layer's arithmetic (no
permutation, no matmul, no activation). Every tensor is drawn from a
``torch.Generator`` seeded per configuration, on the device the caller names,
so the oracle and the HIP path always see the same values within one process.

Workload recipe (the pages benchmark one MoE layer at Qwen3 shapes with
128 experts, top-8 and random routing, router excluded; see the MarkTechPost
article, "How fast is Prime Mega MoE?", single-layer table):

* x ~ N(0, 1), dY ~ N(0, 1), W13 and W2 ~ N(0, 0.02), all rounded to bf16.
* topk_w = softmax over the k slots of N(0, 1) logits (fp32). For k = 1 it is
  one component of a softmax over 8 logits, so it is not identically 1.
* "uniform" routing: k distinct experts per token, uniformly at random.
* "zipf" routing: expert popularity p_r proportional to r^-s (s = 1.2) for
  the hottest ranks 1..E-8 and zero for the 8 coldest ranks, ranks mapped to
  experts by a seeded permutation; each token draws k distinct experts without
  replacement in proportion to p (Gumbel top-k), so some experts get no rows
  and the hottest gets more than a tenth of them.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts
    k: int          # experts per token
    routing: str    # "uniform" | "zipf"
    precision: str  # "bf16" | "fp8_block" | "mxfp8" | "fp8_bwd" | "fp8_fp4" (forward only)
    seed: int
    zipf_s: float = 1.2
    zipf_cold: int = 8

    @property
    def M(self) -> int:
        return self.T * self.k

    def flops_fwd(self) -> float:
        return 6.0 * self.M * self.H * self.I

    def flops_bwd(self) -> float:
        return 12.0 * self.M * self.H * self.I

    def scaled(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny layer: several tiles only at the smallest tile sizes
    "tiny": LayerConfig("tiny", 64, 256, 128, 8, 2, "uniform", "bf16", 0),
    # Qwen3-30B-A3B-shaped layer, all 128 experts local
    "qwen3_30b": LayerConfig("qwen3_30b", 16384, 2048, 768, 128, 8, "uniform", "bf16", 1),
    # one EP=8 rank's share of the 30B layer: 16 local experts, 131072 rows
    "ep8_share": LayerConfig("ep8_share", 131072, 2048, 768, 16, 1, "uniform", "fp8_block_f32", 2),
    # Qwen3-235B-A22B-shaped layer
    "qwen3_235b": LayerConfig("qwen3_235b", 16384, 4096, 1536, 128, 8, "uniform", "fp8_bwd_f32", 3),
    # skewed routing on the 30B shape
    "zipf": LayerConfig("zipf", 16384, 2048, 768, 128, 8, "zipf", "mxfp8", 4),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_bf16(shape, std, g, device) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if out.numel() == 0:
        return out
    # draw slab by slab along the first axis to bound fp32 temporaries
    flat = out.view(shape[0], -1)
    step = max(1, (1 << 26) // max(1, flat.shape[1]))
    for s in range(0, shape[0], step):
        e = min(shape[0], s + step)
        r = torch.randn((e - s, flat.shape[1]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            r.mul_(std)
        flat[s:e].copy_(r)
    return out


def zipf_popularity(E: int, s: float, cold: int, g: torch.Generator, device) -> torch.Tensor:
    """Per-expert popularity (fp64, sums to 1): rank r gets r^-s, the `cold`
    coldest ranks get 0, ranks assigned to experts by a seeded permutation."""
    ranks = torch.arange(1, E + 1, dtype=torch.float64, device=device)
    p = ranks.pow(-s)
    if cold > 0:
        p[E - cold:] = 0.0
    p = p / p.sum()
    perm = torch.randperm(E, generator=g, device=device)
    pop = torch.empty_like(p)
    pop[perm] = p
    return pop


def make_routing(T: int, E: int, k: int, routing: str, g: torch.Generator, device,
                 zipf_s: float = 1.2, zipf_cold: int = 8):
    """topk_idx int32 [T, k] (distinct experts per token) and topk_w fp32 [T, k]."""
    if k > E:
        raise ValueError("k must not exceed E")
    if routing == "uniform":
        scores = torch.rand((T, E), generator=g, device=device)
    elif routing == "zipf":
        pop = zipf_popularity(E, zipf_s, zipf_cold, g, device)
        u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64)
        u = u.clamp_min(1e-300)
        gumbel = -torch.log(-torch.log(u))
        scores = torch.log(pop).unsqueeze(0) + gumbel
    else:
        raise ValueError(f"unknown routing {routing!r}")
    idx = torch.topk(scores, k, dim=1).indices.to(torch.int32)
    n_logits = max(k, 8) if k == 1 else k
    logits = torch.randn((T, n_logits), generator=g, device=device, dtype=torch.float32)
    w = torch.softmax(logits, dim=1)[:, :k].contiguous()
    return idx.contiguous(), w


def make_layer_inputs(cfg: LayerConfig, device="cpu", with_dy: bool = True) -> dict:
    """All inputs of one forward + backward call, as tensors on `device`."""
    g = _gen(cfg.seed, device)
    x = _normal_bf16((cfg.T, cfg.H), 1.0, g, device)
    idx, w = make_routing(cfg.T, cfg.E, cfg.k, cfg.routing, g, device, cfg.zipf_s, cfg.zipf_cold)
    W13 = _normal_bf16((cfg.E, 2 * cfg.I, cfg.H), 0.02, g, device)
    W2 = _normal_bf16((cfg.E, cfg.H, cfg.I), 0.02, g, device)
    out = {"x": x, "topk_idx": idx, "topk_w": w, "W13": W13, "W2": W2}
    if with_dy:
        out["dy"] = _normal_bf16((cfg.T, cfg.H), 1.0, g, device)
    return out


def make_random_routing_only(T: int, E: int, k: int, seed: int, device="cpu", routing="uniform"):
    g = _gen(seed, device)
    return make_routing(T, E, k, routing, g, device)


def make_router_logits(T: int, E: int, seed: int, device="cpu", skew: float = 0.0, ties: bool = False):
    """fp32 router logits [T, E]: N(0, 1) per (token, expert), plus a fixed
    per-expert bias -skew * log(1 + rank) (ranks a seeded permutation of the
    experts), so that skew > 0 concentrates tokens on a few experts the way
    Zipf-like popularity does. ties: logits rounded to multiples of 1/2
    (many equal values)."""
    g = _gen(seed, device)
    z = torch.randn((T, E), generator=g, device=device, dtype=torch.float32)
    if skew:
        rank = torch.randperm(E, generator=g, device=device).to(torch.float32)
        z = z - skew * torch.log1p(rank)[None, :]
    if ties:
        z = torch.round(z * 2.0) / 2.0
    return z


def describe(cfg: LayerConfig) -> str:
    return (f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} "
            f"routing={cfg.routing} precision={cfg.precision} seed={cfg.seed}")


__all__ = ["LayerConfig", "CONFIGS", "make_layer_inputs", "make_routing",
           "make_random_routing_only", "make_router_logits", "zipf_popularity", "describe"]
