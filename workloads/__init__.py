"""Seeded synthetic inputs for the fused post-experts boundary.

This module only *draws* inputs.  It holds none of the boundary's arithmetic: it
never sums partials, weights expert rows, applies a gate, adds a residual or
normalises.  The CPU oracle tests and the GPU path both take their inputs from
here, so they see identical bytes.

Workload shapes follow the decode boundary the pages describe: hidden sizes 7168
(DeepSeek-V3, sglang PR #37104 "fuse trailing TP all-reduce with final RMSNorm",
Performance table), 6144 (GLM-5.2, sglang PR #37196 "Share the CuTe DSL AR fusion
core ...", Known gaps) and 8192 with top_k=10 (same page, Known gaps: the shipped
routing profiles), 1-128 tokens (PR #37104, Performance table) and up to 8192 tokens
for the bandwidth roofline.

Representation
--------------
bf16 tensors are numpy ``uint16`` arrays of raw bf16 bit patterns; routing weights
and gate logits are ``float32``; the expanded-row index map is ``int32``.

Draw order (one ``numpy.random.Generator(PCG64(seed))``, fixed): partials
P_0..P_{R-1}, residual X, gamma, routing logits [T, E], expert rows [T*K, H],
shared-expert output S, gate logits g.  Values are drawn in float64 and stored as
bf16 (via float32, round-to-nearest-even).

Routing: logits ~ N(0,1); the top-K experts per token are taken by a stable sort
of the softmax probabilities (ties: lower expert id first), and the weights are
those K probabilities renormalised to sum to one (stored as float32).  Expanded
rows are ordered the way a grouped expert GEMM emits them: the (expert, token,
slot) triples are sorted lexicographically and ``idx[t, k]`` is the rank of
(t, k) in that order, so the gather is scattered while each row is contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "Case",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_case",
    "make_case_torch",
    "CONFIGS",
    "case_for_config",
    "to_torch",
]


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (inputs only; no NaN)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Case:
    """One call's worth of inputs, host side."""

    T: int
    H: int
    partials: List[np.ndarray]
    residual: np.ndarray
    gamma: np.ndarray
    weight_bias: float = 0.0
    eps: float = 1e-6
    expert_out: Optional[np.ndarray] = None  # [N, H] bf16 bits
    idx: Optional[np.ndarray] = None  # [T, K] int32
    weights: Optional[np.ndarray] = None  # [T, K] float32
    shared: Optional[np.ndarray] = None  # [T, H] bf16 bits
    gate: Optional[np.ndarray] = None  # [T] float32
    num_experts: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return len(self.partials)

    @property
    def K(self) -> int:
        return 0 if self.idx is None else int(self.idx.shape[1])

    @property
    def finalize(self) -> bool:
        return self.idx is not None


def _bf16(rng_values: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(rng_values.astype(np.float32))


def _routing(rng: np.random.Generator, T: int, E: int, K: int):
    """Top-K routing of N(0,1) logits; returns expert ids [T,K] and fp32 weights."""
    logits = rng.standard_normal((T, E))
    # softmax probabilities, then the K largest by a stable descending sort
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    ptop = np.take_along_axis(p, order, axis=1)
    w = (ptop / ptop.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int64), w


def _expanded_index(expert_ids: np.ndarray) -> np.ndarray:
    """Rank of (expert, t, k) in lexicographic order -> idx[t, k] (int32)."""
    T, K = expert_ids.shape
    t = np.repeat(np.arange(T), K)
    k = np.tile(np.arange(K), T)
    e = expert_ids.reshape(-1)
    order = np.lexsort((k, t, e))  # primary key e, then t, then k
    rank = np.empty(T * K, dtype=np.int64)
    rank[order] = np.arange(T * K)
    return rank.reshape(T, K).astype(np.int32)


def make_case(
    T: int,
    H: int,
    R: int,
    *,
    seed: int = 0,
    partial_std: float = 0.5,
    residual_std: float = 1.0,
    gamma_dist: str = "uniform",  # "uniform" -> U(0.5,1.5); "normal01" -> N(0,0.1)
    weight_bias: float = 0.0,
    eps: float = 1e-6,
    K: int = 0,
    num_experts: int = 256,
    expert_std: float = 0.3,
    shared: bool = False,
    shared_std: float = 0.3,
    gate: bool = False,
) -> Case:
    """Draw one case on the host (numpy), in the documented order."""
    if K > num_experts and K > 0:
        raise ValueError("top_k larger than the number of experts")
    rng = np.random.Generator(np.random.PCG64(seed))
    partials = [_bf16(rng.normal(0.0, partial_std, (T, H))) for _ in range(R)]
    residual = _bf16(rng.normal(0.0, residual_std, (T, H)))
    if gamma_dist == "uniform":
        gamma = _bf16(rng.uniform(0.5, 1.5, H))
    elif gamma_dist == "normal01":
        gamma = _bf16(rng.normal(0.0, 0.1, H))
    else:
        raise ValueError(gamma_dist)
    c = Case(T=T, H=H, partials=partials, residual=residual, gamma=gamma,
             weight_bias=float(weight_bias), eps=float(eps))
    if K > 0:
        experts, w = _routing(rng, T, num_experts, K)
        c.idx = _expanded_index(experts)
        c.weights = w
        c.expert_out = _bf16(rng.normal(0.0, expert_std, (T * K, H)))
        c.num_experts = num_experts
        c.meta["expert_ids"] = experts.astype(np.int32)
    if shared:
        c.shared = _bf16(rng.normal(0.0, shared_std, (T, H)))
    if gate:
        c.gate = rng.standard_normal(T).astype(np.float32)
    return c


# ---------------------------------------------------------------------------
# The workload shapes and the headline sweep.  Values a shape does not fix take
# those of the R=2 token sweep (partials N(0,0.5), residual N(0,1), gamma
# U(0.5,1.5)) and of the DeepSeek-shaped finalize (experts, shared N(0,0.3)).
# "N(0, s)" is read as standard deviation s.
# ---------------------------------------------------------------------------
CONFIGS = {
    # reduce + residual + RMSNorm, one token, R=2, partials N(0,1)
    "reduce_r2_t1": dict(H=7168, R=2, partial_std=1.0, T=(1,)),
    # reduce + residual + RMSNorm, token sweep, R=2
    "reduce_r2_sweep": dict(H=7168, R=2, T=(1, 2, 4, 8, 16, 32, 64, 128)),
    # DeepSeek-V3-shaped finalize: 256 experts, top-8, shared expert, R=8
    "deepseek_h7168_top8": dict(H=7168, R=8, K=8, num_experts=256, shared=True, T=(16,)),
    # GLM-5.2-shaped finalize: H=6144, top-8 of 256, R=8
    "glm_h6144_top8": dict(H=6144, R=8, K=8, num_experts=256, shared=True, T=(1, 4, 16, 64, 128)),
    # Qwen3.5-style large H: top-10 of 512, sigmoid-gated shared expert,
    # Gemma-style norm gamma N(0,0.1) with weight_bias 1
    "gated_h8192_top10": dict(H=8192, R=8, K=10, num_experts=512, shared=True, gate=True,
               gamma_dist="normal01", weight_bias=1.0, T=(128, 2048, 8192)),
    # headline sweep: H=7168, R=8, finalize with K=8 of 256 and the shared expert
    "headline": dict(H=7168, R=8, K=8, num_experts=256, shared=True,
                     T=(1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)),
}


def case_for_config(name: str, T: int, seed: int = 0, **overrides) -> Case:
    cfg = dict(CONFIGS[name])
    cfg.pop("T")
    cfg.update(overrides)
    H = cfg.pop("H")
    R = cfg.pop("R")
    return make_case(T, H, R, seed=seed, **cfg)


def to_torch(case: Case, device):
    """Move a host case to torch tensors on ``device`` (bf16 viewed from bits)."""
    import torch

    def b(x):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        return t.view(torch.bfloat16).to(device)

    def f(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)

    return dict(
        partials=[b(p) for p in case.partials],
        residual=b(case.residual),
        gamma=b(case.gamma),
        expert_out=b(case.expert_out),
        idx=f(case.idx),
        weights=f(case.weights),
        shared=b(case.shared),
        gate=f(case.gate),
    )


def make_case_torch(
    T: int,
    H: int,
    R: int,
    *,
    device,
    seed: int = 0,
    partial_std: float = 0.5,
    residual_std: float = 1.0,
    gamma_dist: str = "uniform",
    weight_bias: float = 0.0,
    eps: float = 1e-6,
    K: int = 0,
    num_experts: int = 256,
    expert_std: float = 0.3,
    shared: bool = False,
    shared_std: float = 0.3,
    gate: bool = False,
) -> dict:
    """Same recipe drawn with a seeded torch generator on ``device``.

    Used for the large shapes (gigabytes of input) where a host draw and copy
    would dominate; the bytes differ from :func:`make_case` but the recipe is the
    same.  Returns torch tensors plus the scalar arguments.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal(shape, std):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)

    out = dict(T=T, H=H, weight_bias=float(weight_bias), eps=float(eps))
    out["partials"] = [normal((T, H), partial_std) for _ in range(R)]
    out["residual"] = normal((T, H), residual_std)
    if gamma_dist == "uniform":
        out["gamma"] = (torch.rand((H,), generator=g, device=device) + 0.5).to(torch.bfloat16)
    else:
        out["gamma"] = normal((H,), 0.1)
    out["expert_out"] = out["idx"] = out["weights"] = out["shared"] = out["gate"] = None
    if K > 0:
        logits = torch.randn((T, num_experts), generator=g, device=device, dtype=torch.float64)
        p = torch.softmax(logits, dim=1)
        order = torch.argsort(-p, dim=1, stable=True)[:, :K]
        ptop = torch.gather(p, 1, order)
        out["weights"] = (ptop / ptop.sum(dim=1, keepdim=True)).to(torch.float32).contiguous()
        t = torch.arange(T, device=device).repeat_interleave(K)
        k = torch.arange(K, device=device).repeat(T)
        key = order.reshape(-1).to(torch.int64) * (T * K) + t * K + k
        perm = torch.argsort(key, stable=True)
        rank = torch.empty_like(perm)
        rank[perm] = torch.arange(T * K, device=device)
        out["idx"] = rank.reshape(T, K).to(torch.int32).contiguous()
        out["expert_out"] = normal((T * K, H), expert_std)
    if shared:
        out["shared"] = normal((T, H), shared_std)
    if gate:
        out["gate"] = torch.randn((T,), generator=g, device=device, dtype=torch.float32)
    return out
