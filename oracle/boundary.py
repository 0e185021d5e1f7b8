"""CPU oracle for the fused post-experts boundary.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``reduce_moe_finalize_amd``) never imports it, never calls it and has no CPU
fallback.  It shares no code with the HIP path.

What is computed (per token row t, rows independent)
----------------------------------------------------
The boundary folds the post-experts partial sums, the MoE finalize and the
shared-expert add into the next layer's input RMSNorm (sglang PR #37196, "Share
the CuTe DSL AR fusion core and wire it for DeepSeek-V3 / GLM-5.x", Motivation),
and writes both the normed activations and the updated residual (sglang PR
#37104, "fuse trailing TP all-reduce with final RMSNorm", Motivation: the
"residual RMSNorm" boundary)::

    x_t      = sum_r P_r[t]                                  # partial sums
             + sum_{k valid} w[t,k] * E[idx[t,k]]            # MoE finalize
             + s_t * S[t]                                    # shared expert (once)
             + X[t]                                          # residual
    residual = bf16(x_t)
    normed   = bf16( x_t / sqrt(mean_h(x_t^2) + eps) * (gamma + weight_bias) )

* The norm multiplies by ``(gamma + weight_bias)`` (PR #37196, Modifications
  part 1: the kernel scales by gamma plus weight_bias; weight_bias is 0 for
  both the plain and the Gemma flavour, whose stored weight already holds the +1).
  The root-mean-square form with eps inside the root over the mean is the
  standard RMSNorm definition, which the pages name but do not print.
* The shared expert is added exactly once (PR #37196, Modifications part 2: a
  replicated shared expert would otherwise be counted once per rank).  Where the
  family gates it with a sigmoid (Qwen3.5, same passage), ``s_t = sigmoid(g_t)``
  rounded once to fp32; otherwise ``s_t = 1``.
* A residual is required (PR #37104, Changes: fail loudly without one).
* Readings where the pages are silent: an index outside [0, N) marks a skipped
  slot; routing weights are applied as given (no renormalisation, no scaling).

Two tracks
----------
Track A (``*_f64``): every input read exactly into float64, summed in the fixed
canonical order (partials 0..R-1, expert slots 0..K-1, shared, residual), norm
in float64, each output rounded *directly* from float64 to bf16 (round to
nearest, ties to even).  This is the reference for ``normed``.

Track B (``residual_contract``): the same order, every step one IEEE float32
operation with no fused multiply-add (``a = 0``; ``a += P_r``; ``a += fl32(w*E)``;
``a += fl32(s*S)``; ``a += X``), then bf16.  This is the exact value the
residual output must equal: the bf16 rounding of the fp32 sum.

Parity status: every function here is pinned by CPU tests (closed forms, a
50-digit decimal brute force, torch's fp64 rms_norm, bf16 rounding cases).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "bf16_to_f64",
    "f64_to_bf16",
    "shared_scale",
    "accumulate_f64",
    "accumulate_f32",
    "rms_norm_f64",
    "evaluate",
    "split_evaluate",
    "reduce_rmsnorm",
    "moe_finalize_rmsnorm",
]

# bf16: 8 significant bits, exponent range of fp32
_BF16_SIG_BITS = 8
_BF16_MIN_NORMAL_EXP = -126  # smallest normal 2**-126
_BF16_QUANTUM_MIN = 2.0 ** (_BF16_MIN_NORMAL_EXP - (_BF16_SIG_BITS - 1))  # subnormal step 2**-133
_BF16_OVERFLOW = 2.0 ** 128


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bits, one rounding (to nearest, ties to even).

    For |x| in binade [2**(e-1), 2**e) the bf16 spacing is 2**(e-8) (8
    significant bits), never below the subnormal step 2**-133.  Dividing by the
    spacing is exact in float64 (a power of two), ``np.rint`` rounds half to
    even, and multiplying back is exact.  Results at or above 2**128 are
    infinities; NaN maps to the canonical quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, e = np.frexp(x)  # x = mant * 2**e, 0.5 <= |mant| < 1
    del mant
    quantum = np.ldexp(1.0, e - _BF16_SIG_BITS)
    quantum = np.maximum(quantum, _BF16_QUANTUM_MIN)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(x / quantum) * quantum
        r = np.where(np.abs(r) >= _BF16_OVERFLOW, np.copysign(np.inf, x), r)
    r = np.where(np.isinf(x), x, r)
    bits = (np.ascontiguousarray(r.astype(np.float32)).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits


def shared_scale(gate_logits: Optional[np.ndarray], T: int) -> np.ndarray:
    """Per-token shared-expert scale as float32.

    Gated (Qwen3.5 family, PR #37196 Modifications part 2): sigmoid of the fp32
    logit evaluated in float64 and rounded once to float32.  Ungated
    (DeepSeek/GLM family): exactly 1.
    """
    if gate_logits is None:
        return np.ones(T, dtype=np.float32)
    g = np.asarray(gate_logits, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-g))).astype(np.float32)


def _valid_slots(idx: np.ndarray, N: int) -> np.ndarray:
    return (idx >= 0) & (idx < N)


def accumulate_f64(partials, residual, expert_out=None, idx=None, weights=None,
                   shared=None, gate=None) -> np.ndarray:
    """Track A pre-norm row sum x in float64, canonical order.  Returns [T, H]."""
    X = bf16_to_f64(residual)
    T, H = X.shape
    x = np.zeros((T, H), dtype=np.float64)
    for P in partials:  # partial sums, r = 0 .. R-1
        x += bf16_to_f64(P)
    if idx is not None:  # MoE finalize, slot k = 0 .. K-1
        N = expert_out.shape[0]
        idx = np.asarray(idx, dtype=np.int64)
        w = np.asarray(weights, dtype=np.float32).astype(np.float64)
        valid = _valid_slots(idx, N)
        for k in range(idx.shape[1]):
            rows = np.nonzero(valid[:, k])[0]
            if rows.size:
                E = bf16_to_f64(expert_out[idx[rows, k]])
                x[rows] += w[rows, k][:, None] * E  # exact product in fp64
    if shared is not None:  # shared expert, added once
        s = shared_scale(gate, T).astype(np.float64)
        x += s[:, None] * bf16_to_f64(shared)
    x += X  # residual
    return x


def accumulate_f32(partials, residual, expert_out=None, idx=None, weights=None,
                   shared=None, gate=None) -> np.ndarray:
    """Track B pre-norm row sum in IEEE float32, same order, no FMA.  [T, H]."""
    X = bf16_to_f64(residual).astype(np.float32)
    T, H = X.shape
    a = np.zeros((T, H), dtype=np.float32)  # +0.0
    for P in partials:
        a = a + bf16_to_f64(P).astype(np.float32)
    if idx is not None:
        N = expert_out.shape[0]
        idx = np.asarray(idx, dtype=np.int64)
        w = np.asarray(weights, dtype=np.float32)
        valid = _valid_slots(idx, N)
        for k in range(idx.shape[1]):
            rows = np.nonzero(valid[:, k])[0]
            if rows.size:
                E = bf16_to_f64(expert_out[idx[rows, k]]).astype(np.float32)
                p = w[rows, k][:, None] * E  # one fp32 rounding
                a[rows] = a[rows] + p
    if shared is not None:
        s = shared_scale(gate, T)
        a = a + s[:, None] * bf16_to_f64(shared).astype(np.float32)
    a = a + X
    return a


def rms_norm_f64(x: np.ndarray, gamma, weight_bias: float, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * (gamma + weight_bias), all float64.

    ``weight_bias`` and ``eps`` are taken as the float32 values a caller passes.
    """
    H = x.shape[-1]
    wb = float(np.float32(weight_bias))
    e = float(np.float32(eps))
    scale = bf16_to_f64(gamma) + wb
    ms = np.sum(x * x, axis=-1, keepdims=True) / H
    return x / np.sqrt(ms + e) * scale


def evaluate(partials: Sequence[np.ndarray], residual: np.ndarray, gamma: np.ndarray,
             weight_bias: float = 0.0, eps: float = 1e-6, expert_out=None, idx=None,
             weights=None, shared=None, gate=None, chunk_rows: int = 256,
             keep_unrounded: bool = False) -> dict:
    """Both tracks for a whole call, rows processed in chunks.

    Returns a dict of bf16 bit arrays: ``normed`` (track A), ``residual``
    (track A) and ``residual_contract`` (track B); with ``keep_unrounded`` also
    the float64 ``x`` and ``y``.
    """
    residual = np.asarray(residual)
    T, H = residual.shape
    out = {
        "normed": np.empty((T, H), np.uint16),
        "residual": np.empty((T, H), np.uint16),
        "residual_contract": np.empty((T, H), np.uint16),
    }
    if keep_unrounded:
        out["x"] = np.empty((T, H), np.float64)
        out["y"] = np.empty((T, H), np.float64)
    for r0 in range(0, T, chunk_rows):
        sl = slice(r0, min(T, r0 + chunk_rows))
        kw = dict(
            partials=[np.asarray(P)[sl] for P in partials],
            residual=residual[sl],
            expert_out=expert_out,
            idx=None if idx is None else np.asarray(idx)[sl],
            weights=None if weights is None else np.asarray(weights)[sl],
            shared=None if shared is None else np.asarray(shared)[sl],
            gate=None if gate is None else np.asarray(gate)[sl],
        )
        x = accumulate_f64(**kw)
        y = rms_norm_f64(x, gamma, weight_bias, eps)
        out["normed"][sl] = f64_to_bf16(y)
        out["residual"][sl] = f64_to_bf16(x)
        out["residual_contract"][sl] = f64_to_bf16(accumulate_f32(**kw).astype(np.float64))
        if keep_unrounded:
            out["x"][sl] = x
            out["y"][sl] = y
    return out


def split_evaluate(partials: Sequence[np.ndarray], residual: np.ndarray, gamma: np.ndarray,
                   weight_bias: float = 0.0, eps: float = 1e-6, expert_out=None, idx=None,
                   weights=None, shared=None, gate=None, chunk_rows: int = 256) -> dict:
    """The unfused (split) flow the fused boundary replaces.

    The pages compare the fused boundary against two launches: the reduction
    (and the MoE finalize) materialised as a bf16 tensor, then a separate
    residual RMSNorm (sglang PR #37104, Motivation and Performance table; the
    owed reduction materialised before the ordinary norm after a decline, same
    page, Changes; the standalone deferred finalize, PR #37196, Modifications
    part 2).  Stage 1 is the bf16 rounding of the fp32 canonical-order sum of
    partials, expert slots and shared expert (track B arithmetic without the
    residual); stage 2 is the fused definition applied to that single tensor and
    the residual.  Returns ``sum`` (stage 1, bf16 bits) plus the keys of
    :func:`evaluate` for stage 2.
    """
    residual = np.asarray(residual)
    T, H = residual.shape
    y = np.empty((T, H), np.uint16)
    zero = np.zeros((min(T, chunk_rows), H), np.uint16)  # +0: leaves the fp32 sum unchanged
    for r0 in range(0, T, chunk_rows):
        sl = slice(r0, min(T, r0 + chunk_rows))
        n = sl.stop - sl.start
        a = accumulate_f32([np.asarray(P)[sl] for P in partials], zero[:n], expert_out=expert_out,
                           idx=None if idx is None else np.asarray(idx)[sl],
                           weights=None if weights is None else np.asarray(weights)[sl],
                           shared=None if shared is None else np.asarray(shared)[sl],
                           gate=None if gate is None else np.asarray(gate)[sl])
        y[sl] = f64_to_bf16(a.astype(np.float64))
    out = evaluate([y], residual, gamma, weight_bias, eps, chunk_rows=chunk_rows)
    out["sum"] = y
    return out


def reduce_rmsnorm(partials, residual, gamma, weight_bias=0.0, eps=1e-6, **kw) -> dict:
    """Partial sums + residual + RMSNorm (no MoE finalize)."""
    return evaluate(partials, residual, gamma, weight_bias, eps, **kw)


def moe_finalize_rmsnorm(partials, expert_out, idx, weights, shared, gate, residual, gamma,
                         weight_bias=0.0, eps=1e-6, **kw) -> dict:
    """Partial sums + MoE finalize (+ optional gated shared expert) + residual + RMSNorm."""
    return evaluate(partials, residual, gamma, weight_bias, eps, expert_out=expert_out,
                    idx=idx, weights=weights, shared=shared, gate=gate, **kw)


def run_case_split(case, **kw) -> dict:
    """Convenience: the split flow for a :class:`workloads.Case`-like object."""
    return split_evaluate(case.partials, case.residual, case.gamma, case.weight_bias, case.eps,
                          expert_out=case.expert_out, idx=case.idx, weights=case.weights,
                          shared=case.shared, gate=case.gate, **kw)


def run_case(case, **kw) -> dict:
    """Convenience: evaluate a :class:`workloads.Case`-like object."""
    return evaluate(case.partials, case.residual, case.gamma, case.weight_bias, case.eps,
                    expert_out=case.expert_out, idx=case.idx, weights=case.weights,
                    shared=case.shared, gate=case.gate, **kw)
