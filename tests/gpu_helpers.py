"""Shared helpers for the GPU parity tests: run the HIP path through the binding,
bring results back as bf16 bit patterns, and compare with the oracle."""
from __future__ import annotations

import sys
from types import SimpleNamespace

import numpy as np
import torch

import oracle

ATOL = 2e-2  # normed: |gpu - ref| <= ATOL + RTOL * |ref|  (bf16 outputs)
RTOL = 1e-2


def say(msg: str):
    sys.stderr.write(f"[gpu] {msg}\n")
    sys.stderr.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def call(t: dict, finalize: bool, eps=1e-6, weight_bias=0.0, workspace="auto", out=None,
         residual_out=None):
    import reduce_moe_finalize_amd as fb

    if finalize:
        return fb.fused_moe_finalize_rmsnorm(
            t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
            shared_out=t.get("shared"), shared_gate_logits=t.get("gate"), eps=eps,
            weight_bias=weight_bias, workspace=workspace, out=out, residual_out=residual_out)
    return fb.fused_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], eps=eps,
                                   weight_bias=weight_bias, workspace=workspace, out=out,
                                   residual_out=residual_out)


def compare(normed_bits, resid_bits, ref, what=""):
    """Assert the parity bar: residual bit-exact vs the fp32 contract, normed in tolerance."""
    bad = np.argwhere(resid_bits != ref["residual_contract"])
    assert bad.size == 0, (f"{what}: residual differs from bf16(fp32 sum) at {bad[:5].tolist()} "
                           f"({len(bad)} elements)")
    a = oracle.bf16_to_f64(normed_bits)
    b = oracle.bf16_to_f64(ref["normed"])
    err = np.abs(a - b)
    lim = ATOL + RTOL * np.abs(b)
    worst = np.argwhere(~(err <= lim))
    assert worst.size == 0, (f"{what}: normed outside tolerance at {worst[:5].tolist()}, "
                             f"max|diff|={np.nanmax(err):.4g}")
    # away from cancellation (|ref| >= 1/64) the rounded results are at most 1 bf16 ulp apart
    big = np.abs(b) >= 1.0 / 64
    if np.any(big):
        ulp = 2.0 ** (np.floor(np.log2(np.abs(b[big]))) - 7)
        worst_ulp = float(np.max(err[big] / ulp))
        assert worst_ulp <= 1.0, f"{what}: normed off by {worst_ulp} bf16 ulp"
    return float(np.nanmax(err)) if err.size else 0.0


def torch_case_to_host(t: dict, rows: np.ndarray):
    """Gather the inputs of ``rows`` (and the expert rows they reference) to the host,
    as a Case-like namespace the oracle can evaluate.  Rows are independent, so the
    oracle's result for these rows equals its result for the full call."""
    dev = t["residual"].device
    r = torch.from_numpy(rows.astype(np.int64)).to(dev)

    def host_rows(x):
        return bits(x.index_select(0, r))

    ns = SimpleNamespace(
        partials=[host_rows(p) for p in t["partials"]],
        residual=host_rows(t["residual"]),
        gamma=bits(t["gamma"]),
        weight_bias=t.get("weight_bias", 0.0),
        eps=t.get("eps", 1e-6),
        expert_out=None, idx=None, weights=None, shared=None, gate=None,
    )
    if t.get("idx") is not None:
        idx = t["idx"].index_select(0, r)  # [n, K]
        N = t["expert_out"].shape[0]
        flat = idx.reshape(-1).to(torch.int64)
        valid = (flat >= 0) & (flat < N)
        safe = torch.where(valid, flat, torch.zeros_like(flat))
        ns.expert_out = bits(t["expert_out"].index_select(0, safe))
        local = torch.arange(flat.numel(), device=dev)
        local = torch.where(valid, local, torch.full_like(local, -1))
        ns.idx = local.reshape(idx.shape).to(torch.int32).cpu().numpy()
        ns.weights = t["weights"].index_select(0, r).cpu().numpy()
    if t.get("shared") is not None:
        ns.shared = host_rows(t["shared"])
    if t.get("gate") is not None:
        ns.gate = t["gate"].index_select(0, r).cpu().numpy()
    return ns


def sample_rows(T: int) -> np.ndarray:
    rows = set(range(min(16, T))) | set(range(max(0, T - 16), T)) | set(range(0, T, 64))
    return np.array(sorted(rows), dtype=np.int64)
