"""The split (unfused) flow on the GPU against the oracle's split definition.

Stage 1 (bf16 sum of partials, routed experts and shared expert) must equal the
oracle bit for bit; stage 2 follows the fused parity bar (residual bit-exact,
normed within tolerance).  Also covers the shapes the fused path declines
(H % 8 != 0, 2-byte aligned views), which run the scalar kernels, and the
``on_decline="split"`` fallback.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import bits, compare, say
from workloads import case_for_config, make_case, to_torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import reduce_moe_finalize_amd  # noqa: F401

    torch.cuda.set_device(DEV)
    yield
    torch.cuda.synchronize()


def run_split(t, case, residual_out=None, sum_out=None):
    import reduce_moe_finalize_amd as fb

    if case.finalize:
        return fb.split_moe_finalize_rmsnorm(
            t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
            shared_out=t["shared"], shared_gate_logits=t["gate"], eps=case.eps,
            weight_bias=case.weight_bias, residual_out=residual_out, sum_out=sum_out)
    if case.shared is not None:
        y = fb.split_sum(t["partials"], t["residual"], shared_out=t["shared"],
                         shared_gate_logits=t["gate"], out=sum_out)
        return fb.split_residual_rmsnorm(y, t["residual"], t["gamma"], case.eps, case.weight_bias,
                                         residual_out=residual_out)
    return fb.split_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], eps=case.eps,
                                   weight_bias=case.weight_bias, residual_out=residual_out,
                                   sum_out=sum_out)


def check_split(case, what, t=None):
    say(f"split {what}: T={case.T} H={case.H} R={case.R} K={case.K}")
    t = to_torch(case, DEV) if t is None else t
    y = torch.empty(case.T, case.H, dtype=torch.bfloat16, device=DEV)
    normed, resid = run_split(t, case, sum_out=y)
    torch.cuda.synchronize()
    ref = oracle.run_case_split(case)
    bad = np.argwhere(bits(y) != ref["sum"])
    assert bad.size == 0, f"{what}: stage-1 sum differs at {bad[:5].tolist()}"
    compare(bits(normed), bits(resid), ref, what)


@pytest.mark.parametrize("name,T", [("reduce_r2_t1", 1), ("reduce_r2_sweep", 16), ("deepseek_h7168_top8", 16), ("glm_h6144_top8", 64), ("gated_h8192_top10", 128),
                                    ("headline", 1), ("headline", 256)])
def test_split_workloads(name, T):
    check_split(case_for_config(name, T), f"{name}-T{T}")


@pytest.mark.parametrize("H", [12, 20, 1000, 7170, 16383])
def test_split_any_hidden(H):
    check_split(make_case(4, H, 3, seed=H, K=3, num_experts=8, shared=True, gate=True), f"H={H}")
    check_split(make_case(3, H, 2, seed=H + 1), f"H={H} reduce")


def _misaligned(x):
    """Same values, stored one element (2 bytes) past a 16-byte boundary."""
    flat = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
    v = flat[1:].view(x.shape)
    v.copy_(x)
    return v


def test_split_misaligned_views_and_in_place():
    case = make_case(6, 7168, 4, seed=41, K=4, num_experts=16, shared=True)
    t = to_torch(case, DEV)
    for k in ("residual", "expert_out", "shared", "gamma"):
        t[k] = _misaligned(t[k])
    t["partials"] = [_misaligned(p) for p in t["partials"]]
    assert t["residual"].data_ptr() % 16 == 2
    check_split(case, "misaligned", t=t)
    # in-place residual on the scalar stage-2 kernel
    say("split misaligned in place")
    normed, resid = run_split(t, case, residual_out=t["residual"])
    torch.cuda.synchronize()
    assert resid.data_ptr() == t["residual"].data_ptr()
    compare(bits(normed), bits(resid), oracle.run_case_split(case), "misaligned in place")


def test_on_decline_split_fallback():
    import reduce_moe_finalize_amd as fb

    case = make_case(5, 20, 2, seed=42, K=2, num_experts=8, shared=True)
    t = to_torch(case, DEV)
    say("on_decline fallback H=20")
    with pytest.raises(fb.FusedBoundaryDeclined):
        fb.fused_moe_finalize_rmsnorm(t["partials"], t["expert_out"], t["idx"], t["weights"],
                                      t["residual"], t["gamma"], shared_out=t["shared"])
    normed, resid = fb.fused_moe_finalize_rmsnorm(
        t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
        shared_out=t["shared"], on_decline="split")
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), oracle.run_case_split(case), "fallback")
    red = make_case(3, 12, 2, seed=43)
    rt = to_torch(red, DEV)
    n2, r2 = fb.fused_reduce_rmsnorm(rt["partials"], rt["residual"], rt["gamma"], on_decline="split")
    torch.cuda.synchronize()
    compare(bits(n2), bits(r2), oracle.run_case_split(red), "fallback reduce")


def test_stage2_is_the_fused_reduce_with_one_partial():
    import reduce_moe_finalize_amd as fb

    case = make_case(24, 7168, 1, seed=44)
    t = to_torch(case, DEV)
    say("stage 2 == fused R=1")
    n1, r1 = fb.split_residual_rmsnorm(t["partials"][0], t["residual"], t["gamma"])
    n2, r2 = fb.fused_reduce_rmsnorm([t["partials"][0]], t["residual"], t["gamma"], workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(r1, r2)


def test_split_skipped_slots_and_no_partials():
    case = make_case(8, 512, 0, seed=45, K=4, num_experts=8, shared=False)
    case.idx = case.idx.copy()
    case.weights = case.weights.copy()
    case.idx[0, 1] = -1
    case.idx[3, 3] = case.expert_out.shape[0]
    case.weights[0, 1] = np.float32("nan")
    case.weights[3, 3] = np.float32("inf")
    check_split(case, "skipped slots, R=0")


def test_forced_decline_on_headline_shape_falls_back_once():
    """The mocked runtime decline: an ordinary T=16 headline call declined from
    the host raises with its outputs untouched; with on_decline="split" the
    split flow runs instead (its stage 2 then also meets the decline and takes
    the scalar kernel) and matches the oracle's split definition."""
    import reduce_moe_finalize_amd as fb

    case = case_for_config("headline", 16)
    t = to_torch(case, DEV)
    out = torch.full((case.T, case.H), 3.0, dtype=torch.bfloat16, device=DEV)
    ro = torch.full_like(out, 5.0)
    say("forced decline, raise")
    with fb.force_decline():
        with pytest.raises(fb.FusedBoundaryDeclined):
            fb.fused_moe_finalize_rmsnorm(t["partials"], t["expert_out"], t["idx"], t["weights"],
                                          t["residual"], t["gamma"], shared_out=t["shared"],
                                          out=out, residual_out=ro)
        torch.cuda.synchronize()
        assert bool((out == 3.0).all()) and bool((ro == 5.0).all())
        say("forced decline, split fallback")
        normed, resid = fb.fused_moe_finalize_rmsnorm(
            t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
            shared_out=t["shared"], out=out, residual_out=ro, on_decline="split")
        torch.cuda.synchronize()
    assert normed.data_ptr() == out.data_ptr() and resid.data_ptr() == ro.data_ptr()
    compare(bits(normed), bits(resid), oracle.run_case_split(case), "forced decline")
    # outside the block the fused kernel runs again
    n2, r2 = fb.fused_moe_finalize_rmsnorm(t["partials"], t["expert_out"], t["idx"], t["weights"],
                                           t["residual"], t["gamma"], shared_out=t["shared"])
    torch.cuda.synchronize()
    compare(bits(n2), bits(r2), oracle.run_case(case), "after forced decline")


def test_forced_decline_on_reduce_entry_falls_back_once():
    """The same mocked decline on the reduce entry point, the trailing reduction
    + final RMSNorm of the NextN head (PR #37104, Changes and Correctness): a
    T=16, H=7168 call raises with its outputs untouched, and with
    on_decline="split" the split flow runs and matches the oracle's split
    definition."""
    import reduce_moe_finalize_amd as fb

    case = case_for_config("headline", 16, K=0, shared=False)
    t = to_torch(case, DEV)
    out = torch.full((case.T, case.H), 3.0, dtype=torch.bfloat16, device=DEV)
    ro = torch.full_like(out, 5.0)
    say("forced decline on the reduce entry, raise")
    with fb.force_decline():
        with pytest.raises(fb.FusedBoundaryDeclined):
            fb.fused_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], out=out,
                                    residual_out=ro)
        torch.cuda.synchronize()
        assert bool((out == 3.0).all()) and bool((ro == 5.0).all())
        say("forced decline on the reduce entry, split fallback")
        normed, resid = fb.fused_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], out=out,
                                                residual_out=ro, on_decline="split")
        torch.cuda.synchronize()
    assert normed.data_ptr() == out.data_ptr() and resid.data_ptr() == ro.data_ptr()
    compare(bits(normed), bits(resid), oracle.run_case_split(case), "reduce forced decline")
    n2, r2 = fb.fused_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"])
    torch.cuda.synchronize()
    compare(bits(n2), bits(r2), oracle.run_case(case), "reduce after forced decline")
