"""The allocation-free entry point against the entry points that take a
workspace (needs a GPU).  Its split rows exchange through the library's static
per-GPU scratch, which every call on the GPU shares and which keeps the last
call's records, so calls of different shapes follow each other here."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import bits, call, compare, say
from workloads import make_case, to_torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import reduce_moe_finalize_amd  # noqa: F401  (raises if the library is missing)

    torch.cuda.set_device(DEV)
    yield
    torch.cuda.synchronize()


def _noalloc(t, finalize, case):
    import reduce_moe_finalize_amd as fb

    out = torch.empty(case.T, case.H, dtype=torch.bfloat16, device=DEV)
    ro = torch.empty_like(out)
    if finalize:
        return fb.fused_moe_finalize_rmsnorm_noalloc(
            t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
            shared_out=t.get("shared"), shared_gate_logits=t.get("gate"), eps=case.eps,
            weight_bias=case.weight_bias, out=out, residual_out=ro)
    return fb.fused_moe_finalize_rmsnorm_noalloc(
        t["partials"], None, None, None, t["residual"], t["gamma"], eps=case.eps,
        weight_bias=case.weight_bias, out=out, residual_out=ro)


def _check_against_workspace_entry(case, finalize, what):
    import reduce_moe_finalize_amd as fb

    t = to_torch(case, DEV)
    plan = fb.get_plan(case.T, case.H, case.R, case.K if finalize else 0,
                       finalize and case.shared is not None, fb.workspace_bytes(case.T, case.H))
    say(f"{what}: T={case.T} H={case.H} finalize={finalize} plan={plan}")
    n0, r0 = _noalloc(t, finalize, case)
    ws = torch.zeros(fb.workspace_bytes(case.T, case.H), dtype=torch.uint8, device=DEV)
    n1, r1 = call(t, finalize, eps=case.eps, weight_bias=case.weight_bias, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(r0), bits(r1)), f"{what}: residual differs from the workspace entry"
    assert np.array_equal(bits(n0), bits(n1)), f"{what}: normed differs from the workspace entry"
    compare(bits(n0), bits(r0), oracle.run_case(case), what)
    return plan


def test_noalloc_matches_workspace_entry_two_calls_second_smaller():
    big = make_case(64, 7168, 8, seed=80, K=8, num_experts=256, shared=True)
    small = make_case(5, 7168, 8, seed=81, K=8, num_experts=256, shared=True)
    p_big = _check_against_workspace_entry(big, True, "first call (T=64)")
    p_small = _check_against_workspace_entry(small, True, "second call, smaller (T=5)")
    assert p_big["split"] > 1 and p_small["split"] > 1  # both exchange through the scratch


def test_noalloc_reduce_and_gated_shapes_share_the_scratch():
    cases = [
        (make_case(16, 7168, 8, seed=82), False, "reduce T=16"),
        (make_case(128, 8192, 8, seed=83, K=10, num_experts=512, shared=True, gate=True,
                   gamma_dist="normal01", weight_bias=1.0), True, "gated top-10 T=128"),
        (make_case(300, 7168, 8, seed=84, K=8, num_experts=256, shared=True), True,
         "finalize T=300"),
        (make_case(3, 6144, 2, seed=85), False, "reduce T=3 H=6144"),
    ]
    for case, fin, what in cases:
        _check_against_workspace_entry(case, fin, what)


def test_noalloc_rejects_more_rows_than_the_scratch_holds():
    import reduce_moe_finalize_amd as fb

    T, H = fb.NOALLOC_MAX_ROWS + 1, 64
    case = make_case(T, H, 1, seed=86)
    t = to_torch(case, DEV)
    out = torch.full((T, H), 3.0, dtype=torch.bfloat16, device=DEV)
    ro = torch.full_like(out, 5.0)
    say("no-alloc entry beyond its row capacity")
    with pytest.raises(ValueError, match="FB_NOALLOC_MAX_ROWS"):
        fb.fused_moe_finalize_rmsnorm_noalloc(t["partials"], None, None, None, t["residual"],
                                              t["gamma"], out=out, residual_out=ro)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((ro == 5.0).all())
    # at the capacity itself it runs
    case = make_case(fb.NOALLOC_MAX_ROWS, H, 1, seed=87)
    _check_against_workspace_entry(case, False, "at capacity")


@pytest.mark.parametrize("T", [16, 300])
def test_noalloc_in_place_residual(T):
    """The allocation-free entry point with residual_out == residual_in (split
    latency rows at T=16, the balanced kernel at T=300): the same bits as the
    workspace entry point writing a separate residual_out."""
    import reduce_moe_finalize_amd as fb

    case = make_case(T, 7168, 8, seed=300 + T, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    say(f"noalloc in place: T={T}")
    ws = torch.zeros(fb.workspace_bytes(T, 7168), dtype=torch.uint8, device=DEV)
    n1, r1 = call(t, True, eps=case.eps, weight_bias=case.weight_bias, workspace=ws)
    torch.cuda.synchronize()
    n1, r1 = bits(n1), bits(r1)
    out = torch.empty(T, 7168, dtype=torch.bfloat16, device=DEV)
    fb.fused_moe_finalize_rmsnorm_noalloc(
        t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
        shared_out=t.get("shared"), shared_gate_logits=t.get("gate"), eps=case.eps,
        weight_bias=case.weight_bias, out=out, residual_out=t["residual"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(t["residual"]), r1)
    assert np.array_equal(bits(out), n1)
