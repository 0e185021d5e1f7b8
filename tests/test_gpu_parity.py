"""Parity of the HIP path with the CPU oracle, through the C ABI (needs a GPU).

Bar: residual_out bit-exact to bf16 of the fp32 canonical-order sum (oracle
track B); normed_out within |d| <= 2e-2 + 1e-2 |ref| of the fp64 reference
(oracle track A) and within 1 bf16 ulp away from cancellation.
"""
import contextlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import bits, call, compare, sample_rows, say, torch_case_to_host
from workloads import CONFIGS, case_for_config, make_case, make_case_torch, to_torch

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


def run_and_check(case, what, workspace="auto"):
    say(f"{what}: T={case.T} H={case.H} R={case.R} K={case.K} "
        f"shared={case.shared is not None} gate={case.gate is not None}")
    t = to_torch(case, DEV)
    normed, resid = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias,
                         workspace=workspace)
    torch.cuda.synchronize()
    ref = oracle.run_case(case)
    return compare(bits(normed), bits(resid), ref, what), bits(normed), bits(resid)


# ------------------------------------------------------------- the five workloads
def test_reduce_r2_single_token():
    run_and_check(case_for_config("reduce_r2_t1", 1), "reduce_r2_t1")


@pytest.mark.parametrize("T", CONFIGS["reduce_r2_sweep"]["T"])
def test_reduce_r2_token_sweep(T):
    run_and_check(case_for_config("reduce_r2_sweep", T), "reduce_r2_sweep")


def test_deepseek_h7168_top8_finalize():
    run_and_check(case_for_config("deepseek_h7168_top8", 16), "deepseek_h7168_top8")


@pytest.mark.parametrize("T", CONFIGS["glm_h6144_top8"]["T"])
def test_glm_h6144_top8_finalize(T):
    run_and_check(case_for_config("glm_h6144_top8", T), "glm_h6144_top8")


def test_gated_h8192_top10_t128():
    run_and_check(case_for_config("gated_h8192_top10", 128), "gated_h8192_top10")


@pytest.mark.parametrize("T", [192, 300, 640])
def test_gated_h8192_top10_at_plan_boundaries(T):
    """The config-5 shape (512-lane latency variant) where the automatic plan
    splits rows 4 ways (T = 192, 300) and where it streams 2 vectors per lane."""
    run_and_check(case_for_config("gated_h8192_top10", T, seed=T), f"gated H=8192 top-10 T={T}")


@pytest.mark.parametrize("name,T,streamed", [
    ("headline", 274, False), ("headline", 275, True), ("headline", 365, True),
    ("headline", 366, False), ("glm_h6144_top8", 320, False), ("glm_h6144_top8", 321, True),
    ("glm_h6144_top8", 426, True), ("glm_h6144_top8", 427, False),
    ("gated_h8192_top10", 257, True), ("gated_h8192_top10", 320, True),
    ("gated_h8192_top10", 321, False)])
def test_streamed_form_at_its_plan_boundaries(name, T, streamed):
    """Both sides of each boundary of the balanced kernel's streamed form (15
    to 20 units of 512 elements per CU at H = 6144 / 7168 / 8192): the automatic
    plan takes the form exactly inside, and matches the oracle on both sides."""
    import reduce_moe_finalize_amd as fb

    case = case_for_config(name, T, seed=T)
    plan = fb.get_plan(T, case.H, case.R, case.K, True, fb.workspace_bytes(T, case.H))
    assert (plan["units_per_wave"] == 1 and plan["sources_per_batch"] == 2) == streamed, plan
    run_and_check(case, f"{name} T={T} streamed={streamed}")


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16, 32, 64, 128, 256, 300, 512, 640, 1024])
@pytest.mark.parametrize("finalize", [False, True], ids=["reduce", "finalize"])
def test_headline_sweep(T, finalize):
    over = {} if finalize else dict(K=0, shared=False)
    run_and_check(case_for_config("headline", T, **over), f"headline-{'fin' if finalize else 'red'}")


# Full-size shapes: inputs drawn on the GPU, outputs checked on sampled rows
# (rows are independent, so the oracle evaluates just those rows).
LARGE = [
    ("headline-fin", dict(H=7168, R=8, K=8, num_experts=256, shared=True), 2048),
    ("headline-fin", dict(H=7168, R=8, K=8, num_experts=256, shared=True), 8192),
    ("headline-red", dict(H=7168, R=8), 8192),
    ("gated_h8192_top10", dict(H=8192, R=8, K=10, num_experts=512, shared=True, gate=True, gamma_dist="normal01",
                weight_bias=1.0), 2048),
    ("gated_h8192_top10", dict(H=8192, R=8, K=10, num_experts=512, shared=True, gate=True, gamma_dist="normal01",
                weight_bias=1.0), 8192),
    # 4 vectors per lane on 192-lane workgroups, 4 per CU (16+ rows per CU)
    ("glm_h6144_top8", dict(H=6144, R=8, K=8, num_experts=256, shared=True), 4096),
    ("H5120", dict(H=5120, R=8, K=8, num_experts=256, shared=True), 4096),
    ("H5120-red", dict(H=5120, R=8), 8192),
    # narrow rows: 2 vectors per lane at about 16 waves per CU
    ("H2048", dict(H=2048, R=8, K=8, num_experts=256, shared=True), 8192),
    ("H1024-red", dict(H=1024, R=8), 4096),
    # wide rows: 2 vectors per lane on one 1024-lane workgroup per CU (H=16384);
    # 4 vectors per lane at 12 waves per CU (H=12288)
    ("H16384", dict(H=16384, R=8, K=8, num_experts=256, shared=True), 4096),
    ("H12288-red", dict(H=12288, R=8), 4096),
]


@pytest.mark.parametrize("name,cfg,T", LARGE, ids=[f"{n}-T{T}" for n, _, T in LARGE])
def test_full_size_sampled(name, cfg, T):
    cfg = dict(cfg)
    H, R = cfg.pop("H"), cfg.pop("R")
    say(f"{name} full size T={T} H={H} R={R} {cfg}")
    t = make_case_torch(T, H, R, device=DEV, seed=1, **cfg)
    fin = t["idx"] is not None
    normed, resid = call(t, fin, eps=t["eps"], weight_bias=t["weight_bias"])
    torch.cuda.synchronize()
    rows = sample_rows(T)
    host = torch_case_to_host(t, rows)
    ref = oracle.run_case(host)
    r = torch.from_numpy(rows).to(DEV)
    compare(bits(normed.index_select(0, r)), bits(resid.index_select(0, r)), ref, f"{name}-T{T}")


# ------------------------------------------------------------- every launch shape
PLANS = [
    # latency kernel: (block, 1, 0) -> rows split ceil(896 / block) ways
    (64, 1, 0), (128, 1, 0), (192, 1, 0), (256, 1, 0), (448, 1, 0), (896, 1, 0), (1024, 1, 0),
    # stream kernel: (block, vectors per lane, sources per batch)
    (1024, 1, 1), (896, 1, 8), (512, 2, 1), (448, 2, 4), (256, 4, 1), (256, 4, 2), (256, 4, 4),
    (256, 4, 8), (128, 8, 1), (128, 8, 2), (128, 8, 8),
    # stream kernel held to a number of workgroups per CU: (block, vpt, batch, per CU)
    (256, 4, 1, 3), (128, 8, 1, 4), (128, 8, 2, 2), (448, 2, 2, 16),
]


@pytest.mark.parametrize("plan", PLANS, ids=["x".join(map(str, p)) for p in PLANS])
def test_every_plan_same_residual(plan):
    import reduce_moe_finalize_amd as fb

    case = make_case(20, 7168, 3, seed=11, K=4, num_experts=32, shared=True, gate=True)
    say(f"plan {plan}")
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    with fb.plan_override(*plan):
        normed, resid = call(t, True)
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), ref, f"plan {plan}")


@pytest.mark.parametrize("block", [64, 192, 512])
def test_latency_kernel_top10(block):
    """R = 8 with K in 9..12 selects the 12-slot latency variant (blocks up to 512)."""
    import reduce_moe_finalize_amd as fb

    case = make_case(9, 8192, 8, seed=13, K=10, num_experts=512, shared=True, gate=True,
                     gamma_dist="normal01", weight_bias=1.0)
    case.idx = case.idx.copy()
    case.idx[2, 9] = -1  # one skipped slot among the ten
    say(f"latency top-10 block={block}")
    t = to_torch(case, DEV)
    with fb.plan_override(block, 1, 0):
        normed, resid = call(t, True, weight_bias=1.0)
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), oracle.run_case(case), f"top-10 latency {block}")


@pytest.mark.parametrize("block", [64, 128, 256])
def test_latency_kernel_large_r_k(block):
    """R + 2 > 10 or K > 8 selects the wide latency variant (blocks up to 256)."""
    import reduce_moe_finalize_amd as fb

    case = make_case(6, 7168, 12, seed=12, K=10, num_experts=64, shared=True, gate=True)
    say(f"latency large R,K block={block}")
    t = to_torch(case, DEV)
    with fb.plan_override(block, 1, 0):
        normed, resid = call(t, True)
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), oracle.run_case(case), f"large latency {block}")
    with pytest.raises(ValueError):  # too wide for the R=12, K=10 variant
        with fb.plan_override(512, 1, 0):
            call(t, True)


# Register-slot boundaries of the latency variants: slot 0 residual, slot 1 shared
# (a zero-masked dummy without one), slots 2.. partials; R + 2 > 10 or K > 12
# selects the wide variant.  T=16 takes the latency kernel at these sizes.
VARIANT_EDGES = [(8, 0, False), (9, 0, False), (16, 0, False), (8, 8, False), (8, 8, True),
                 (9, 8, True), (1, 8, True), (0, 12, True), (8, 12, False), (2, 13, True)]


@pytest.mark.parametrize("R,K,shared", VARIANT_EDGES, ids=[f"R{r}-K{k}-{'S' if s else 'noS'}"
                                                          for r, k, s in VARIANT_EDGES])
def test_latency_variant_slot_edges(R, K, shared):
    ne = max(64, 2 * K)
    run_and_check(make_case(16, 2048, R, seed=70 + 3 * R + K, K=K, num_experts=ne, shared=shared,
                            gate=shared and K % 2 == 0), f"slots R={R} K={K}")


# ------------------------------------------------------------- edge cases
@pytest.mark.parametrize("H", [8, 24, 64, 520, 1032, 7176, 16384])
def test_ragged_and_extreme_hidden(H):
    run_and_check(make_case(5, H, 2, seed=H, K=3, num_experts=8, shared=True), f"H={H}")
    run_and_check(make_case(3, H, 1, seed=H + 1), f"H={H} reduce")


def test_max_partials_and_top_k():
    run_and_check(make_case(9, 2048, 16, seed=21, K=16, num_experts=64, shared=True, gate=True),
                  "R=16 K=16")


def test_no_partials_finalize_only():
    run_and_check(make_case(7, 4096, 0, seed=22, K=8, num_experts=256), "R=0")


def test_skipped_slots_ignore_their_weights():
    case = make_case(12, 1024, 2, seed=23, K=6, num_experts=64, shared=True)
    N = case.expert_out.shape[0]
    case.idx = case.idx.copy()
    case.weights = case.weights.copy()
    case.idx[0, :] = -1
    case.idx[1, 2] = N
    case.idx[2, 5] = 2**31 - 1
    case.idx[3, 0] = -(2**31)
    for (r, k) in [(0, 0), (0, 3), (1, 2), (2, 5), (3, 0)]:
        case.weights[r, k] = np.float32("nan")  # a skipped slot contributes nothing
    run_and_check(case, "skipped slots")


@pytest.mark.parametrize("T", [1, 16, 33, 192, 300, 640, 2048])
@pytest.mark.parametrize("finalize", [True, False], ids=["finalize", "reduce"])
def test_in_place_residual(T, finalize):
    """residual_out == residual_in under every kind of plan the T walks through
    (split latency rows, whole latency rows, the balanced kernel, the stream
    kernel): the outputs are the oracle's, and the same bits as a call that
    writes a separate residual_out, call after call on one workspace."""
    import reduce_moe_finalize_amd as fb

    kw = dict(K=8, num_experts=256, shared=True) if finalize else {}
    case = make_case(T, 7168, 8, seed=24 + T, **kw)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    ws = torch.zeros(fb.workspace_bytes(T, 7168), dtype=torch.uint8, device=DEV)
    plan = fb.get_plan(T, 7168, 8, 8 if finalize else 0, finalize, ws.numel())
    say(f"in-place residual T={T} finalize={finalize} plan={plan}")
    n0, r0 = call(t, finalize, workspace=ws)
    torch.cuda.synchronize()
    n0, r0 = bits(n0), bits(r0)
    resid0 = t["residual"].clone()
    for _ in range(3):
        t["residual"].copy_(resid0)
        normed, resid = call(t, finalize, residual_out=t["residual"], workspace=ws)
        torch.cuda.synchronize()
        assert resid.data_ptr() == t["residual"].data_ptr()
        assert np.array_equal(bits(normed), n0) and np.array_equal(bits(resid), r0)
    compare(n0, r0, ref, "in place")
    assert fb.workspace_status(ws) == 0


@pytest.mark.parametrize("T", [16, 300, 640])
def test_in_place_residual_that_is_also_a_partial(T):
    """A partial buffer that is the residual buffer itself, updated in place:
    every lane reads both at the position it later writes (split rows only
    after their exchange), so the result is the oracle's for that input."""
    case = make_case(T, 7168, 4, seed=40 + T, K=8, num_experts=256, shared=True)
    case.partials[0] = case.residual.copy()
    ref = oracle.run_case(case)
    t = to_torch(case, DEV)
    t["partials"][0] = t["residual"]
    say(f"in place, partial 0 is the residual: T={T}")
    normed, resid = call(t, True, residual_out=t["residual"])
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), ref, "partial is the residual")


def test_zero_tokens_is_noop():
    import reduce_moe_finalize_amd as fb

    r = torch.empty((0, 7168), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(7168, dtype=torch.bfloat16, device=DEV)
    n, o = fb.fused_reduce_rmsnorm([r], r, g)
    assert n.shape == (0, 7168) and o.shape == (0, 7168)


def test_constant_rows_give_gamma_bitwise():
    T, H = 40, 7168
    case = make_case(T, H, 2, seed=25)
    one = np.uint16(0x3F80)
    half = np.uint16(0x3F00)
    case.partials = [np.full((T, H), half, np.uint16), np.full((T, H), half, np.uint16)]
    case.residual = np.full((T, H), np.uint16(0x8000), np.uint16)  # -0
    t = to_torch(case, DEV)
    say("constant rows")
    normed, resid = call(t, False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(resid), np.full((T, H), one, np.uint16))
    assert np.array_equal(bits(normed), np.broadcast_to(case.gamma, (T, H)))


def test_zero_and_negative_zero_rows():
    T, H = 4, 512
    case = make_case(T, H, 2, seed=26)
    case.partials = [np.full((T, H), np.uint16(0x8000), np.uint16)] * 2
    case.residual = np.full((T, H), np.uint16(0x8000), np.uint16)
    t = to_torch(case, DEV)
    say("zero rows")
    normed, resid = call(t, False)
    torch.cuda.synchronize()
    assert np.all(bits(resid) == 0x0000)  # the sum starts at +0: -0 + -0 ... stays +0
    assert np.all(bits(normed) == 0x0000)


def test_negative_zero_rows_with_masked_slots():
    """All-(-0) sources through the finalize with a skipped slot, a gated shared
    expert and masked register slots: every masked slot adds +0, and the sum
    starts at +0, so the result is +0 exactly as the fp32 contract says."""
    T, H = 6, 1024
    case = make_case(T, H, 1, seed=27, K=3, num_experts=8, shared=True, gate=True)
    nz = np.uint16(0x8000)
    case.partials = [np.full((T, H), nz, np.uint16)]
    case.residual = np.full((T, H), nz, np.uint16)
    case.shared = np.full((T, H), nz, np.uint16)
    case.expert_out = np.full_like(case.expert_out, nz)
    case.idx = case.idx.copy()
    case.idx[1, 2] = -1
    ref = oracle.run_case(case)
    assert np.all(ref["residual_contract"] == 0x0000)
    for plan in [(64, 1, 0), (1024, 1, 0), (128, 8, 1)]:
        import reduce_moe_finalize_amd as fb

        say(f"-0 rows plan={plan}")
        t = to_torch(case, DEV)
        with fb.plan_override(*plan):
            normed, resid = call(t, True)
        torch.cuda.synchronize()
        assert np.all(bits(resid) == 0x0000), plan
        assert np.all(bits(normed) == 0x0000), plan


def test_concurrent_streams_with_own_workspaces():
    """Two streams run split-row calls at the same time, each on its own
    workspace: both match the oracle on every round."""
    import reduce_moe_finalize_amd as fb

    cases = [make_case(16, 7168, 8, seed=80 + i, K=8, num_experts=256, shared=True)
             for i in range(2)]
    ts = [to_torch(c, DEV) for c in cases]
    refs = [oracle.run_case(c) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.zeros(fb.workspace_bytes(16, 7168), dtype=torch.uint8, device=DEV) for _ in range(2)]
    outs = [(torch.empty(16, 7168, dtype=torch.bfloat16, device=DEV),
             torch.empty(16, 7168, dtype=torch.bfloat16, device=DEV)) for _ in range(2)]
    torch.cuda.synchronize()
    say("two streams")
    for it in range(20):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                call(ts[i], True, workspace=wss[i], out=outs[i][0], residual_out=outs[i][1])
        torch.cuda.synchronize()
        for i in range(2):
            compare(bits(outs[i][0]), bits(outs[i][1]), refs[i], f"stream {i} round {it}")
    assert fb.workspace_status(wss[0]) == 0 and fb.workspace_status(wss[1]) == 0


def test_random_shapes_auto_plans():
    """Seeded random shapes across every kernel and variant the automatic plan
    can pick: T 1..600, H a multiple of 8 up to 4096, R 0..16, K 0..16, shared
    and gate on or off, weight_bias and gamma family, a few skipped slots; each
    case again under a random forced plan (either kernel, any batch and per-CU
    limit), which must give bit-identical residuals."""
    rng = np.random.Generator(np.random.PCG64(90))
    for it in range(36):
        K = int(rng.choice([0, 0, 1, 2, 6, 8, 8, 10, 12, 16]))
        R = int(rng.integers(1 if K == 0 else 0, 17))
        T = int(rng.choice([1, 3, 16, 31, 64, 100, 129, 255, 256, 300, 513, 600]))
        H = 8 * int(rng.integers(1, 513))
        shared = K > 0 and bool(rng.integers(0, 2))
        gate = shared and bool(rng.integers(0, 2))
        wb = float(rng.choice([0.0, 1.0]))
        case = make_case(T, H, R, seed=1000 + it, K=K, num_experts=max(K, 32), shared=shared,
                         gate=gate, weight_bias=wb,
                         gamma_dist="normal01" if wb else "uniform")
        if K > 0:
            case.idx = case.idx.copy()
            n = case.expert_out.shape[0]
            for _ in range(int(rng.integers(0, 4))):
                case.idx[int(rng.integers(0, T)), int(rng.integers(0, K))] = int(
                    rng.choice([-1, n, -(2**31)]))
        _, n0, r0 = run_and_check(case, f"random it={it}")
        # the same case under a random forced plan gives the same residual bits
        import reduce_moe_finalize_amd as fb

        vpt = int(rng.choice([1, 2, 4, 8]))
        if vpt == 1:
            plan = (64 * int(rng.integers(1, 5)), 1, 0)
        else:
            lanes = -(-(H // 8) // vpt)
            block = max(64, (lanes + 63) // 64 * 64)
            if block > {2: 1024, 4: 512, 8: 256}[vpt]:
                continue
            plan = (block, vpt, int(rng.choice([1, 2, 4, 8])), int(rng.integers(0, 7)))
        t = to_torch(case, DEV)
        try:
            with fb.plan_override(*plan):
                normed, resid = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias)
        except ValueError:
            continue  # the plan does not fit this R/K variant
        torch.cuda.synchronize()
        assert np.array_equal(bits(resid), r0), f"random it={it} plan={plan}"
        compare(bits(normed), bits(resid), oracle.run_case(case), f"random it={it} plan={plan}")


def test_random_shapes_across_plan_boundaries():
    """Seeded random shapes with T on both sides of every plan boundary of the
    small and middle range (16/17, 32/33, 64/65, 128/129, 256/257, 320/321,
    ...), H up to 8192, any R and K: the automatic plan matches the oracle,
    the workspace status stays clear, and two forced balanced plans on the same
    case give the same residual bits and match the oracle too."""
    import reduce_moe_finalize_amd as fb

    rng = np.random.Generator(np.random.PCG64(92))
    tees = [1, 2, 5, 16, 17, 31, 33, 48, 64, 65, 96, 100, 128, 129, 192, 255, 256, 257, 292,
            300, 320, 321, 384, 513, 600, 700]
    for it in range(60):
        K = int(rng.choice([0, 0, 1, 2, 6, 8, 8, 10, 12, 16]))
        R = int(rng.integers(1 if K == 0 else 0, 17))
        T = int(rng.choice(tees))
        H = 8 * int(rng.integers(1, 1025))
        shared = K > 0 and bool(rng.integers(0, 2))
        gate = shared and bool(rng.integers(0, 2))
        wb = float(rng.choice([0.0, 1.0]))
        case = make_case(T, H, R, seed=3000 + it, K=K, num_experts=max(K, 32), shared=shared,
                         gate=gate, weight_bias=wb,
                         gamma_dist="normal01" if wb else "uniform")
        if K > 0:
            case.idx = case.idx.copy()
            n = case.expert_out.shape[0]
            for _ in range(int(rng.integers(0, 4))):
                case.idx[int(rng.integers(0, T)), int(rng.integers(0, K))] = int(
                    rng.choice([-1, n, -(2**31)]))
        what = f"boundary it={it}"
        _, _, r0 = run_and_check(case, what)
        assert fb.default_workspace_status() == 0, what
        t = to_torch(case, DEV)
        ref = oracle.run_case(case)
        for block, upw, wpc in ((512, int(rng.choice([1, 2, 3, 4])), 2),
                                (256, int(rng.choice([1, 2])), 4)):
            try:
                with fb.plan_override(block, 1, 0, wpc, upw):
                    normed, resid = call(t, case.finalize, eps=case.eps,
                                         weight_bias=case.weight_bias)
            except ValueError:
                continue  # does not fit these sizes or this variant
            torch.cuda.synchronize()
            assert np.array_equal(bits(resid), r0), f"{what} balanced {block},{upw},{wpc}"
            compare(bits(normed), bits(resid), ref, f"{what} balanced {block},{upw},{wpc}")


def test_random_large_shapes_auto_plans():
    """Seeded random large shapes under the automatic plan, over the stream
    kernel's width classes and row counts (about 3 to 20 rows per CU): T
    700..5000, H a multiple of 8 up to 16384 (ragged row tails included), R
    1..16, K 0..16, shared and gate on or off, a few skipped slots; outputs
    checked against the oracle on sampled rows (rows are independent)."""
    rng = np.random.Generator(np.random.PCG64(91))
    for it in range(10):
        K = int(rng.choice([0, 8, 10, 16]))
        R = int(rng.integers(1, 17))
        T = int(rng.integers(700, 5001))
        H = 8 * int(rng.integers(1, 2049))
        shared = K > 0 and bool(rng.integers(0, 2))
        gate = shared and bool(rng.integers(0, 2))
        say(f"random large it={it}: T={T} H={H} R={R} K={K} shared={shared} gate={gate}")
        t = make_case_torch(T, H, R, device=DEV, seed=2000 + it, K=K, num_experts=max(2 * K, 64),
                            shared=shared, gate=gate)
        if K > 0:
            n = t["expert_out"].shape[0]
            for _ in range(3):
                t["idx"][int(rng.integers(0, T)), int(rng.integers(0, K))] = int(
                    rng.choice([-1, n, -(2**31)]))
        normed, resid = call(t, K > 0, eps=t["eps"], weight_bias=t["weight_bias"])
        torch.cuda.synchronize()
        rows = sample_rows(T)
        ref = oracle.run_case(torch_case_to_host(t, rows))
        r = torch.from_numpy(rows).to(DEV)
        compare(bits(normed.index_select(0, r)), bits(resid.index_select(0, r)), ref,
                f"random large it={it} T={T} H={H}")
        del t, normed, resid
        torch.cuda.empty_cache()


def test_non_finite_inputs_propagate_like_ieee_fp32():
    """Inf and NaN inputs follow IEEE fp32 arithmetic: an Inf element makes its
    row's sum of squares infinite (finite outputs of the row normalise to 0,
    the infinite one to NaN); Inf - Inf or a NaN input makes the normed row NaN;
    a skipped slot's row is never read into the sum, even if it holds Inf.
    NaN outputs are compared as NaN (any quiet NaN); everything else bitwise
    for the residual and to the usual tolerance for normed."""
    T, H = 8, 1024
    case = make_case(T, H, 2, seed=33, K=3, num_experts=8, shared=True, gate=True)
    inf, ninf, nan = np.uint16(0x7F80), np.uint16(0xFF80), np.uint16(0x7FC1)
    case.partials = [p.copy() for p in case.partials]
    case.residual = case.residual.copy()
    case.shared = case.shared.copy()
    case.expert_out = case.expert_out.copy()
    case.idx = case.idx.copy()
    case.partials[0][0, 5] = inf                     # row 0: one infinite element
    case.partials[0][1, 7] = inf                     # row 1: Inf - Inf = NaN
    case.partials[1][1, 7] = ninf
    case.residual[2, 3] = nan                        # row 2: a NaN input
    case.expert_out[case.idx[3, 1], 9] = inf         # row 3: Inf in a skipped slot's row
    case.idx[3, 1] = -1
    case.shared[4, 11] = ninf                        # row 4: -Inf through the gated shared term
    with np.errstate(invalid="ignore"):
        ref = oracle.run_case(case)
    for plan in [None, (64, 1, 0), (128, 8, 1)]:
        import reduce_moe_finalize_amd as fb

        say(f"non-finite inputs plan={plan}")
        t = to_torch(case, DEV)
        with (fb.plan_override(*plan) if plan else contextlib.nullcontext()):
            normed, resid = call(t, True)
        torch.cuda.synchronize()
        rb, nb = bits(resid), bits(normed)
        rv, nv = oracle.bf16_to_f64(rb), oracle.bf16_to_f64(nb)
        rref = oracle.bf16_to_f64(ref["residual_contract"])
        nref = oracle.bf16_to_f64(ref["normed"])
        assert np.array_equal(np.isnan(rv), np.isnan(rref)), plan
        ok = ~np.isnan(rref)
        assert np.array_equal(rb[ok], ref["residual_contract"][ok]), plan
        assert np.array_equal(np.isnan(nv), np.isnan(nref)), plan
        fin = ~np.isnan(nref)
        assert np.all(np.abs(nv[fin] - nref[fin]) <= 2e-2 + 1e-2 * np.abs(nref[fin])), plan
        # the expected shapes of the damage
        assert rb[0, 5] == 0x7F80 and np.isnan(nv[0, 5]) and np.all(nv[0, :5] == 0)
        assert np.isnan(rv[1, 7]) and np.all(np.isnan(nv[1]))
        assert np.isnan(rv[2, 3]) and np.all(np.isnan(nv[2]))
        assert np.all(np.isfinite(nv[3])) and np.all(np.isfinite(rv[3]))
        assert rb[4, 11] == 0xFF80 and np.isnan(nv[4, 11])
        assert np.all(np.isfinite(nv[5:]))


def test_extreme_gate_logits():
    """Gate logits across the whole fp32 range, infinities included: the sigmoid
    (fp64, rounded once to fp32) saturates to 0 and 1 without NaN, and every row
    matches the oracle (residual bitwise) in both kernels."""
    import reduce_moe_finalize_amd as fb

    logits = np.array([-np.inf, -1e30, -200.0, -100.0, -88.7, -20.0, -1e-3, -0.0, 1e-3, 20.0,
                       88.7, 200.0, 1e30, np.inf], np.float32)
    T, H = len(logits), 1024
    case = make_case(T, H, 2, seed=34, K=3, num_experts=8, shared=True, gate=True)
    case.gate = logits
    with np.errstate(over="ignore"):
        ref = oracle.run_case(case)
        scale = oracle.shared_scale(logits, T)
    assert scale[0] == 0.0 and scale[7] == 0.5 and scale[-1] == 1.0
    t = to_torch(case, DEV)
    for plan in [None, (64, 1, 0), (128, 1, 2)]:
        say(f"extreme gate logits plan={plan}")
        with (fb.plan_override(*plan) if plan else contextlib.nullcontext()):
            normed, resid = call(t, True)
        torch.cuda.synchronize()
        assert np.all(np.isfinite(oracle.bf16_to_f64(bits(normed)))), plan
        compare(bits(normed), bits(resid), ref, f"extreme gate logits plan={plan}")


# ------------------------------------------------------------- decline and errors
def test_decline_leaves_outputs_untouched():
    import reduce_moe_finalize_amd as fb

    T, H = 4, 12
    x = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    out = torch.full((T, H), 7.0, device=DEV, dtype=torch.bfloat16)
    ro = torch.full((T, H), 7.0, device=DEV, dtype=torch.bfloat16)
    g = torch.ones(H, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(fb.FusedBoundaryDeclined):
        fb.fused_reduce_rmsnorm([x], x, g, out=out, residual_out=ro)
    assert torch.all(out == 7.0) and torch.all(ro == 7.0)
    # misaligned (2-byte offset) views are declined too
    base = torch.zeros(T * 64 + 1, device=DEV, dtype=torch.bfloat16)
    mis = base[1:].view(T, 64)
    out2 = torch.full((T, 64), 7.0, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(fb.FusedBoundaryDeclined):
        fb.fused_reduce_rmsnorm([mis], torch.zeros(T, 64, device=DEV, dtype=torch.bfloat16),
                                torch.ones(64, device=DEV, dtype=torch.bfloat16), out=out2)
    assert torch.all(out2 == 7.0)


def test_invalid_arguments_raise():
    import reduce_moe_finalize_amd as fb

    x = torch.zeros(4, 64, device=DEV, dtype=torch.bfloat16)
    g = torch.ones(64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fb.fused_reduce_rmsnorm([], x, g)
    with pytest.raises(ValueError):
        fb.fused_reduce_rmsnorm([x], x, g, eps=float("nan"))
    with pytest.raises(ValueError):
        fb.fused_reduce_rmsnorm([x], x, g, out=x)  # output aliases an input
    with pytest.raises(ValueError):
        fb.fused_reduce_rmsnorm([x.cpu()], x, g)
    # a strided view of the gate logits has the right shape but not the layout
    idx = torch.zeros(4, 1, device=DEV, dtype=torch.int32)
    w = torch.ones(4, 1, device=DEV, dtype=torch.float32)
    logits = torch.zeros(4, 2, device=DEV, dtype=torch.float32)
    with pytest.raises(ValueError):
        fb.fused_moe_finalize_rmsnorm([x], x, idx, w, x.clone(), g, shared_out=x,
                                      shared_gate_logits=logits[:, 0])
    with pytest.raises(ValueError):
        fb.split_sum([x], x, shared_out=x, shared_gate_logits=logits[:, 0])


# ------------------------------------------------------------- exact invariants
def test_determinism_and_split_vs_whole_row():
    import reduce_moe_finalize_amd as fb

    case = make_case(16, 7168, 8, seed=27, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    say("determinism")
    plan = fb.get_plan(16, 7168, 8, 8, True, fb.workspace_bytes(16, 7168))
    assert plan["split"] > 1, plan
    runs = []
    for _ in range(4):
        n, r = call(t, True)
        runs.append((bits(n), bits(r)))
    for n, r in runs[1:]:
        assert np.array_equal(n, runs[0][0]) and np.array_equal(r, runs[0][1])
    n1, r1 = call(t, True, workspace=None)  # whole-row plan
    torch.cuda.synchronize()
    assert np.array_equal(bits(r1), runs[0][1]), "residual depends on the launch plan"
    compare(bits(n1), bits(r1), oracle.run_case(case), "whole row")


def test_expert_row_permutation_invariance():
    case = make_case(24, 2048, 2, seed=28, K=8, num_experts=64, shared=True, gate=True)
    _, n0, r0 = run_and_check(case, "perm base")
    N = case.expert_out.shape[0]
    perm = np.random.Generator(np.random.PCG64(5)).permutation(N)
    inv = np.empty(N, np.int64)
    inv[perm] = np.arange(N)
    case.expert_out = case.expert_out[perm]
    case.idx = inv[case.idx].astype(np.int32)
    _, n1, r1 = run_and_check(case, "perm")
    assert np.array_equal(n0, n1) and np.array_equal(r0, r1)


def test_k1_unit_weight_equals_extra_partial():
    case = make_case(10, 4096, 3, seed=29, K=1, num_experts=16)
    case.weights = np.ones_like(case.weights)
    _, n0, r0 = run_and_check(case, "K=1 w=1")
    rows = case.expert_out[case.idx[:, 0]]
    red = make_case(10, 4096, 3, seed=29)
    red.partials = case.partials + [rows]
    red.residual, red.gamma = case.residual, case.gamma
    _, n1, r1 = run_and_check(red, "extra partial")
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)


def test_gate_zero_equals_half_shared():
    case = make_case(8, 2048, 2, seed=30, shared=True, K=2, num_experts=8)
    case.gate = np.zeros(8, np.float32)
    _, n0, r0 = run_and_check(case, "gate 0")
    b = case.shared.astype(np.int32)
    e = (b >> 7) & 0xFF
    case.shared = np.where(e > 1, b - (1 << 7), b).astype(np.uint16)  # exact halving
    case.gate = None
    _, n1, r1 = run_and_check(case, "S/2 ungated")
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)


def test_power_of_two_scaling_of_residual():
    case = make_case(6, 7168, 4, seed=31)
    _, _, r0 = run_and_check(case, "scale base")

    def scale(b, k):
        b = b.astype(np.int32)
        e = (b >> 7) & 0xFF
        return np.where(e != 0, b + (k << 7), b).astype(np.uint16)

    case.partials = [scale(p, 2) for p in case.partials]
    case.residual = scale(case.residual, 2)
    _, _, r1 = run_and_check(case, "scaled x4")
    assert np.array_equal(r1, scale(r0, 2))


# ------------------------------------------------------------- graph capture
@pytest.mark.parametrize("T,plan", [(16, None), (64, (256, 4, 1, 3))],
                         ids=["latency-split", "stream-per-CU-cap"])
def test_hip_graph_replay_with_changing_inputs(T, plan):
    """Capture one call, replay it on new inputs: the split-row protocol (T=16)
    and the stream kernel launched with the LDS reservation that caps the
    workgroups per CU (forced at T=64) both replay correctly."""
    import reduce_moe_finalize_amd as fb

    H = 7168
    case = make_case(T, H, 8, seed=32, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
    normed = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    resid = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    say(f"graph capture T={T} plan={plan}")
    g = torch.cuda.CUDAGraph()
    with (fb.plan_override(*plan) if plan else contextlib.nullcontext()):
        call(t, True, workspace=ws, out=normed, residual_out=resid)  # warm up outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call(t, True, workspace=ws, out=normed, residual_out=resid)
    for it in range(4):
        new = make_case(T, H, 8, seed=100 + it, K=8, num_experts=256, shared=True)
        nt = to_torch(new, DEV)
        for dst, src in zip(t["partials"], nt["partials"]):
            dst.copy_(src)
        for k in ("residual", "gamma", "expert_out", "idx", "weights", "shared"):
            t[k].copy_(nt[k])
        g.replay()
        torch.cuda.synchronize()
        compare(bits(normed), bits(resid), oracle.run_case(new), f"replay {it}")
        # eager on the same inputs agrees bitwise (same plan, same workspace protocol)
        with (fb.plan_override(*plan) if plan else contextlib.nullcontext()):
            en, er = call(t, True, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(en), bits(normed)) and np.array_equal(bits(er), bits(resid))
    assert fb.workspace_status(ws) == 0


@pytest.mark.parametrize("T,plan", [(16, None), (300, None), (16, (128, 1, 0))],
                         ids=["T16-auto", "T300-balanced", "T16-128lanes"])
def test_hip_graph_replay_in_place(T, plan):
    """A captured call that updates the residual in place (split rows store it
    only after their exchange), replayed on fresh inputs several times with
    eager calls on the same workspace in between: every replay matches the
    oracle, and the slots keep one epoch per row."""
    import reduce_moe_finalize_amd as fb

    H = 7168
    case = make_case(T, H, 8, seed=33, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
    normed = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    say(f"graph capture in place T={T} plan={plan}")
    g = torch.cuda.CUDAGraph()
    with (fb.plan_override(*plan) if plan else contextlib.nullcontext()):
        call(t, True, workspace=ws, out=normed, residual_out=t["residual"])  # warm up
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call(t, True, workspace=ws, out=normed, residual_out=t["residual"])
    for it in range(4):
        new = make_case(T, H, 8, seed=200 + it, K=8, num_experts=256, shared=True)
        nt = to_torch(new, DEV)
        for dst, src in zip(t["partials"], nt["partials"]):
            dst.copy_(src)
        for k in ("residual", "gamma", "expert_out", "idx", "weights", "shared"):
            t[k].copy_(nt[k])
        g.replay()
        torch.cuda.synchronize()
        compare(bits(normed), bits(t["residual"]), oracle.run_case(new), f"in-place replay {it}")
        # an eager in-place call on the same workspace between replays
        t["residual"].copy_(nt["residual"])
        with (fb.plan_override(*plan) if plan else contextlib.nullcontext()):
            en, er = call(t, True, workspace=ws, residual_out=t["residual"])
        torch.cuda.synchronize()
        compare(bits(en), bits(er), oracle.run_case(new), f"eager in place after replay {it}")
        ep = _slot_epochs(ws)[:T]
        assert np.all(ep == ep[:, :1]), "slots of a row disagree"
    assert fb.workspace_status(ws) == 0


def test_graph_keeps_a_cached_workspace_after_the_cache_grows():
    """A graph captured with the stream's cached workspace, taken before capture
    and passed explicitly, keeps writing to that buffer on every replay.  When
    a later, larger call on the same stream grows the cache, the old buffer must
    stay allocated: memory handed to a new tensor instead would be overwritten
    by each replay."""
    import reduce_moe_finalize_amd as fb

    T, H = 16, 7168
    case = make_case(T, H, 8, seed=33, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    normed = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    resid = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream(device=DEV)
    say("graph on a cached workspace, then the cache grows")
    with torch.cuda.stream(s):
        ws = fb.default_workspace(T, H)
        call(t, True, workspace=ws, out=normed, residual_out=resid)  # warm up
    s.synchronize()
    old_bytes = ws.numel()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(t, True, workspace=ws, out=normed, residual_out=resid)
    del ws
    # a larger call on the same stream grows the cached workspace (narrow rows keep it cheap)
    big_T = old_bytes // 512 + 1
    big = make_case(big_T, 64, 1, seed=34)
    bt = to_torch(big, DEV)
    with torch.cuda.stream(s):
        bn, br = call(bt, False)
        victim = torch.full((old_bytes,), 0x5A, dtype=torch.uint8, device=DEV)
    s.synchronize()
    compare(bits(bn), bits(br), oracle.run_case(big), "growing call")
    assert fb._workspaces[(DEV.index, s.cuda_stream)].numel() >= fb.workspace_bytes(big_T, 64)
    for it in range(4):
        new = make_case(T, H, 8, seed=200 + it, K=8, num_experts=256, shared=True)
        nt = to_torch(new, DEV)
        for dst, src in zip(t["partials"], nt["partials"]):
            dst.copy_(src)
        for k in ("residual", "gamma", "expert_out", "idx", "weights", "shared"):
            t[k].copy_(nt[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(bits(normed), bits(resid), oracle.run_case(new), f"replay {it}")
        assert bool((victim == 0x5A).all()), f"replay {it} wrote into a tensor allocated later"


def test_graph_capture_with_default_workspace_runs_whole_rows():
    """A default-argument call (workspace="auto") captured with torch.cuda.graph
    (torch's shared capture stream) takes no cached workspace: the graph holds
    the one boundary kernel and nothing else, no cache entry appears for the
    capture stream, and replays on changing inputs match the oracle."""
    import reduce_moe_finalize_amd as fb

    T, H = 16, 7168
    case = make_case(T, H, 8, seed=35, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    normed = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    resid = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    say("graph capture with workspace='auto'")
    call(t, True, out=normed, residual_out=resid)  # eager warm-up on the current stream
    torch.cuda.synchronize()
    keys_before = set(fb._workspaces)
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g):
        call(t, True, out=normed, residual_out=resid)
    assert set(fb._workspaces) == keys_before, "capture created or grew a cached workspace"
    from test_gpu_contract import graph_kernel_nodes
    assert graph_kernel_nodes(g) == 1
    g.instantiate()
    for it in range(3):
        new = make_case(T, H, 8, seed=210 + it, K=8, num_experts=256, shared=True)
        nt = to_torch(new, DEV)
        for dst, src in zip(t["partials"], nt["partials"]):
            dst.copy_(src)
        for k in ("residual", "gamma", "expert_out", "idx", "weights", "shared"):
            t[k].copy_(nt[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(bits(normed), bits(resid), oracle.run_case(new), f"replay {it}")


# ------------------------------------------------------------- split-row protocol
def test_split_protocol_stress_mixed_shapes_one_workspace():
    """Interleave calls of different T, H and splits on one workspace: stale slots
    from earlier calls must never be taken for the current call's."""
    import reduce_moe_finalize_amd as fb

    ws = torch.zeros(fb.workspace_bytes(64, 8192), dtype=torch.uint8, device=DEV)
    rng = np.random.Generator(np.random.PCG64(60))
    cases = {}
    for T, H in [(1, 7168), (5, 7168), (16, 7168), (64, 7168), (16, 6144), (7, 8192)]:
        c = make_case(T, H, 4, seed=T * 7 + H, K=4, num_experts=16, shared=True)
        cases[(T, H)] = (c, to_torch(c, DEV), oracle.run_case(c))
    plans = [(64, 1, 0), (128, 1, 0), (192, 1, 0), (256, 1, 0), (448, 1, 0)]
    say("split protocol stress")
    for it in range(60):
        key = list(cases)[rng.integers(len(cases))]
        c, t, ref = cases[key]
        block = plans[rng.integers(len(plans))]
        with fb.plan_override(*block):
            normed, resid = call(t, True, workspace=ws)
        torch.cuda.synchronize()
        compare(bits(normed), bits(resid), ref, f"stress it={it} T,H={key} plan={block}")
    assert fb.workspace_status(ws) == 0


def _row_records(ws: torch.Tensor) -> np.ndarray:
    """The workspace's per-row records as uint64 [rows, 64] (256-byte header, then
    512 bytes per row of 64-bit slots {epoch << 32 | value}; slots 0..31 in use)."""
    words = ws.cpu().numpy().view(np.uint64)
    return words[256 // 8:].reshape(-1, 64)


def _slot_epochs(ws: torch.Tensor) -> np.ndarray:
    """The 32-bit epochs of slots 0..31 of every row record, uint64 [rows, 32]."""
    return _row_records(ws)[:, :32] >> np.uint64(32)


def test_split_slots_end_at_row_epoch_and_epoch_wraps():
    """After every split call each of the 32 slots of a row it touched carries the
    row's next epoch (slots the call left unused included), so whichever slot a
    later call's workgroup reads its epoch from, all agree, and no slot can
    match a later call's epoch before that call publishes; rows it did not touch
    are left alone; and the 32-bit epoch wraps (0xFFFFFFFF -> 0) with correct
    results."""
    import reduce_moe_finalize_amd as fb

    H = 7168
    ws = torch.zeros(fb.workspace_bytes(64, H), dtype=torch.uint8, device=DEV)
    cases = {}
    for T in (16, 48):
        c = make_case(T, H, 8, seed=70 + T, K=8, num_experts=256, shared=True)
        cases[T] = (to_torch(c, DEV), oracle.run_case(c))
    say("split slots end at the next epoch")
    for T, plan in [(16, None), (48, (256, 1, 0)), (16, (448, 1, 0)), (48, (128, 1, 0)),
                    (16, (64, 1, 0))]:
        t, ref = cases[T]
        before = _row_records(ws)
        ctx = fb.plan_override(*plan) if plan else contextlib.nullcontext()
        with ctx:
            split = fb.get_plan(T, H, 8, 8, True, ws.numel())["split"]
            normed, resid = call(t, True, workspace=ws)
        torch.cuda.synchronize()
        assert split > 1, (T, plan)
        compare(bits(normed), bits(resid), ref, f"T={T} plan={plan}")
        rec = _row_records(ws)
        ep_before = before[:T, :32] >> np.uint64(32)
        assert np.all(ep_before == ep_before[:, :1]), "slots of a row disagreed before the call"
        ep = rec[:T, :32] >> np.uint64(32)
        assert np.all(ep == ep_before[:, :1] + 1), (T, plan, split)
        assert np.array_equal(rec[T:], before[T:]), "a row the call did not touch changed"
    # every touched row at the last epoch before the wrap
    T = 16
    t, ref = cases[T]
    words = ws.view(torch.int64)
    rows = words[256 // 8:].view(-1, 64)
    rows[:T, :32] = -(1 << 32)  # epoch 0xFFFFFFFF in the high half, value 0
    say("split epoch wrap")
    normed, resid = call(t, True, workspace=ws)
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), ref, "epoch wrap")
    assert np.all(_slot_epochs(ws)[:T] == 0)
    assert fb.workspace_status(ws) == 0


def test_auto_workspace_timeout_is_reported_and_reset():
    """The cached "auto" workspaces: a forced time-out (every split row gives up
    without polling) leaves the outputs exactly as a normal call's, shows in
    their status, and reset_default_workspaces() clears it."""
    import reduce_moe_finalize_amd as fb

    T, H = 32, 7168
    case = make_case(T, H, 8, seed=62, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    say("auto workspace time-out and reset")
    fb.reset_default_workspaces()
    with fb.plan_override(64, 1, 0):
        n0, r0 = call(t, True)
    torch.cuda.synchronize()
    with fb.wait_limit(fb.WAIT_NO_POLL), fb.plan_override(64, 1, 0):
        n1, r1 = call(t, True)
    torch.cuda.synchronize()
    assert fb.default_workspace_status() & 1
    assert np.array_equal(bits(n1), bits(n0)) and np.array_equal(bits(r1), bits(r0))
    compare(bits(n1), bits(r1), ref, "timed out")
    fb.reset_default_workspaces()
    torch.cuda.synchronize()
    assert fb.default_workspace_status() == 0
    with fb.plan_override(64, 1, 0):
        normed, resid = call(t, True)
    torch.cuda.synchronize()
    compare(bits(normed), bits(resid), ref, "after reset")
    assert fb.default_workspace_status() == 0


@pytest.mark.parametrize("finalize", [True, False], ids=["finalize", "reduce"])
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_split_wait_timeout_recomputes_exactly(finalize, in_place):
    """Every split row gives up without polling (host-set limit): each workgroup
    takes its siblings' published parts or recomputes them, so both outputs are
    bit-identical to a normal call with the same plan, also with the residual
    updated in place (a sibling overwrites it only once its part is visible);
    the status word is set.  The slots still end the call at the next epoch,
    so the next call on the same workspace exchanges normally; a poll limit of
    one (rows may or may not give up) is exact too; zero-filling clears the
    status."""
    import reduce_moe_finalize_amd as fb

    T, H = 64, 7168
    kw = dict(K=8, num_experts=256, shared=True) if finalize else {}
    case = make_case(T, H, 8, seed=61, **kw)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
    plan = (64, 1, 0)
    resid0 = t["residual"].clone()

    def run(**hooks):
        ro = None
        if in_place:
            t["residual"].copy_(resid0)
            ro = t["residual"]
        with contextlib.ExitStack() as st:
            if "limit" in hooks:
                st.enter_context(fb.wait_limit(hooks["limit"]))
            st.enter_context(fb.plan_override(*plan))
            n, r = call(t, finalize, workspace=hooks.get("ws", ws), residual_out=ro)
        torch.cuda.synchronize()
        return bits(n), bits(r)

    say(f"forced wait time-out, finalize={finalize}, in_place={in_place}")
    n0, r0 = run(ws=torch.zeros_like(ws))
    compare(n0, r0, ref, "normal")
    n1, r1 = run(limit=fb.WAIT_NO_POLL)
    assert np.array_equal(n1, n0) and np.array_equal(r1, r0)
    assert fb.workspace_status(ws) == 1
    assert np.all(_slot_epochs(ws)[:T] == 1), "slots not at the next epoch"
    # the next call exchanges through the slots again (they carry its epoch)
    n2, r2 = run()
    assert np.array_equal(n2, n0) and np.array_equal(r2, r0)
    assert np.all(_slot_epochs(ws)[:T] == 2)
    assert fb.workspace_status(ws) == 1
    # a poll limit of one: rows may or may not give up; the outputs are exact either way
    n3, r3 = run(limit=1)
    assert np.array_equal(n3, n0) and np.array_equal(r3, r0)
    ws.zero_()
    n4, r4 = run()
    compare(n4, r4, ref, "after re-zeroing")
    assert fb.workspace_status(ws) == 0
    assert np.all(_slot_epochs(ws)[:T] == 1)
    if in_place:
        t["residual"].copy_(resid0)


@pytest.mark.parametrize("shape", [
    # T, H, R, K, shared, gate, plan block
    (48, 8192, 8, 10, True, True, 256),    # the K <= 12 variant
    (24, 4096, 16, 16, True, False, 128),  # the general variant (any R and K)
    (40, 6144, 12, 0, False, False, 64),   # no experts, R > 8
], ids=lambda s: "T{}-H{}-R{}-K{}".format(*s[:4]))
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_split_wait_timeout_every_latency_variant(shape, in_place):
    """The forced give-up on the other builds of the latency kernel: outputs
    bit-identical to a normal call with the same plan, in place too, and the
    slots at the next epoch."""
    import reduce_moe_finalize_amd as fb

    T, H, R, K, sh, gt, block = shape
    kw = dict(K=K, num_experts=max(32, K), shared=sh, gate=gt) if K else {}
    case = make_case(T, H, R, seed=T + H + R, weight_bias=1.0 if gt else 0.0,
                     gamma_dist="normal01" if gt else "uniform", **kw)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    resid0 = t["residual"].clone()

    def run(ws, limit=None):
        ro = None
        if in_place:
            t["residual"].copy_(resid0)
            ro = t["residual"]
        with contextlib.ExitStack() as st:
            if limit is not None:
                st.enter_context(fb.wait_limit(limit))
            st.enter_context(fb.plan_override(block, 1, 0))
            n, r = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias, workspace=ws,
                        residual_out=ro)
        torch.cuda.synchronize()
        return bits(n), bits(r)

    say(f"latency variant time-out {shape} in_place={in_place}")
    n0, r0 = run(torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV))
    compare(n0, r0, ref, f"{shape} normal")
    ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
    n1, r1 = run(ws, fb.WAIT_NO_POLL)
    assert np.array_equal(n1, n0) and np.array_equal(r1, r0)
    assert fb.workspace_status(ws) == 1
    assert np.all(_slot_epochs(ws)[:T] == 1)
    n2, r2 = run(ws, 1)
    assert np.array_equal(n2, n0) and np.array_equal(r2, r0)
    assert np.all(_slot_epochs(ws)[:T] == 2)
    if in_place:
        t["residual"].copy_(resid0)


@pytest.mark.parametrize("shape", [
    # T, H, R, K, shared, gate, plan (block, upw, wpc)
    (97, 1000, 3, 5, True, True, (256, 2, 3)),   # ragged rows: last unit 61 lanes
    (40, 2056, 16, 16, True, False, (128, 6, 4)),  # the general variant
    (257, 7168, 8, 0, False, False, (1024, 2, 1)),  # no experts
    # the streamed form (plan: block, upw, wpc, sources per batch)
    (97, 1000, 3, 5, True, True, (256, 1, 6, 2)),
    (40, 2056, 16, 16, True, False, (128, 1, 8, 2)),
    (300, 7168, 8, 0, False, False, (768, 1, 2, 2)),
], ids=lambda s: "T{}-H{}-R{}-K{}{}".format(*s[:4], "-streamed" if len(s[6]) > 3 else ""))
def test_balanced_timeout_other_shapes_in_place(shape):
    """The balanced kernel's forced give-up on ragged, general-variant and
    expert-free shapes with the residual updated in place: bit-identical to a
    normal call with a separate residual_out."""
    import reduce_moe_finalize_amd as fb

    T, H, R, K, sh, gt, plan = shape
    block, upw, wpc = plan[:3]
    spb = plan[3] if len(plan) > 3 else 0
    kw = dict(K=K, num_experts=max(16, K), shared=sh, gate=gt) if K else {}
    case = make_case(T, H, R, seed=T + H, weight_bias=0.5 if gt else 0.0, **kw)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    if _balanced_plan(fb, case, plan) is None:
        pytest.skip("plan does not fit these sizes")
    say(f"balanced time-out {shape}")
    with fb.plan_override(block, 1, spb, wpc, upw):
        n0, r0 = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias,
                      workspace=torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        n0, r0 = bits(n0), bits(r0)
        compare(n0, r0, ref, f"{shape} normal")
        ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
        resid0 = t["residual"].clone()
        with fb.wait_limit(fb.WAIT_NO_POLL):
            n1, r1 = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias, workspace=ws,
                          residual_out=t["residual"])
        torch.cuda.synchronize()
    assert np.array_equal(bits(n1), n0) and np.array_equal(bits(r1), r0)
    assert fb.workspace_status(ws) == 1
    t["residual"].copy_(resid0)


# ------------------------------------------------------------- balanced kernel
BALANCED_PLANS = [  # (block, units_per_wave, workgroups_per_cu[, sources_per_batch])
    (1024, 1, 1), (1024, 2, 1), (768, 3, 1), (512, 4, 2), (256, 2, 3), (512, 8, 1), (128, 6, 4),
    (64, 4, 8), (512, 1, 2),
    # the streamed form: one unit per wave, sources two at a time
    (768, 1, 2, 2), (512, 1, 3, 2), (256, 1, 6, 2), (64, 1, 16, 2)]


def _override(fb, plan):
    block, upw, wpc = plan[:3]
    return fb.plan_override(block, 1, plan[3] if len(plan) > 3 else 0, wpc, upw)


def _balanced_plan(fb, case, plan):
    """The completed plan, or None if it does not fit these sizes."""
    try:
        with _override(fb, plan):
            return fb.get_plan(case.T, case.H, case.R, case.K if case.finalize else 0,
                               case.shared is not None, fb.workspace_bytes(case.T, case.H))
    except ValueError:
        return None


BALANCED_CASES = [
    # T, H, R, K, shared, gate
    (300, 7168, 8, 8, True, False),
    (257, 7168, 8, 0, False, False),
    (97, 1000, 3, 5, True, True),     # ragged row: 125 vectors, last unit 61 lanes
    (700, 512, 2, 0, False, False),   # one unit per row
    (64, 8192, 8, 10, True, True),
    (40, 2056, 16, 16, True, False),  # the general variant, 5 units per row (last 1 lane)
    (333, 24, 1, 2, False, False),    # 3 vectors per row
    (512, 7168, 8, 8, True, False),   # whole rows per workgroup: nothing shared
    (300, 7168, 0, 8, True, True),    # no partials, gated shared expert
]


@pytest.mark.parametrize("shape", BALANCED_CASES, ids=lambda s: "T{}-H{}-R{}-K{}".format(*s[:4]))
def test_balanced_kernel_plans_match_oracle(shape):
    """The balanced kernel under forced plans (lanes per workgroup, units per
    wave, workgroups per CU): each matches the oracle; the residual is the same
    fp32 sum under every plan; a plan repeated on the same workspace gives the
    same bits."""
    import reduce_moe_finalize_amd as fb

    T, H, R, K, sh, gt = shape
    kw = dict(K=K, num_experts=max(16, K), shared=sh, gate=gt) if K else {}
    case = make_case(T, H, R, seed=T + H, weight_bias=0.5 if gt else 0.0, **kw)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    resid0 = None
    ran = 0
    for plan in BALANCED_PLANS:
        full = _balanced_plan(fb, case, plan)
        if full is None:
            continue
        ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
        say(f"balanced {shape} plan={full}")
        with _override(fb, plan):
            normed, resid = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias,
                                 workspace=ws)
            torch.cuda.synchronize()
            compare(bits(normed), bits(resid), ref, f"balanced {shape} {full}")
            n2, r2 = call(t, case.finalize, eps=case.eps, weight_bias=case.weight_bias,
                          workspace=ws)
            torch.cuda.synchronize()
        assert np.array_equal(bits(n2), bits(normed)) and np.array_equal(bits(r2), bits(resid))
        if resid0 is None:
            resid0 = bits(resid)
        assert np.array_equal(bits(resid), resid0), full
        assert fb.workspace_status(ws) == 0
        ran += 1
    assert ran >= 2, shape


@pytest.mark.parametrize("plan", [(1024, 1, 0, 1, 2), (768, 1, 2, 2, 1)], ids=["allin", "streamed"])
@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
def test_balanced_kernel_timeout_recomputes_exactly(in_place, plan):
    """Every shared row gives up without polling: the polling wave takes the
    other workgroups' published parts or recomputes them, so the outputs are
    bit-identical to a normal call, also with the residual updated in place;
    the status word is set and every shared row's slots still end the call at
    the next epoch."""
    import reduce_moe_finalize_amd as fb

    T, H = 300, 7168
    case = make_case(T, H, 8, seed=90, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    ref = oracle.run_case(case)
    resid0 = t["residual"].clone()

    def run(ws, limit=None):
        ro = None
        if in_place:
            t["residual"].copy_(resid0)
            ro = t["residual"]
        with contextlib.ExitStack() as st:
            if limit is not None:
                st.enter_context(fb.wait_limit(limit))
            st.enter_context(fb.plan_override(*plan))
            n, r = call(t, True, workspace=ws, residual_out=ro)
        torch.cuda.synchronize()
        return bits(n), bits(r)

    say(f"balanced forced time-out, plan={plan} in_place={in_place}")
    n0, r0 = run(torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV))
    compare(n0, r0, ref, "balanced normal")
    ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=DEV)
    n1, r1 = run(ws, fb.WAIT_NO_POLL)
    assert np.array_equal(n1, n0) and np.array_equal(r1, r0)
    assert fb.workspace_status(ws) == 1
    ep = _slot_epochs(ws)[:T]
    shared_rows = ep[:, 0] != 0
    assert shared_rows.sum() > T // 2, shared_rows.sum()  # most rows at 1.17 per CU
    assert np.all(ep[shared_rows] == 1) and np.all(ep[~shared_rows] == 0)
    n2, r2 = run(ws)
    assert np.array_equal(n2, n0) and np.array_equal(r2, r0)
    assert np.all(_slot_epochs(ws)[:T][shared_rows] == 2)
    if in_place:
        t["residual"].copy_(resid0)


def test_balanced_and_latency_share_one_workspace():
    """Calls alternating between the balanced kernel (slots per workgroup part)
    and split latency rows (slots per workgroup) on one workspace stay exact:
    the stamp of unused slots keeps every slot of a touched row at one epoch."""
    import reduce_moe_finalize_amd as fb

    H = 7168
    ws = torch.zeros(fb.workspace_bytes(320, H), dtype=torch.uint8, device=DEV)
    cases = {}
    for T in (16, 300):
        c = make_case(T, H, 8, seed=91 + T, K=8, num_experts=256, shared=True)
        cases[T] = (to_torch(c, DEV), oracle.run_case(c))
    plans = {16: [(128, 1, 0, 0, 0), (448, 1, 0, 0, 0), (64, 1, 0, 4, 1)],
             300: [(1024, 1, 0, 1, 2), (512, 1, 0, 2, 2), (256, 1, 0, 3, 2), (768, 1, 2, 2, 1)]}
    say("balanced and latency on one workspace")
    for it in range(16):
        T = (16, 300)[it % 2]
        plan = plans[T][(it // 2) % len(plans[T])]
        t, ref = cases[T]
        with fb.plan_override(*plan):
            normed, resid = call(t, True, workspace=ws)
        torch.cuda.synchronize()
        compare(bits(normed), bits(resid), ref, f"it={it} T={T} plan={plan}")
    assert fb.workspace_status(ws) == 0
