"""Launch counts and the benchmark's output contract (needs a GPU).

* One kernel per fused call, two for the split flow: the call is captured in a
  HIP graph and its kernel nodes are counted (the pages count one fused call
  where the split flow had two: PR #37104, Correctness; PR #42020, Test plan).
* ``bench.py`` prints one JSON line with the fields the harness reads.
"""
import ctypes
import json
import os
import subprocess
import sys

import pytest
import torch

from gpu_helpers import say
from workloads import make_case, to_torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(DEV)
    yield
    torch.cuda.synchronize()


def _hip_runtime():
    """The HIP runtime this process already uses (torch's), by its mapped path."""
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert paths, "HIP runtime not loaded"
    lib = ctypes.CDLL(sorted(paths)[0])
    lib.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    lib.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    return lib


def kernel_nodes(fn):
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g):
        fn()
    n = graph_kernel_nodes(g)
    del g
    return n


def graph_kernel_nodes(g):
    """Kernel nodes of a torch CUDAGraph captured with keep_graph=True."""
    hip = _hip_runtime()
    graph = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    kinds = []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        kinds.append(t.value)
    return sum(1 for k in kinds if k == 0)  # hipGraphNodeTypeKernel


@pytest.mark.parametrize("T", [16, 2048])
def test_one_kernel_per_fused_call_two_for_split(T):
    import reduce_moe_finalize_amd as fb

    case = make_case(T, 7168, 8, seed=50, K=8, num_experts=256, shared=True)
    t = to_torch(case, DEV)
    ws = torch.zeros(fb.workspace_bytes(T, 7168), dtype=torch.uint8, device=DEV)
    out = torch.empty(T, 7168, dtype=torch.bfloat16, device=DEV)
    ro = torch.empty_like(out)
    y = torch.empty_like(out)
    say(f"launch count T={T}")

    def fused():
        fb.fused_moe_finalize_rmsnorm(t["partials"], t["expert_out"], t["idx"], t["weights"],
                                      t["residual"], t["gamma"], shared_out=t["shared"],
                                      workspace=ws, out=out, residual_out=ro)

    def fused_reduce():
        fb.fused_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], workspace=ws, out=out,
                                residual_out=ro)

    def split():
        fb.split_moe_finalize_rmsnorm(t["partials"], t["expert_out"], t["idx"], t["weights"],
                                      t["residual"], t["gamma"], shared_out=t["shared"], out=out,
                                      residual_out=ro, sum_out=y)

    assert kernel_nodes(fused) == 1
    assert kernel_nodes(fused_reduce) == 1
    assert kernel_nodes(split) == 2


def test_bench_json_contract():
    say("bench.py contract")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--no-sweep", "--cpu-seconds", "1",
           "--steps", "3", "--warmup", "1", "--T", "256"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip().startswith("{")]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["unit"] == "GB/s" and d["checked_vs_oracle"] is True
    assert "workload" in d["config"]
    p10, p50, p90 = d["us_per_call_p10_p50_p90"]
    assert 0 < p10 <= p50 <= p90
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and 0 < r["frac"] < 1
    assert abs(r["achieved"] - d["value"]) < 1e-6
    assert r["attainable_loads_GBps"] > 0 and r["attainable_loads_stores_GBps"] > 0
    assert r["frac_of_attainable"] > 0
    # the oracle baseline only runs on the headline workload
    assert d["cpu_baseline"] is None
    # one vector per lane (up to 2 rows per CU): the probe beside it widens its rows
    res3 = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--no-sweep",
                           "--cpu-seconds", "0", "--steps", "2", "--warmup", "1", "--T", "512"],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res3.returncode == 0, res3.stderr[-2000:]
    d3 = json.loads([ln for ln in res3.stdout.splitlines() if ln.strip().startswith("{")][0])
    assert d3["config"]["plan"]["vec_per_thread"] == 1
    assert d3["roofline"]["attainable_loads_stores_GBps"] > 0
    res2 = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res2.returncode != 0 and "one GPU" in res2.stderr


def test_planner_residency_matches_the_runtime():
    """Every kernel variant and block size the planner may use for a launch
    whose workgroups wait for each other: the workgroups per CU it counts on
    never exceed what the runtime's occupancy query reports on this GPU."""
    import reduce_moe_finalize_amd as fb

    lib = fb._lib
    lib.fused_boundary_resident_workgroups.argtypes = [ctypes.c_int32] * 5 + [
        ctypes.POINTER(ctypes.c_int32)] * 2
    checked = 0
    for R, K in ((8, 0), (16, 0), (8, 8), (8, 12), (16, 16)):
        # (units per wave, sources per batch): the latency kernel, the balanced
        # kernel's builds, and its streamed form
        for upw, spb in [(u, 0) for u in (0, 1, 2, 3, 4, 6, 8)] + [(1, 2)]:
            for block in range(64, 1025, 64):
                planned, device = ctypes.c_int32(), ctypes.c_int32()
                rc = lib.fused_boundary_resident_workgroups(R, K, upw, spb, block,
                                                            ctypes.byref(planned),
                                                            ctypes.byref(device))
                if rc == 1:  # block beyond the latency variant's bound
                    continue
                assert rc == 0, (R, K, upw, spb, block, rc)
                assert planned.value <= device.value, (R, K, upw, spb, block, planned.value,
                                                       device.value)
                checked += 1
    say(f"residency checked for {checked} kernel/block pairs")
    assert checked >= 300


@pytest.mark.parametrize("vpt,wgcu,T,H", [(4, 3, 37, 7168), (2, 0, 5, 6144), (1, 4, 3, 512)])
def test_bandwidth_probe_reads_what_it_claims(vpt, wgcu, T, H):
    """The probe that bench.py times for the attainable rate really loads every
    direct row and every gathered row whose index lies inside the buffer (an
    index outside it is skipped) and writes each output row as the XOR of all
    of them with the output's ordinal: checked against torch's integer XOR."""
    import reduce_moe_finalize_amd as fb

    say(f"bandwidth probe vpt={vpt} wgcu={wgcu} T={T} H={H}")
    g = torch.Generator(device="cpu").manual_seed(T * 7 + H)
    def rnd(*shape):
        return torch.randint(-2**15, 2**15, shape, generator=g, dtype=torch.int16).view(
            torch.bfloat16).to(DEV)
    N, K = 40, 8
    direct = [rnd(T, H) for _ in range(10)]
    gathered = rnd(N, H)
    idx = torch.randint(0, N, (T, K), generator=g, dtype=torch.int32)
    idx[0, 1], idx[-1, 0], idx[T // 2, 3] = -1, N, 2**31 - 1
    idx = idx.to(DEV)
    outs = [torch.empty(T, H, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    fb.bandwidth_probe(direct, gathered, idx, outs, vpt, wgcu)
    torch.cuda.synchronize()
    acc = torch.zeros(T, H // 2, dtype=torch.int32, device=DEV)
    for d in direct:
        acc ^= d.view(torch.int32)
    g32 = gathered.view(torch.int32)
    valid = (idx >= 0) & (idx < N)
    for k in range(K):
        rows = g32[idx[:, k].clamp(0, N - 1).long()]
        acc ^= torch.where(valid[:, k:k + 1], rows, torch.zeros_like(rows))
    for d, o in enumerate(outs):
        assert torch.equal(o.view(torch.int32), acc ^ d), d


@pytest.mark.parametrize("finalize,T", [(True, 300), (False, 16)])
def test_bench_sweep_point(finalize, T):
    """One entry of bench.py's T sweep (the code the default run loops over):
    every timing is positive and ordered, the small-T extras and the probe
    appear where they should."""
    sys.path.insert(0, ROOT)
    import bench
    import reduce_moe_finalize_amd as fb

    say(f"sweep point finalize={finalize} T={T}")
    flush = torch.empty(bench.FLUSH_BYTES, dtype=torch.uint8, device=DEV)
    e = bench.sweep_point(torch, fb, DEV, flush, finalize, T)
    del flush
    assert e["T"] == T and e["us_graph"] > 0 and e["pct_cold"] > 0
    p10, p50, p90 = e["us_cold_kernel"]
    assert 0 < p10 <= p50 <= p90
    assert ("us_busy_kernel" in e) == (T <= 16) and ("us_cold_kernel_no_event" in e) == (T <= 16)
    assert ("us_idle_kernel" in e) == (T <= 16)
    assert ("probe_pct_cold" in e) == (finalize and 256 <= T <= 2048)


def test_bandwidth_probe_checks_its_tensors():
    """Every row tensor the probe touches must be contiguous bf16 [T, H] on
    the same GPU (the kernel takes T and H from the first); the index map
    int32 [T, k]: a mismatch raises before any launch."""
    import reduce_moe_finalize_amd as fb

    T, H = 4, 64
    ok = lambda: torch.zeros(T, H, dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(T, 2, dtype=torch.int32, device=DEV)
    gathered = torch.zeros(8, H, dtype=torch.bfloat16, device=DEV)
    bad = [
        dict(direct=[ok(), torch.zeros(T - 1, H, dtype=torch.bfloat16, device=DEV)]),
        dict(direct=[ok()], outputs=[torch.zeros(T + 1, H, dtype=torch.bfloat16, device=DEV)]),
        dict(direct=[ok(), torch.zeros(T, H, dtype=torch.float32, device=DEV)]),
        dict(direct=[ok(), torch.zeros(H, T, dtype=torch.bfloat16, device=DEV).t()]),
        dict(direct=[ok()], gathered=gathered, gather_idx=idx.to(torch.int64)),
        dict(direct=[ok()], gathered=gathered, gather_idx=idx[:2]),
        dict(direct=[ok()], gathered=gathered[:, :32], gather_idx=idx),
        dict(direct=[ok()], gathered=gathered),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            fb.bandwidth_probe(**kw)
    fb.bandwidth_probe([ok()], gathered, idx, [ok()])  # the well-formed call runs
    torch.cuda.synchronize()


@pytest.mark.parametrize("level,sgprs,waves_per_simd", [(0, 22, 8), (1, 88, 7), (2, 104, 6)])
def test_scalar_registers_limit_residency(level, sgprs, waves_per_simd):
    """What a CU really holds at once, against the rule the planner's residency
    table is checked with (a wave holds its SGPR count plus 16, rounded up to a
    multiple of 16, of 800 per SIMD): one-wave workgroups, 32 per CU asked for,
    fit 4 x that many waves per SIMD; two 16-wave workgroups fit on a CU only
    where 8 waves per SIMD do.  (The runtime's occupancy query counts two
    16-wave workgroups of level 1 as fitting.)"""
    import reduce_moe_finalize_amd as fb
    from test_abi import sgpr_waves_per_simd

    assert sgpr_waves_per_simd(sgprs) == waves_per_simd
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"residency probe level={level}")
    most = fb.residency_probe(level, 32 * cus, 64)
    assert len(most) == cus, len(most)
    assert max(most.values()) == 4 * waves_per_simd, sorted(set(most.values()))
    assert sum(v == 4 * waves_per_simd for v in most.values()) >= 0.9 * cus
    most = fb.residency_probe(level, 2 * cus, 1024)
    assert max(most.values()) == (2 if waves_per_simd == 8 else 1), sorted(set(most.values()))
