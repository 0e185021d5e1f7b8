"""Benchmark of the fused post-experts boundary on one MI355X.

Prints ONE JSON line.  The step is one call of ``fused_moe_finalize_rmsnorm`` on
the headline workload: T=8192 token rows, H=7168, R=8 bf16 partial buffers,
top-8 of 256 experts (expert buffer [T*8, H]), ungated shared expert, residual,
RMSNorm (eps 1e-6).  Inputs are synthetic, drawn on the GPU and resident in HBM
before timing starts.

* value / unit: achieved algorithmic HBM bandwidth (GB/s) of the headline step,
  i.e. algorithmic bytes per call / average call time over --steps back-to-back
  calls timed with HIP events on the launch stream; ``us_per_call_p10_p50_p90``
  repeats the calls one by one between their own events.
* roofline: the same figure against the 8 TB/s HBM peak; ``traffic`` is the
  HBM byte count from rocprofv3 FETCH_SIZE/WRITE_SIZE counters recorded under
  profiles/ (null when the kernel's device code or launch plan changed since
  they were taken).
* sweep: per-call time and GB/s for T = 1 .. 8192 for both entry points (R=8):
  ``us_graph`` is a 100-call HIP graph replay divided by 100 (back-to-back
  kernels, launch overhead amortised; above T=1024 eager back-to-back calls),
  ``us_cold_kernel`` the p10 / median / p90 of the kernel's own duration
  (device timestamps from torch's profiler) when each call follows a 1 GiB
  cache flush (4x the 256 MB MALL) and sits between its own pair of HIP events;
  ``GBps_cold`` and ``pct_cold`` use its median.  At T <= 16 also
  ``us_cold_kernel_no_event`` (the call queued directly behind the flush) and
  ``us_busy_kernel`` (right after a 0.17 ms spin kernel that touches no memory).
  For the finalize at T = 256..2048, ``probe_us_cold_kernel`` / ``probe_pct_cold``
  time fused_boundary_bandwidth_probe (the step's loads and two row stores, whole
  rows, 2 vectors per lane, no arithmetic) the same cold way: what the part
  attains for this traffic at this T.  ``empty_kernel_us_graph`` and ``empty_kernel_us_cold`` are the
  same two measures for a one-element kernel.  ``us_split_graph`` times the
  unfused two-launch flow the fused kernel replaces (bf16 sum materialised,
  then residual RMSNorm) the same way.
* targets (last key of the line): over T = 1..16 for both entry points, the
  worst per-call time in a graph and the worst kernel time (p10 / median /
  p90) cold, right after a busy spin kernel, and queued directly behind the
  flush with no event between (reported; ``met`` counts the first three),
  against 5 us; the lowest cold % of HBM peak over T >= 2048 for both entry
  points and the H=8192 top-10 gated shape, against 70 %.
* roofline.attainable_*: what this part attains for the step's own memory
  traffic, timed in the same run on the same buffers: the boundary's loads
  (10 direct rows and 8 gathered rows per token row, 16-byte nontemporal
  loads, same launch shape) with no arithmetic, alone and with its two row
  stores (fused_boundary_bandwidth_probe); frac_of_attainable is the step's
  figure over the latter.  copy_GBps: torch's device copy over 1 GiB (read +
  written bytes), a generic 1:1 stream, for context.
* configs: per-call time and GB/s of the finalize entry point at points of the
  other workload shapes (H=6144 top-8; H=8192 top-10 with a gated shared expert,
  gamma N(0,0.1), weight_bias 1), each spot-checked against the oracle.
* cpu_baseline: the CPU oracle (NumPy, fp64) on a bounded sample of rows of the
  same workload, on the host's cores.

Algorithmic bytes per call: T*H*2*(R+3) + H*2 (partials, residual in, normed and
residual out, gamma) + T*K*(2H+8) (gathered expert rows, indices, weights)
+ T*H*2 (shared expert) [+ T*4 gate logits].
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call and achieved HBM GB/s (% of peak) vs T at H=7168, R=8"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2**20  # MI355X last-level (Infinity) cache
FLUSH_BYTES = 1 << 30     # cold calls follow a write of 4x the MALL
KERNEL_NAMES = ("latency_kernel", "stream_kernel", "balanced_kernel")
SMALL_T_TARGET_US = 5.0
LARGE_T_TARGET_PCT = 70.0
SRC = os.path.join(ROOT, "reduce_moe_finalize_amd", "csrc", "fused_boundary.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_moe_finalize_T8192_H7168.md")

H, R, K, E = 7168, 8, 8, 256
HEADLINE_T = 8192

# The workload configurations (values not fixed by a configuration follow
# the R=2 token sweep and the DeepSeek-shaped finalize: partials N(0,0.5), residual N(0,1),
# experts and shared N(0,0.3)).
WORKLOADS = {
    # H=7168, R=8, top-8 of 256 + shared expert (the DeepSeek-V3 shape of the sweep)
    "headline": dict(H=7168, R=8, K=8, E=256, gate=False, gamma_dist="uniform", wb=0.0),
    # GLM-5.2 shape: H=6144, top-8 of 256
    "glm_h6144_top8": dict(H=6144, R=8, K=8, E=256, gate=False, gamma_dist="uniform", wb=0.0),
    # Qwen3.5-style large H: H=8192, top-10 of 512, sigmoid-gated shared, gamma N(0,0.1), wb=1
    "gated_h8192_top10": dict(H=8192, R=8, K=10, E=512, gate=True, gamma_dist="normal01", wb=1.0),
}
# (workload, T) points reported in the "configs" section of the JSON line
CONFIG_POINTS = [("headline", 16), ("glm_h6144_top8", 1), ("glm_h6144_top8", 16), ("glm_h6144_top8", 128), ("gated_h8192_top10", 128),
                 ("gated_h8192_top10", 2048), ("gated_h8192_top10", 8192)]
SWEEP_T = (1, 2, 4, 8, 16, 32, 64, 128, 256, 300, 384, 512, 640, 1024, 2048, 4096, 8192)


def algorithmic_bytes(T, H, R, K=0, shared=False, gate=False):
    b = T * H * 2 * (R + 3) + H * 2
    if K:
        b += T * K * (2 * H + 8)
    if shared:
        b += T * H * 2
    if gate:
        b += T * 4
    return b


HOST_SIDE_MARKER = "// ----------------------------------------------------------------- host side"


def source_sha256():
    """Fingerprint of the device code in the kernel source (everything above the
    host-side marker): comments, indentation and blank lines do not count, so
    comment and launcher edits keep recorded counters valid.  The launch shape
    is checked separately against the plan the counters were taken with."""
    with open(SRC) as f:
        text = f.read()
    cut = text.find(HOST_SIDE_MARKER)
    if cut >= 0:
        text = text[:cut]
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).strip() for ln in text.splitlines())
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def read_traffic(plan=None):
    """Per-launch HBM bytes from the committed counter summary, if it was taken
    with this device code and (when given) this launch plan."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m = re.search(r"kernel_code_sha256:\s*([0-9a-f]{64})", text)
    f = re.search(r"fetch_bytes_per_launch:\s*([0-9.eE+]+)", text)
    w = re.search(r"write_bytes_per_launch:\s*([0-9.eE+]+)", text)
    p = re.search(r"plan_block_vec_batch_wgcu:\s*(\d+)\s+(\d+)\s+(\d+)\s+(\d+)", text)
    if not (m and f and w and p) or m.group(1) != source_sha256():
        return None
    if plan is not None and tuple(int(x) for x in p.groups()) != (
            plan["block"], plan["vec_per_thread"], plan["sources_per_batch"],
            plan["workgroups_per_cu"]):
        return None
    return float(f.group(1)) + float(w.group(1))


def make_inputs(T, finalize, device, seed=0, workload="headline"):
    from workloads import make_case_torch

    w = WORKLOADS[workload]
    cfg = dict(K=w["K"], num_experts=w["E"], shared=True, gate=w["gate"]) if finalize else {}
    return make_case_torch(T, w["H"], w["R"], device=device, seed=seed, gamma_dist=w["gamma_dist"],
                           weight_bias=w["wb"], **cfg)


def make_call(fb, t, finalize, workspace, out, resid_out):
    wb = t.get("weight_bias", 0.0)
    if finalize:
        def run():
            return fb.fused_moe_finalize_rmsnorm(
                t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
                shared_out=t["shared"], shared_gate_logits=t.get("gate"), eps=1e-6,
                weight_bias=wb, workspace=workspace, out=out, residual_out=resid_out)
    else:
        def run():
            return fb.fused_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], eps=1e-6,
                                           weight_bias=wb, workspace=workspace, out=out,
                                           residual_out=resid_out)
    return run


def make_split_call(fb, t, finalize, out, resid_out, y):
    """The two-launch split flow on the same inputs (bf16 intermediate ``y``)."""
    if finalize:
        def run():
            return fb.split_moe_finalize_rmsnorm(
                t["partials"], t["expert_out"], t["idx"], t["weights"], t["residual"], t["gamma"],
                shared_out=t["shared"], eps=1e-6, out=out, residual_out=resid_out, sum_out=y)
    else:
        def run():
            return fb.split_reduce_rmsnorm(t["partials"], t["residual"], t["gamma"], eps=1e-6,
                                           out=out, residual_out=resid_out, sum_out=y)
    return run


def time_eager(torch, run, steps, warmup):
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()  # on the current stream, which is the launch stream
    for _ in range(steps):
        run()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / steps  # us per call


def time_graph(torch, run, calls=100, reps=5):
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            run()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1e3 / calls
        best = us if best is None else min(best, us)
    del g
    return best


def time_cold(torch, run, flush, calls=20, reps=3, before=None):
    """Median per-call time with every call preceded by a cache flush.

    Each call is bracketed by a pair of HIP events recorded right after the
    flush kernel, so the figure is the call's GPU time from a cold cache (the
    event packets add a little; rocprofv3's kernel trace is the reference).
    ``before``, if given, replaces the flush as the work queued ahead of each
    call.  ``reps`` is kept for the call signature; the median over ``calls``
    calls is returned."""
    import statistics

    pre = before if before is not None else (lambda: flush.fill_(1))
    run()
    torch.cuda.synchronize()
    n = max(calls, 5)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        pre()
        starts[i].record()
        run()
        ends[i].record()
    torch.cuda.synchronize()
    return statistics.median(s_.elapsed_time(e_) * 1e3 for s_, e_ in zip(starts, ends))


def pcts(v):
    """p10 / median / p90 of a list of times."""
    import statistics

    v = sorted(v)
    q = statistics.quantiles(v, n=10, method="inclusive") if len(v) > 1 else v * 9
    return [round(q[0], 2), round(statistics.median(v), 2), round(q[-1], 2)]


def kernel_times_cold(torch, run, flush, calls=20, names=KERNEL_NAMES, exclude=("Fill",),
                      before=None, events=True):
    """The kernel's own duration (device timestamps from torch's profiler), each
    call right after a write of the whole flush buffer, in microseconds.  With
    ``events`` a HIP event pair brackets each call (flush, event, call, event:
    the cold protocol); without, the call is queued directly behind the flush
    and starts while the flush's writes are still draining.  ``before``, if
    given, is queued ahead of each call instead of the flush."""
    from torch.profiler import ProfilerActivity, profile

    pre = before if before is not None else (lambda: flush.fill_(1))
    run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls if events else 0)]
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for i in range(calls):
            pre()
            if events:
                evs[i][0].record()
            run()
            if events:
                evs[i][1].record()
        torch.cuda.synchronize()
    d = [e.device_time for e in prof.events()
         if any(n in e.name for n in names) and not any(x in e.name for x in exclude)]
    assert len(d) == calls, f"found {len(d)} kernel records for {calls} calls"
    return d


SPIN_CYCLES = 400000  # torch's one-wave spin kernel: ~0.17 ms on MI355X
IDLE_S = 50e-6        # host pause before each call of the idle-GPU measure


def kernel_times_busy(torch, run, calls=20):
    """The kernel's own duration when the GPU is busy right up to the call (a
    spin kernel that touches no memory is queued ahead of it, and outlasts the
    host's next launch), as in a layer where the boundary follows the expert
    GEMMs; in microseconds."""
    return kernel_times_cold(torch, run, None, calls=calls, exclude=("spin",),
                             before=lambda: torch.cuda._sleep(SPIN_CYCLES))


def kernel_times_idle(torch, run, calls=20):
    """The kernel's own duration when the GPU has been idle before the call (the
    host synchronises and pauses about 50 us, then launches); in
    microseconds.  Reported beside the other measures: an idle GPU starts the
    kernel in its low-power state."""
    return kernel_times_cold(torch, run, None, calls=calls, events=False,
                             before=lambda: (torch.cuda.synchronize(), time.sleep(IDLE_S)))


def attainable_copy(torch, dev, nbytes=FLUSH_BYTES, reps=5):
    """GB/s (read + written bytes) of torch's plain device copy over nbytes, best
    of reps: a generic 1:1 read/write stream, for context."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        b.copy_(a)
        e.record()
        e.synchronize()
        ms = s.elapsed_time(e)
        best = ms if best is None else min(best, ms)
    del a, b
    torch.cuda.empty_cache()
    return round(2 * nbytes / best / 1e6, 1)


def probe_shape(plan, H, max_lanes=512):
    """Vectors per lane and workgroups per CU for the bandwidth probe beside a
    step with this plan: the stream kernel's own shape where it streams,
    else 4 vectors per lane with no cap; widened (2, 4, 8 vectors per lane)
    until a row fits the probe's 512 lanes."""
    vpt = plan["vec_per_thread"] if plan["sources_per_batch"] else 4
    wgcu = plan["workgroups_per_cu"] if plan["sources_per_batch"] else 0
    while -(-(H // 8) // vpt) > max_lanes and vpt < 8:
        vpt *= 2
    return vpt, wgcu


def attainable_probe(torch, fb, t, outputs, plan, steps=20, warmup=3):
    """GB/s of the boundary's own memory traffic without its arithmetic
    (fused_boundary_bandwidth_probe on the step's buffers, same vectors per
    lane and per-CU limit, back-to-back calls between events): the loads
    alone, and the loads with the two row stores."""
    direct = list(t["partials"]) + [t["shared"], t["residual"]]
    T, Hh = t["residual"].shape
    k = t["idx"].shape[1]
    vpt, wgcu = probe_shape(plan, Hh)
    load_bytes = T * Hh * 2 * len(direct) + T * k * (2 * Hh + 4)
    res = {}
    for name, outs in (("loads", []), ("loads_stores", list(outputs))):
        def run():
            fb.bandwidth_probe(direct, t["expert_out"], t["idx"], outs, vpt, wgcu)
        us = time_eager(torch, run, steps, warmup)
        res[name] = round((load_bytes + len(outs) * T * Hh * 2) / us / 1e3, 1)
    return res


def per_call_percentiles(torch, run, calls):
    """p10 / median / p90 of single calls, each between its own HIP events, in a
    separate pass after the timed one (so the timed pass carries no extra
    packets).  Each figure includes an event pair's few microseconds."""
    import statistics

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    for i in range(calls):
        starts[i].record()
        run()
        ends[i].record()
    torch.cuda.synchronize()
    v = sorted(a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends))
    q = statistics.quantiles(v, n=10, method="inclusive") if len(v) > 1 else v * 9
    return [round(q[0], 2), round(statistics.median(v), 2), round(q[-1], 2)]


def time_empty_graph(torch, dev, calls=100):
    """Per-launch floor: a graph of tiny one-element kernels."""
    x = torch.zeros(1, device=dev)
    return time_graph(torch, lambda: x.add_(1.0), calls=calls)


def spot_check(torch, t, normed, resid, rows):
    """Compare a few output rows with the CPU oracle (guards the timed numbers)."""
    import numpy as np

    import oracle

    host = rows_to_host(torch, t, rows)
    ref = oracle.run_case(host)
    r = torch.tensor(rows, device=normed.device)
    nb = normed.index_select(0, r).cpu().view(torch.int16).numpy().view(np.uint16)
    rb = resid.index_select(0, r).cpu().view(torch.int16).numpy().view(np.uint16)
    a, b = oracle.bf16_to_f64(nb), oracle.bf16_to_f64(ref["normed"])
    return bool(np.array_equal(rb, ref["residual_contract"])
                and np.all(np.abs(a - b) <= 2e-2 + 1e-2 * np.abs(b)))


def rows_to_host(torch, t, rows):
    import numpy as np
    from types import SimpleNamespace

    dev = t["residual"].device
    r = torch.tensor(rows, device=dev, dtype=torch.int64)

    def hb(x):
        return x.index_select(0, r).cpu().view(torch.int16).numpy().view(np.uint16)

    ns = SimpleNamespace(partials=[hb(p) for p in t["partials"]], residual=hb(t["residual"]),
                         gamma=t["gamma"].cpu().view(torch.int16).numpy().view(np.uint16),
                         weight_bias=t.get("weight_bias", 0.0), eps=1e-6, expert_out=None,
                         idx=None, weights=None, shared=None, gate=None)
    if t.get("idx") is not None:
        idx = t["idx"].index_select(0, r).reshape(-1).to(torch.int64)
        ns.expert_out = t["expert_out"].index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16)
        ns.idx = np.arange(idx.numel(), dtype=np.int32).reshape(len(rows), -1)
        ns.weights = t["weights"].index_select(0, r).cpu().numpy()
    if t.get("shared") is not None:
        ns.shared = hb(t["shared"])
        if t.get("gate") is not None:
            ns.gate = t["gate"].index_select(0, r).cpu().numpy()
    return ns


def measure_configs(torch, fb, dev, flush):
    """Per-call time and GB/s at the configuration points (finalize entry point);
    from T = 2048 on also the cold kernel time."""
    res = []
    for name, T in CONFIG_POINTS:
        w = WORKLOADS[name]
        t = make_inputs(T, True, dev, seed=T, workload=name)
        o = torch.empty(T, w["H"], dtype=torch.bfloat16, device=dev)
        ro = torch.empty_like(o)
        ws = torch.zeros(fb.workspace_bytes(T, w["H"]), dtype=torch.uint8, device=dev)
        run = make_call(fb, t, True, ws, o, ro)
        us = time_graph(torch, run) if T <= 1024 else time_eager(torch, run, 20, 5)
        b = algorithmic_bytes(T, w["H"], w["R"], w["K"], shared=True, gate=w["gate"])
        ok = spot_check(torch, t, o, ro, sorted({0, T // 2, T - 1}))
        entry = {"workload": name, "T": T, "H": w["H"], "top_k": w["K"], "gate": w["gate"],
                 "us_per_call": round(us, 2), "GBps": round(b / us / 1e3, 1),
                 "pct_peak": round(100 * b / us / 1e3 / HBM_PEAK_GBS, 1),
                 "checked_vs_oracle": ok,
                 "plan": fb.get_plan(T, w["H"], w["R"], w["K"], True, ws.numel())}
        if T >= 2048:
            c = pcts(kernel_times_cold(torch, run, flush, calls=8))
            entry["us_cold_kernel"] = c
            entry["pct_cold"] = round(100 * b / c[1] / 1e3 / HBM_PEAK_GBS, 1)
        res.append(entry)
        del t, o, ro, ws, run
        torch.cuda.empty_cache()
    return res


def host_cpu():
    """Model name and logical CPU count of the host running the oracle."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def cpu_baseline(torch, t, seconds, workers=0):
    """The oracle as it stands on the host cores, two ways: one process on
    consecutive rows until ~seconds of oracle time, and (workers > 1) the same
    rows split into blocks over a pool of fresh processes (rows are
    independent, so the results are identical)."""
    import oracle

    T = t["residual"].shape[0]
    chunk = 256
    done = 0
    busy = 0.0
    while done < T and busy < seconds:
        rows = list(range(done, min(T, done + chunk)))
        host = rows_to_host(torch, t, rows)
        t0 = time.perf_counter()
        oracle.run_case(host)
        busy += time.perf_counter() - t0
        done += len(rows)
    b = algorithmic_bytes(done, H, R, K, shared=True)
    single = {"value": round(b / busy / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "sample": f"{done} of {T} rows of the headline workload (T={T}, H={H}, R={R}, "
                        f"K={K}/{E}, shared), NumPy fp64 track A + fp32 track B, one process; "
                        f"{busy:.1f} s of oracle time",
              "seconds": round(busy, 2), "rows": done, **host_cpu()}
    pool = _oracle_pool_run(torch, t, done, workers) if workers > 1 else None
    if pool is None:
        return single
    slowest, wall = pool
    return {"value": round(b / slowest / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"the same {done} rows in blocks of {chunk} rows dealt over {workers} worker "
                      f"processes (one core each; inputs memory-mapped from files); value = bytes "
                      f"/ the slowest worker's {slowest:.2f} s of oracle time ({wall:.2f} s wall "
                      f"clock including interpreter start-up)",
            "seconds": round(slowest, 2), "rows": done, **host_cpu(), "single_process": single}


_ORACLE_ARRAYS = ("partials", "residual", "gamma", "expert_out", "idx", "weights", "shared")


def oracle_worker(d, blocks, k):
    """Worker process (``bench.py --oracle-worker``): the oracle on row blocks of
    arrays memory-mapped from directory d; prints the oracle seconds as JSON."""
    import numpy as np
    from types import SimpleNamespace

    import oracle

    a = {n: np.load(os.path.join(d, n + ".npy"), mmap_mode="r") for n in _ORACLE_ARRAYS}
    busy, rows = 0.0, 0
    for r0, r1 in blocks:
        case = SimpleNamespace(
            partials=list(a["partials"][:, r0:r1]), residual=a["residual"][r0:r1],
            gamma=np.asarray(a["gamma"]), weight_bias=0.0, eps=1e-6,
            expert_out=a["expert_out"][r0 * k:r1 * k], idx=np.asarray(a["idx"][r0:r1]) - r0 * k,
            weights=np.asarray(a["weights"][r0:r1]), shared=a["shared"][r0:r1], gate=None)
        t0 = time.perf_counter()
        oracle.run_case(case)
        busy += time.perf_counter() - t0
        rows += r1 - r0
    print(json.dumps({"seconds": busy, "rows": rows}), flush=True)


def _oracle_pool_run(torch, t, rows, workers, chunk=256, timeout=300):
    """The oracle on rows [0, rows) in blocks over `workers` child processes (each
    a fresh interpreter running only NumPy).  Returns (slowest worker's oracle
    seconds, wall seconds) or None if a worker failed."""
    import shutil
    import subprocess
    import tempfile

    import numpy as np

    host = rows_to_host(torch, t, list(range(rows)))
    k = host.idx.shape[1]
    need = sum(a.nbytes for a in host.partials) + sum(
        getattr(host, n).nbytes for n in _ORACLE_ARRAYS[1:])
    base = None  # the default temporary directory, unless shared memory has room
    if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > 2 * need:
        base = "/dev/shm"
    d = tempfile.mkdtemp(prefix="oracle_rows_", dir=base)
    procs = []
    try:
        np.save(os.path.join(d, "partials.npy"), np.stack(host.partials))
        for n in _ORACLE_ARRAYS[1:]:
            np.save(os.path.join(d, n + ".npy"), getattr(host, n))
        del host
        blocks = [(r0, min(rows, r0 + chunk)) for r0 in range(0, rows, chunk)]
        env = dict(os.environ, OMP_NUM_THREADS="1")
        t0 = time.perf_counter()
        for w in range(workers):
            mine = blocks[w::workers]
            if not mine:
                continue
            arg = ",".join(f"{r0}:{r1}" for r0, r1 in mine)
            procs.append(subprocess.Popen(
                [sys.executable, os.path.abspath(__file__), "--oracle-worker", d, arg, str(k)],
                stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env))
        done, slowest = 0, 0.0
        for p in procs:
            out, err = p.communicate(timeout=timeout)
            if p.returncode != 0:
                sys.stderr.write(f"oracle worker failed: {err[-500:]}\n")
                return None
            r = json.loads(out.strip().splitlines()[-1])
            done += r["rows"]
            slowest = max(slowest, r["seconds"])
        wall = time.perf_counter() - t0
        assert done == rows
        return slowest, wall
    except subprocess.TimeoutExpired:
        return None
    finally:
        for p in procs:
            if p.poll() is None:
                p.kill()
                p.wait()
        shutil.rmtree(d, ignore_errors=True)


def small_and_large_targets(sweep, configs):
    """The two targets, worst case first, from the sweep and the config points."""
    out = {"small_T_target_us": SMALL_T_TARGET_US, "large_T_target_pct": LARGE_T_TARGET_PCT,
           "small_T_us_per_call_graph_max": {}, "small_T_busy_kernel_us_worst": {},
           "small_T_cold_kernel_us_worst": {}, "small_T_cold_no_event_kernel_us_worst": {},
           "small_T_idle_kernel_us_worst": {}, "large_T_cold_pct_min": {}}
    for entry in ("finalize", "reduce"):
        small = [s for s in sweep if s["entry"] == entry and s["T"] <= 16]
        large = [s for s in sweep if s["entry"] == entry and s["T"] >= 2048]
        if small:
            out["small_T_us_per_call_graph_max"][entry] = max(s["us_graph"] for s in small)
            for key, field in (("small_T_busy_kernel_us_worst", "us_busy_kernel"),
                               ("small_T_cold_no_event_kernel_us_worst",
                                "us_cold_kernel_no_event"),
                               ("small_T_idle_kernel_us_worst", "us_idle_kernel")):
                have = [s for s in small if field in s]
                if have:
                    wb = max(have, key=lambda s: s[field][1])
                    out[key][entry] = {"T": wb["T"], "p10_p50_p90": wb[field]}
            worst = max(small, key=lambda s: s["us_cold_kernel"][1])
            out["small_T_cold_kernel_us_worst"][entry] = {"T": worst["T"],
                                                           "p10_p50_p90": worst["us_cold_kernel"]}
        if large:
            out["large_T_cold_pct_min"][entry] = min(s["pct_cold"] for s in large)
    gated = [c["pct_cold"] for c in configs if c["workload"] == "gated_h8192_top10" and "pct_cold" in c]
    if gated:
        out["large_T_cold_pct_min"]["gated_h8192_top10"] = min(gated)
    small_ok = [v <= SMALL_T_TARGET_US for v in out["small_T_us_per_call_graph_max"].values()]
    small_ok += [v["p10_p50_p90"][1] <= SMALL_T_TARGET_US
                 for key in ("small_T_busy_kernel_us_worst", "small_T_cold_kernel_us_worst")
                 for v in out[key].values()]
    large_ok = [v >= LARGE_T_TARGET_PCT for v in out["large_T_cold_pct_min"].values()]
    out["met"] = {"small_T": bool(small_ok) and all(small_ok),
                  "large_T": bool(large_ok) and all(large_ok)}
    return out


def reap_children():
    """End any child process still alive (none is expected: the oracle pool's
    workers are waited for); returns how many there were."""
    try:
        import psutil
    except ImportError:
        return None
    kids = psutil.Process().children(recursive=True)
    for k in kids:
        try:
            sys.stderr.write(f"child process still running at exit: {k.pid} {k.cmdline()}\n")
            k.kill()
        except psutil.Error:
            pass
    psutil.wait_procs(kids, timeout=10)
    return len(kids)


def sweep_point(torch, fb, dev, flush, finalize, T):
    """One sweep entry: the headline shape at T rows, both timings, the split
    flow, and (finalize, T = 256..2048) the bandwidth probe."""
    ti = make_inputs(T, finalize, dev, seed=T)
    o = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ro = torch.empty_like(o)
    ws = torch.zeros(fb.workspace_bytes(T, H), dtype=torch.uint8, device=dev)
    rr = make_call(fb, ti, finalize, ws, o, ro)
    y = torch.empty_like(o)
    rs = make_split_call(fb, ti, finalize, o, ro, y)
    bt = algorithmic_bytes(T, H, R, K if finalize else 0, shared=finalize)
    ub = (pcts(kernel_times_busy(torch, rr))
          if T <= 16 and hasattr(torch.cuda, "_sleep") else None)
    un = pcts(kernel_times_cold(torch, rr, flush, events=False)) if T <= 16 else None
    ui = pcts(kernel_times_idle(torch, rr)) if T <= 16 else None
    if T <= 1024:
        ug = time_graph(torch, rr)
        uc = pcts(kernel_times_cold(torch, rr, flush, calls=20))
        us_split = time_graph(torch, rs)
    else:
        ug = time_eager(torch, rr, 20, 5)
        uc = pcts(kernel_times_cold(torch, rr, flush, calls=8))
        us_split = time_eager(torch, rs, 20, 5)
    probe_t = None
    if finalize and 256 <= T <= 2048:
        # what the part attains for this step's loads and stores at this T
        direct = list(ti["partials"]) + [ti["shared"], ti["residual"]]
        probe_t = pcts(kernel_times_cold(
            torch, lambda: fb.bandwidth_probe(direct, ti["expert_out"], ti["idx"],
                                              [o, ro], 2, 0),
            flush, calls=10, names=("probe_kernel",)))
    return {"entry": "finalize" if finalize else "reduce", "T": T,
            "us_graph": round(ug, 2), "us_cold_kernel": uc,
            **({"us_busy_kernel": ub} if ub else {}),
            **({"us_cold_kernel_no_event": un} if un else {}),
            **({"us_idle_kernel": ui} if ui else {}),
            "GBps_graph": round(bt / ug / 1e3, 1),
            "GBps_cold": round(bt / uc[1] / 1e3, 1),
            "pct_peak_graph": round(100 * bt / ug / 1e3 / HBM_PEAK_GBS, 1),
            "pct_cold": round(100 * bt / uc[1] / 1e3 / HBM_PEAK_GBS, 1),
            **({"probe_us_cold_kernel": probe_t,
                "probe_pct_cold": round(100 * bt / probe_t[1] / 1e3 / HBM_PEAK_GBS, 1)}
               if probe_t else {}),
            "us_split_graph": round(us_split, 2),
            "fused_speedup_vs_split": round(us_split / ug, 2),
            "plan": fb.get_plan(T, H, R, K if finalize else 0, finalize, ws.numel())}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true", help="headline only")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time budget for cpu_baseline (0 disables)")
    ap.add_argument("--cpu-workers", type=int, default=min(16, os.cpu_count() or 1),
                    help="processes for the all-cores oracle timing (1: single process only)")
    ap.add_argument("--T", type=int, default=HEADLINE_T, help="token rows of the timed step")
    ap.add_argument("--entry", choices=("finalize", "reduce"), default="finalize")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="headline",
                    help="shape family of the timed step (headline: H=7168, top-8 of 256)")
    ap.add_argument("--cold", action="store_true",
                    help="time the step with a 1 GiB cache flush before every call")
    ap.add_argument("--busy-before", choices=("spin",), default=None,
                    help="queue busy work ahead of every timed call instead of leaving the GPU "
                         "idle between calls: a one-wave 400k-cycle spin kernel that touches "
                         "no memory and outlasts the host's next launch")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run 3 plain device copies of this size (counter calibration)")
    ap.add_argument("--oracle-worker", nargs=3, metavar=("DIR", "BLOCKS", "K"),
                    help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.oracle_worker:
        d, blocks, k = args.oracle_worker
        oracle_worker(d, [tuple(int(x) for x in b.split(":")) for b in blocks.split(",")], int(k))
        return
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU's share of the boundary and runs on one GPU "
                         "only (use --gpus 1)\n")
        sys.exit(2)

    import torch

    import reduce_moe_finalize_amd as fb

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    torch.manual_seed(0)

    # ---------------- headline step
    T0 = args.T
    fin = args.entry == "finalize"
    wl = WORKLOADS[args.workload]
    t = make_inputs(T0, fin, dev, workload=args.workload)
    normed = torch.empty(T0, wl["H"], dtype=torch.bfloat16, device=dev)
    resid = torch.empty_like(normed)
    run = make_call(fb, t, fin, "auto", normed, resid)
    torch.cuda.synchronize()
    if args.cold:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            run()
        us = time_cold(torch, run, flush, calls=args.steps, reps=1)
        del flush
    elif args.busy_before:
        if not hasattr(torch.cuda, "_sleep"):
            sys.exit("--busy-before needs torch.cuda._sleep (torch's spin kernel)")

        def pre():  # ~0.17 ms of queued work, so the call is queued before it ends
            torch.cuda._sleep(SPIN_CYCLES)
        for _ in range(args.warmup):
            pre()
            run()
        us = time_cold(torch, run, None, calls=args.steps, reps=1, before=pre)
    else:
        us = time_eager(torch, run, args.steps, args.warmup)
    pct = per_call_percentiles(torch, run, args.steps)
    ok = spot_check(torch, t, normed, resid, sorted({0, 1, T0 // 2, T0 - 1}))
    B = algorithmic_bytes(T0, wl["H"], wl["R"], wl["K"] if fin else 0, shared=fin,
                          gate=fin and wl["gate"])
    gbs = B / us / 1e3
    headline = fin and T0 == HEADLINE_T and args.workload == "headline"
    plan = fb.get_plan(T0, wl["H"], wl["R"], wl["K"] if fin else 0, fin,
                       fb.workspace_bytes(T0, wl["H"]))
    traffic = read_traffic(plan) if headline else None
    probe = attainable_probe(torch, fb, t, (normed, resid), plan) if fin else None
    cpu = None
    if args.cpu_seconds > 0 and headline:
        cpu = cpu_baseline(torch, t, args.cpu_seconds, args.cpu_workers)
    del t, run
    torch.cuda.empty_cache()
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(3)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    copy_gbs = attainable_copy(torch, dev) if not args.no_sweep else None

    # ---------------- latency / bandwidth sweep over T (both entry points)
    sweep = []
    configs = []
    empty_us = time_empty_graph(torch, dev)
    empty_cold_us = None
    if not args.no_sweep:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        for finalize in (True, False):
            for T in SWEEP_T:
                sweep.append(sweep_point(torch, fb, dev, flush, finalize, T))
                torch.cuda.empty_cache()
        x1 = torch.zeros(1, device=dev)
        empty_cold_us = pcts(kernel_times_cold(torch, lambda: x1.add_(1.0), flush,
                                               names=("elementwise",)))[1]
        configs = measure_configs(torch, fb, dev, flush)
        del flush, x1

    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "us_per_call": round(us, 2),
        "us_per_call_p10_p50_p90": pct,
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "timing": ("cold (1 GiB flush before each call)" if args.cold else
                   f"warm, {args.busy_before} kernel queued before each call" if args.busy_before else
                   f"back-to-back; {B / 2**20:.0f} MiB moved per call, {B / MALL_BYTES:.1f}x the "
                   f"256 MB MALL, so every call streams from HBM" if B > 4 * MALL_BYTES else
                   "warm, back-to-back (working set can sit in the 256 MB MALL)"),
        "checked_vs_oracle": ok,
        "config": {"workload": (f"fused_moe_finalize_rmsnorm T={T0} H={wl['H']} R={wl['R']} "
                                f"top_k={wl['K']} of {wl['E']} experts, shared expert"
                                f"{' (sigmoid-gated)' if wl['gate'] else ''}, eps=1e-6"
                                f"{', weight_bias=1' if wl['wb'] else ''}" if fin else
                                f"fused_reduce_rmsnorm T={T0} H={wl['H']} R={wl['R']}, eps=1e-6"),
                   "T": T0, "H": wl["H"], "R": wl["R"], "top_k": wl["K"] if fin else 0,
                   "num_experts": wl["E"] if fin else 0, "shared": fin,
                   "parallelism": "1 GPU (one rank's share)", "plan": plan},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": B,
                     "attainable_loads_GBps": None if probe is None else probe["loads"],
                     "attainable_loads_stores_GBps": None if probe is None else probe["loads_stores"],
                     "frac_of_attainable": None if probe is None else round(gbs / probe["loads_stores"], 4),
                     "copy_GBps": copy_gbs,
                     "kernel": plan_kernel_name(plan) +
                               (" via fused_moe_finalize_rmsnorm" if fin else " via fused_reduce_rmsnorm")},
        "cpu_baseline": cpu,
        "empty_kernel_us_graph": round(empty_us, 2),
        "empty_kernel_us_cold": None if empty_cold_us is None else round(empty_cold_us, 2),
        "configs": configs,
        "sweep": sweep,
    }
    line["children_left_at_exit"] = reap_children()
    if sweep:
        line["targets"] = small_and_large_targets(sweep, configs)
    print(json.dumps(line), flush=True)


def plan_kernel_name(plan):
    if plan.get("units_per_wave"):
        return (f"balanced_kernel ({plan['units_per_wave']} units per wave, {plan['waves']} waves, "
                f"{plan['block']} lanes per workgroup)")
    if plan["sources_per_batch"]:
        return (f"stream_kernel<{plan['vec_per_thread']}, {plan['sources_per_batch']}> ("
                + (f"at most {plan['workgroups_per_cu']} workgroups per CU)"
                   if plan["workgroups_per_cu"] else "no per-CU limit)"))
    return f"latency_kernel ({plan['block']} lanes, rows split {plan['split']} ways)"


if __name__ == "__main__":
    main()
