"""bench.py's host-side bookkeeping (no GPU): the device-code fingerprint that
keeps recorded HBM counters tied to the kernel they were taken on."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_fingerprint_covers_device_code_only(tmp_path, monkeypatch):
    src = open(bench.SRC).read()
    assert bench.HOST_SIDE_MARKER in src
    base = bench.source_sha256()
    device, host = src.split(bench.HOST_SIDE_MARKER, 1)

    def fp(text):
        f = tmp_path / "k.hip"
        f.write_text(text)
        monkeypatch.setattr(bench, "SRC", str(f))
        return bench.source_sha256()

    assert fp(src) == base
    # comments, indentation and blank lines do not count
    assert fp("// note\n" + device.replace("\n", "\n\n") + bench.HOST_SIDE_MARKER + host) == base
    # launcher edits do not count either
    assert fp(device + bench.HOST_SIDE_MARKER + host + "\nint extra_host_fn() { return 1; }\n") == base
    # a device-code edit does
    assert fp(device.replace("kWsRowBytes = 512", "kWsRowBytes = 1024") + bench.HOST_SIDE_MARKER
              + host) != base


def test_traffic_requires_matching_plan(tmp_path, monkeypatch):
    sha = bench.source_sha256()
    prof = tmp_path / "t.md"
    prof.write_text(f"kernel_code_sha256: {sha}\nplan_block_vec_batch_wgcu: 128 8 1 4\n"
                    "fetch_bytes_per_launch: 100\nwrite_bytes_per_launch: 20\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    plan = {"block": 128, "vec_per_thread": 8, "sources_per_batch": 1, "workgroups_per_cu": 4}
    assert bench.read_traffic(plan) == 120.0
    assert bench.read_traffic(dict(plan, workgroups_per_cu=0)) is None
    assert bench.read_traffic(dict(plan, block=256, vec_per_thread=4)) is None
    prof.write_text(prof.read_text().replace(sha, "0" * 64))
    assert bench.read_traffic() is None


def test_oracle_pool_covers_every_row_once():
    """The all-cores oracle timing deals every row block to one worker process."""
    import torch

    from workloads import make_case, to_torch

    case = make_case(40, 256, 2, seed=5, K=3, num_experts=8, shared=True)
    t = to_torch(case, torch.device("cpu"))
    res = bench._oracle_pool_run(torch, t, 40, workers=3, chunk=8, timeout=120)
    assert res is not None
    slowest, wall = res
    assert 0 < slowest <= wall


def test_host_cpu_is_recorded():
    info = bench.host_cpu()
    assert set(info) == {"cpu_model", "os_cpu_count"}
    assert info["os_cpu_count"] == os.cpu_count()


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    import subprocess

    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert res.returncode == 2 and "one GPU" in res.stderr and res.stdout == ""


def test_targets_take_the_worst_case():
    """The targets object reports the slowest small-T call and the lowest
    large-T cold bandwidth, and says whether each target is met."""
    sweep = []
    for entry, small, cold, pct in (("finalize", 4.4, [4.5, 4.8, 5.1], 78.0),
                                    ("reduce", 3.9, [4.3, 4.6, 4.9], 71.0)):
        for T in (1, 16):
            sweep.append({"entry": entry, "T": T, "us_graph": small - (0.2 if T == 1 else 0.0),
                          "us_cold_kernel": [c - (0.3 if T == 1 else 0.0) for c in cold],
                          "us_busy_kernel": [c - (0.5 if T == 16 else 0.6) for c in cold],
                          "us_cold_kernel_no_event": [c - (0.3 if T == 1 else 0.0) + 0.4 for c in cold],
                          "us_idle_kernel": [c + (0.6 if T == 1 else 0.5) for c in cold]})
        for T in (2048, 8192):
            sweep.append({"entry": entry, "T": T, "pct_cold": pct + (1.0 if T == 8192 else 0.0)})
    configs = [{"workload": "gated_h8192_top10", "T": 2048, "pct_cold": 80.0},
               {"workload": "gated_h8192_top10", "T": 8192, "pct_cold": 69.5},
               {"workload": "gated_h8192_top10", "T": 128}]
    t = bench.small_and_large_targets(sweep, configs)
    assert t["small_T_us_per_call_graph_max"] == {"finalize": 4.4, "reduce": 3.9}
    assert t["small_T_cold_kernel_us_worst"]["finalize"] == {"T": 16, "p10_p50_p90": [4.5, 4.8, 5.1]}
    assert t["small_T_busy_kernel_us_worst"]["reduce"] == {"T": 16, "p10_p50_p90": [3.8, 4.1, 4.4]}
    assert t["large_T_cold_pct_min"] == {"finalize": 78.0, "reduce": 71.0, "gated_h8192_top10": 69.5}
    # reported, but not part of "met": the call queued directly behind the flush
    ne = t["small_T_cold_no_event_kernel_us_worst"]["finalize"]
    assert ne["T"] == 16 and ne["p10_p50_p90"] == pytest.approx([4.9, 5.2, 5.5])
    # and a launch onto an idle GPU, over 5 us here, reported only as well
    idle = t["small_T_idle_kernel_us_worst"]["finalize"]
    assert idle["T"] == 1 and idle["p10_p50_p90"] == pytest.approx([5.1, 5.4, 5.7])
    assert t["met"] == {"small_T": True, "large_T": False}
    sweep[1]["us_cold_kernel"] = [5.0, 5.2, 5.4]
    assert bench.small_and_large_targets(sweep, configs[:1])["met"] == {"small_T": False,
                                                                          "large_T": True}
    sweep[1]["us_cold_kernel"] = [4.5, 4.8, 5.1]
    sweep[0]["us_busy_kernel"] = [4.9, 5.1, 5.3]  # T=1 now the worst busy case, over the target
    t = bench.small_and_large_targets(sweep, configs[:1])
    assert t["small_T_busy_kernel_us_worst"]["finalize"]["T"] == 1 and not t["met"]["small_T"]


def test_percentiles_and_kernel_names():
    assert bench.pcts([5.0]) == [5.0, 5.0, 5.0]
    p10, p50, p90 = bench.pcts([float(i) for i in range(1, 101)])
    assert p10 < p50 < p90 and p50 == 50.5
    assert "balanced_kernel" in bench.plan_kernel_name(
        {"units_per_wave": 2, "waves": 4096, "block": 1024, "sources_per_batch": 0})
    assert bench.plan_kernel_name({"units_per_wave": 0, "sources_per_batch": 1, "vec_per_thread": 4,
                                   "workgroups_per_cu": 3}).startswith("stream_kernel<4, 1>")
    assert "latency_kernel" in bench.plan_kernel_name(
        {"units_per_wave": 0, "sources_per_batch": 0, "block": 128, "split": 7})


def test_no_child_process_outlives_the_run():
    assert bench.reap_children() == 0


def test_probe_shape_fits_the_probe():
    """The probe beside the timed step takes the step's own stream shape, and
    never more lanes per row than the probe kernel allows (a whole-row plan
    with one vector per lane, T <= 2 rows per CU, is widened)."""
    stream = {"vec_per_thread": 4, "sources_per_batch": 1, "workgroups_per_cu": 3}
    assert bench.probe_shape(stream, 7168) == (4, 3)
    one_vec = {"vec_per_thread": 1, "sources_per_batch": 2, "workgroups_per_cu": 0}
    assert bench.probe_shape(one_vec, 7168) == (2, 0)
    assert bench.probe_shape(one_vec, 16384) == (4, 0)
    assert bench.probe_shape(one_vec, 4096) == (1, 0)
    latency = {"vec_per_thread": 1, "sources_per_batch": 0, "workgroups_per_cu": 0}
    assert bench.probe_shape(latency, 7168) == (4, 0)
    for H in range(8, 16385, 8):
        vpt, _ = bench.probe_shape(one_vec, H)
        assert -(-(H // 8) // vpt) <= 512, H


def test_every_profile_summary_is_of_the_current_device_code():
    """Each rocprofv3 summary under profiles/ names the device code it was
    measured on; all of them must be of the code in the tree, so no figure
    there outlives a kernel change."""
    prof = os.path.join(ROOT, "profiles")
    sha = bench.source_sha256()
    files = [f for f in sorted(os.listdir(prof)) if f.endswith(".md") and f != "README.md"]
    assert files
    for f in files:
        text = open(os.path.join(prof, f)).read()
        lines = [ln for ln in text.splitlines() if ln.startswith("kernel_code_sha256:")]
        assert lines, f"{f} names no device code"
        assert lines[0].split(":", 1)[1].strip() == sha, f"{f} was measured on other device code"
