"""bench.py's host-side bookkeeping (no GPU): the device-code fingerprint that
keeps recorded HBM counters tied to the kernel they were taken on."""
import os
import sys

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
