"""The C ABI without torch: a plain C program (tests/c_abi_consumer.c) allocates
device memory with hipMalloc, calls an entry point of include/fused_boundary.h on
a stream of its own and writes the outputs; they are checked against the oracle.
The consumer runs as a child process, so the library is loaded in a process
where torch never ran."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import compare, say
from workloads import make_case

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.join(ROOT, "reduce_moe_finalize_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    exe = tmp_path_factory.mktemp("c_consumer") / "c_abi_consumer"
    subprocess.run(["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, "c_abi_consumer.c"), "-o", str(exe),
                    "-L", LIBDIR, "-lfused_boundary", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                   check=True, capture_output=True, text=True)
    return exe


def run_consumer(exe, tmp_path, case, finalize):
    T, H = case.residual.shape
    R = len(case.partials)
    K = case.idx.shape[1] if finalize else 0
    N = case.expert_out.shape[0] if finalize else 0
    shared = finalize and case.shared is not None
    gate = shared and case.gate is not None
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        np.array([T, H, R, K, N, int(shared), int(gate), int(finalize)], np.int64).tofile(f)
        np.array([case.eps, case.weight_bias], np.float32).tofile(f)
        for p in case.partials:
            np.ascontiguousarray(p, np.uint16).tofile(f)
        np.ascontiguousarray(case.residual, np.uint16).tofile(f)
        np.ascontiguousarray(case.gamma, np.uint16).tofile(f)
        if finalize:
            np.ascontiguousarray(case.expert_out, np.uint16).tofile(f)
            np.ascontiguousarray(case.idx, np.int32).tofile(f)
            np.ascontiguousarray(case.weights, np.float32).tofile(f)
            if shared:
                np.ascontiguousarray(case.shared, np.uint16).tofile(f)
            if gate:
                np.ascontiguousarray(case.gate, np.float32).tofile(f)
    dst = tmp_path / "out.bin"
    res = subprocess.run([str(exe), str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    raw = np.fromfile(dst, dtype=np.uint8)
    status = int(raw[:4].view(np.int32)[0])
    body = raw[4:].view(np.uint16)
    return status, body[:T * H].reshape(T, H), body[T * H:].reshape(T, H)


@pytest.mark.parametrize("name,kw,finalize", [
    ("finalize T=16 H=7168 top-8 + shared (split rows)",
     dict(T=16, H=7168, R=8, K=8, num_experts=256, shared=True), True),
    ("reduce T=5 H=4104 R=3", dict(T=5, H=4104, R=3), False),
    ("finalize T=40 H=2048 top-10 gated, weight_bias 1",
     dict(T=40, H=2048, R=2, K=10, num_experts=64, shared=True, gate=True, weight_bias=1.0,
          gamma_dist="normal01"), True),
    ("finalize T=600 H=1024 top-2 + shared (stream kernel)",
     dict(T=600, H=1024, R=2, K=2, num_experts=16, shared=True), True),
])
def test_c_consumer_matches_oracle(consumer, tmp_path, name, kw, finalize):
    kw = dict(kw)
    T, H, R = kw.pop("T"), kw.pop("H"), kw.pop("R")
    case = make_case(T, H, R, seed=T + H, **kw)
    if finalize:
        case.idx = case.idx.copy()
        case.idx[0, 0] = -1  # one skipped slot
    say(f"C consumer: {name}")
    status, normed, resid = run_consumer(consumer, tmp_path, case, finalize)
    assert status == 0
    compare(normed, resid, oracle.run_case(case), f"C consumer {name}")


def test_c_consumer_sees_a_decline(consumer, tmp_path):
    """H % 8 != 0 is declined before anything is launched (status 2)."""
    case = make_case(3, 12, 2, seed=5)
    status, _, _ = run_consumer(consumer, tmp_path, case, False)
    assert status == 2
