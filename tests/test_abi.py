"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side argument checks return before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fused_boundary.h")
LIB = os.path.join(ROOT, "reduce_moe_finalize_amd", "libfused_boundary.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith("fused_")))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (same runtime binding order as the package)

    L = ctypes.CDLL(LIB)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.fused_reduce_rmsnorm.argtypes = [ctypes.POINTER(vp), i32, vp, vp, f32, f32, i64, i64, vp, vp, vp,
                                       sz, vp]
    L.fused_moe_finalize_rmsnorm.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, vp, i32, vp, vp, vp,
                                             vp, f32, f32, i64, i64, vp, vp, vp, sz, vp]
    L.fused_boundary_workspace_bytes.argtypes = [i64, i64]
    L.fused_boundary_workspace_bytes.restype = sz
    L.fused_boundary_status_string.restype = ctypes.c_char_p
    return L


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fused_reduce_rmsnorm", "fused_moe_finalize_rmsnorm", "fused_boundary_workspace_bytes",
            "fused_boundary_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_status_strings_and_workspace(lib):
    assert lib.fused_boundary_status_string(0) == b"ok"
    assert b"declined" in lib.fused_boundary_status_string(2)
    assert lib.fused_boundary_status_string(99) == b"unknown status"
    assert lib.fused_boundary_workspace_bytes(0, 7168) == 256
    assert lib.fused_boundary_workspace_bytes(16, 7168) == 256 + 16 * 512
    assert lib.fused_boundary_workspace_bytes(-1, 7168) == 0


# Fake, never-dereferenced device addresses: each call below must be rejected on
# the host before anything is launched.
A = 0x10000000
SZ = 1 << 24


def fake(i, off=0):
    return ctypes.c_void_p(A + i * SZ + off)


def reduce_call(lib, R=2, resid=True, H=64, T=4, eps=1e-6, wb=0.0, normed=None, misalign=0,
                partial_ptrs=None):
    ps = partial_ptrs or [A + (10 + r) * SZ + (misalign if r == 0 else 0) for r in range(R)]
    arr = (ctypes.c_void_p * max(1, R))(*ps)
    return lib.fused_reduce_rmsnorm(arr, R, fake(1) if resid else None, fake(2), wb, eps, T, H,
                                    normed if normed is not None else fake(3), fake(4), None, 0, None)


def test_reduce_validation(lib):
    assert reduce_call(lib, R=0) == 1
    assert reduce_call(lib, R=17) == 1
    assert reduce_call(lib, resid=False) == 1  # a residual is required
    assert reduce_call(lib, T=-1) == 1
    assert reduce_call(lib, H=0) == 1
    assert reduce_call(lib, eps=float("nan")) == 1
    assert reduce_call(lib, eps=-1.0) == 1
    assert reduce_call(lib, wb=float("inf")) == 1
    assert reduce_call(lib, normed=ctypes.c_void_p(A + 10 * SZ)) == 1  # output overlaps a partial
    assert reduce_call(lib, H=12) == 2  # H % 8 != 0 -> declined
    assert reduce_call(lib, H=16392) == 2  # H > max -> declined
    assert reduce_call(lib, misalign=8) == 2  # misaligned bf16 pointer -> declined
    assert reduce_call(lib, T=0) == 0  # no-op, nothing launched
    arr = (ctypes.c_void_p * 2)(A + 10 * SZ, None)
    assert lib.fused_reduce_rmsnorm(arr, 2, fake(1), fake(2), 0.0, 1e-6, 4, 64, fake(3), fake(4), None,
                                    0, None) == 1


def finalize_call(lib, K=8, N=32, idx=True, w=True, expert=True, T=4, H=64, shared=None, gate=None,
                  resid_out=None, ws=None, ws_bytes=0):
    arr = (ctypes.c_void_p * 1)(A + 10 * SZ)
    return lib.fused_moe_finalize_rmsnorm(
        arr, 1, fake(5) if expert else None, N, fake(6) if idx else None, fake(7) if w else None, K,
        shared, gate, fake(1), fake(2), 0.0, 1e-6, T, H, fake(3),
        resid_out if resid_out is not None else fake(4), ws, ws_bytes, None)


def test_finalize_validation(lib):
    assert finalize_call(lib, K=0) == 1
    assert finalize_call(lib, K=17) == 1
    assert finalize_call(lib, idx=False) == 1
    assert finalize_call(lib, w=False) == 1
    assert finalize_call(lib, expert=False) == 1  # N > 0 needs expert rows
    assert finalize_call(lib, N=-1) == 1
    assert finalize_call(lib, N=(1 << 40) + 1) == 1
    assert finalize_call(lib, expert=False, N=0, H=12) == 2
    assert finalize_call(lib, shared=fake(8, 4)) == 2  # misaligned shared -> declined
    assert finalize_call(lib, gate=fake(9, 2)) == 1  # misaligned fp32 gate
    assert finalize_call(lib, resid_out=fake(5)) == 1  # output overlaps the expert rows
    # in place over an expert buffer that is the residual itself: its rows are
    # gathered at any index, so an in-place update would race with the gathers
    arr = (ctypes.c_void_p * 1)(A + 10 * SZ)
    assert lib.fused_moe_finalize_rmsnorm(
        arr, 1, fake(1), 4, fake(6), fake(7), 8, None, None, fake(1), fake(2), 0.0, 1e-6, 4, 64,
        fake(3), fake(1), None, 0, None) == 1
    assert finalize_call(lib, resid_out=fake(1, 2)) == 1  # partial overlap with residual_in
    assert finalize_call(lib, ws=fake(11, 8), ws_bytes=4096) == 1  # misaligned workspace
    assert finalize_call(lib, ws=fake(3), ws_bytes=4096) == 1  # workspace overlaps an output
    assert finalize_call(lib, T=0) == 0


def noalloc_call(lib, K=8, T=4, H=64, R=1, resid=True):
    arr = (ctypes.c_void_p * max(1, R))(*[A + (10 + r) * SZ for r in range(R)])
    lib.fused_moe_finalize_rmsnorm_noalloc.argtypes = [
        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return lib.fused_moe_finalize_rmsnorm_noalloc(
        arr, R, fake(5), 32, fake(6), fake(7), K, None, None, fake(1) if resid else None, fake(2),
        0.0, 1e-6, T, H, fake(3), fake(4), None)


def test_noalloc_validation_and_row_capacity(lib):
    """The allocation-free entry point checks like the others, and refuses more
    token rows than its static scratch holds, before anything is launched."""
    cap = 1024  # FB_NOALLOC_MAX_ROWS
    assert noalloc_call(lib, T=cap + 1) == 4
    assert noalloc_call(lib, K=0, T=cap + 1) == 4
    assert b"FB_NOALLOC_MAX_ROWS" in lib.fused_boundary_status_string(4)
    assert noalloc_call(lib, resid=False) == 1
    assert noalloc_call(lib, K=17) == 1
    assert noalloc_call(lib, K=0, R=0) == 1  # no finalize needs a partial
    assert noalloc_call(lib, H=12) == 2
    assert noalloc_call(lib, T=0) == 0
    assert noalloc_call(lib, K=0, T=0) == 0
    text = open(HEADER).read()
    assert re.search(r"#define FB_NOALLOC_MAX_ROWS %d\b" % cap, text)


def test_forced_decline_returns_before_launch(lib):
    lib.fused_boundary_set_force_decline.argtypes = [ctypes.c_int]
    lib.fused_boundary_set_force_decline(1)
    try:
        assert reduce_call(lib) == 2  # valid call, declined, nothing launched
        assert finalize_call(lib) == 2
        assert reduce_call(lib, R=0) == 1  # invalid arguments still win
        assert finalize_call(lib, T=0) == 0  # no tokens: still a no-op
    finally:
        lib.fused_boundary_set_force_decline(0)
    assert reduce_call(lib, H=12) == 2 and reduce_call(lib, R=0) == 1


class Plan(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("vec_per_thread", ctypes.c_int32),
                ("split", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("sources_per_batch", ctypes.c_int32), ("workgroups_per_cu", ctypes.c_int32),
                ("units_per_wave", ctypes.c_int32), ("waves", ctypes.c_int32)]


def test_plan_override_validation(lib):
    bad = [Plan(96, 1, 0, 0, 0), Plan(256, 3, 0, 0, 1), Plan(1024, 4, 0, 0, 2),
           Plan(256, 2, 0, 0, 0), Plan(128, 8, 0, 0, 3), Plan(2048, 1, 0, 0, 0),
           Plan(128, 8, 0, 0, 1, 17), Plan(128, 8, 0, 0, 1, -1), Plan(256, 1, 0, 0, 0, 4)]
    for p in bad:
        assert lib.fused_boundary_set_plan_override(ctypes.byref(p)) == 1
    for p in [Plan(512, 2, 0, 0, 4), Plan(256, 1, 0, 0, 0), Plan(128, 8, 0, 0, 1),
              Plan(128, 8, 0, 0, 1, 4)]:
        assert lib.fused_boundary_set_plan_override(ctypes.byref(p)) == 0
    assert lib.fused_boundary_set_plan_override(None) == 0


def test_auto_plan_shapes(lib):
    """The host-side plan: latency kernel (split rows) at small T, stream kernel at large T."""
    lib.fused_boundary_get_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_size_t,
                                            ctypes.POINTER(Plan)]
    ws = lib.fused_boundary_workspace_bytes(16, 7168)

    def plan(T, H, R=8, K=8, sh=1, wsb=None):
        p = Plan()
        rc = lib.fused_boundary_get_plan(T, H, R, K, sh, ws if wsb is None else wsb, ctypes.byref(p))
        return rc, (p.block, p.vec_per_thread, p.split, p.grid, p.sources_per_batch)

    assert plan(16, 7168) == (0, (64, 1, 14, 224, 0))  # latency kernel, one wave, rows split 14 ways
    assert plan(17, 7168, wsb=lib.fused_boundary_workspace_bytes(17, 7168))[1] == (128, 1, 7, 119, 0)
    ws64 = lib.fused_boundary_workspace_bytes(64, 7168)
    assert plan(32, 7168, wsb=ws64)[1] == (128, 1, 7, 224, 0)
    assert plan(64, 7168, wsb=ws64)[1] == (256, 1, 4, 256, 0)
    assert plan(16, 7168, K=0, sh=0)[1] == (64, 1, 14, 224, 0)  # reduce: one wave per workgroup
    # reduce, 17..32 rows: 128 lanes up to H=7168, 4 ways beyond
    assert plan(32, 7168, K=0, sh=0, wsb=ws64)[1] == (128, 1, 7, 224, 0)
    assert plan(32, 8192, K=0, sh=0, wsb=ws64)[1] == (256, 1, 4, 128, 0)
    assert plan(256, 7168, wsb=lib.fused_boundary_workspace_bytes(256, 7168)) == (0, (896, 1, 1, 256, 0))
    # up to 2 rows per CU: whole rows, one vector per lane, 2 sources per batch
    assert plan(512, 7168)[1] == (896, 1, 1, 512, 2)
    assert plan(512, 16384)[1] == (1024, 2, 1, 512, 2)  # rows over 1024 vectors: 2 per lane
    # just past one row per CU with expert gathers: the balanced kernel, 512-element
    # units dealt evenly over 2 (3 waves per SIMD: 1) workgroups per CU (needs the workspace)
    ws384 = lib.fused_boundary_workspace_bytes(384, 8192)
    assert plan(257, 7168, wsb=ws384)[1] == (512, 1, 14, 512, 0)
    assert plan(274, 7168, wsb=ws384)[1] == (512, 1, 14, 512, 0)
    assert plan(320, 6144, wsb=ws384)[1] == (512, 1, 12, 512, 0)
    assert plan(256, 8192, K=10, wsb=ws384)[1] == (768, 1, 16, 256, 0)  # 12-slot variant
    # 15 to 20 units per CU with expert gathers: the streamed form, two 12-wave
    # workgroups per CU, sources two at a time
    assert plan(275, 7168, wsb=ws384)[1] == (768, 1, 14, 512, 2)
    assert plan(300, 7168, wsb=ws384)[1] == (768, 1, 14, 512, 2)
    assert plan(365, 7168, wsb=ws384)[1] == (768, 1, 14, 512, 2)
    assert plan(366, 7168, wsb=ws384)[1] == (896, 1, 1, 366, 2)  # past 20 units per CU
    assert plan(300, 8192, K=10, wsb=ws384)[1] == (768, 1, 16, 512, 2)
    assert plan(352, 6144, wsb=ws384)[1] == (768, 1, 12, 512, 2)
    assert plan(320, 6144, wsb=ws384)[1][4] == 0 and plan(321, 6144, wsb=ws384)[1][4] == 2  # 15 units per CU
    assert plan(300, 7168, K=0, sh=0, wsb=ws384)[1] == (896, 1, 1, 300, 2)  # reduce: stream
    # the streamed form only at the widths it was measured on (H = 6144..8192)
    assert plan(560, 4096, wsb=lib.fused_boundary_workspace_bytes(560, 4096))[1][2] == 1
    assert plan(300, 7168, wsb=0)[1] == (896, 1, 1, 300, 2)  # no workspace: stream kernel

    def wg(T, H, K=8):
        p = Plan()
        assert lib.fused_boundary_get_plan(T, H, 8, K, 1, 0, ctypes.byref(p)) == 0
        return p.vec_per_thread, p.workgroups_per_cu

    # about 60 KiB of source rows in flight per CU with 4 or 8 vectors per lane
    assert wg(2048, 7168) == (4, 4)
    assert wg(1536, 7168) == (4, 3) and wg(3072, 7168) == (4, 3) and wg(1024, 7168) == (4, 4)
    assert wg(2560, 7168) == (4, 5) and wg(3584, 7168) == (4, 3)
    # 16 or more rows per CU: H = 5120..7168 keep 4 vectors per lane at about 12 waves per CU
    assert wg(8192, 7168) == (4, 3) and wg(4096, 7168) == (4, 3) and wg(8192, 6144) == (4, 4)
    assert wg(8192, 5120) == (4, 4)
    assert wg(8192, 8192, K=10) == (8, 4)
    # rows over 1536 vectors: 2 vectors per lane, one 1024-lane workgroup per CU; H=12288: 4 at 12 waves
    assert wg(8192, 16384) == (2, 1) and wg(2048, 16384) == (2, 1)
    assert wg(8192, 12288) == (4, 2) and wg(2048, 12288) == (4, 2)
    # narrow rows beyond 3 per CU: 2 vectors per lane, about 16 waves per CU
    assert wg(8192, 1024) == (2, 16) and wg(8192, 2048) == (2, 8) and wg(1024, 4096) == (2, 4)
    assert wg(16384, 3072) == (2, 5) and wg(768, 4096) == (2, 0)
    assert wg(512, 7168) == (1, 0)  # 1 or 2 vectors per lane: no limit
    assert wg(513, 7168) == (2, 0) and wg(768, 7168) == (2, 0) and wg(769, 7168)[0] == 4
    assert wg(16, 7168)[1] == 0  # latency kernel: no limit
    assert plan(16, 7168, wsb=0) == (0, (896, 1, 1, 16, 0))  # no workspace: whole rows
    assert plan(16, 7168, R=12, K=10, wsb=0)[1][4] > 0  # large R,K without workspace: stream
    rc, p = plan(8192, 7168)
    assert rc == 0 and p[4] > 0 and p[2] == 1 and p[0] * p[1] >= 896
    # other hidden sizes: T<=16 uses one-wave workgroups, whole rows from T=129 to #CU
    assert plan(16, 6144) == (0, (64, 1, 12, 192, 0))
    assert plan(16, 8192, K=10) == (0, (64, 1, 16, 256, 0))
    ws_big = lib.fused_boundary_workspace_bytes(256, 8192)
    assert plan(192, 8192, K=10, wsb=ws_big)[1][:3] == (256, 1, 4)  # 12-slot variant: <= 512 lanes
    # split 4 ways no longer fits at once past 192 rows (3 workgroups per CU): balanced
    assert plan(256, 8192, K=10, wsb=ws_big)[1][:3] == (768, 1, 16)
    assert plan(128, 8192, K=10, wsb=ws_big)[1][:3] == (512, 1, 2)
    assert plan(256, 8192, K=8, wsb=ws_big)[1][:3] == (1024, 1, 1)
    assert plan(2048, 6144)[1] == (192, 4, 1, 2048, 1)
    assert plan(8192, 8192)[1] == (128, 8, 1, 8192, 1)
    assert plan(4096, 7168)[1] == (256, 4, 1, 4096, 1)
    assert plan(8, 12)[0] == 2  # declined shape
    assert plan(-1, 7168)[0] == 1
    lib.fused_boundary_get_plan.argtypes = None


def test_product_path_never_touches_oracle():
    pkg = os.path.join(ROOT, "reduce_moe_finalize_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), f
                assert "workloads" not in text, f


def sgpr_waves_per_simd(sgprs):
    """Waves per SIMD that a kernel's scalar registers allow on MI355X, as
    measured there with probe kernels of 46 to 104 SGPRs (each workgroup
    recording its CU and the realtime counter around a sleep): a wave holds its
    SGPR count plus 16, rounded up to a multiple of 16, of 800 per SIMD -- 8
    waves up to 79 SGPRs, 7 up to 95, 6 up to 111.  The compiler's occupancy
    report and the runtime's occupancy query both leave the 16 out."""
    alloc = -(-(sgprs + 16) // 16) * 16
    return min(8, 800 // alloc)


def test_sgpr_rule_matches_the_measured_points():
    # (SGPRs, waves per SIMD measured resident at once)
    for sg, waves in ((46, 8), (66, 8), (67, 8), (73, 8), (79, 8), (81, 7), (86, 7), (96, 7),
                      (104, 6)):
        assert sgpr_waves_per_simd(sg) == waves, sg


def compiled_occupancy():
    """Waves per SIMD of every kernel instantiation, from the compiler's own
    resource report for gfx950 (independent of the planner's table), lowered
    to what its scalar registers allow (sgpr_waves_per_simd)."""
    import subprocess
    import tempfile

    src = os.path.join(ROOT, "reduce_moe_finalize_amd", "csrc", "fused_boundary.hip")
    with tempfile.TemporaryDirectory() as d:
        cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), src, "-o", os.path.join(d, "x.so"),
               "-Rpass-analysis=kernel-resource-usage"]
        out = subprocess.run(cmd, capture_output=True, text=True, timeout=600).stderr
    occ, name, sgprs = {}, None, None
    for ln in out.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name, sgprs = m.group(1), None
            continue
        m = re.search(r"TotalSGPRs: (\d+)", ln)
        if m:
            sgprs = int(m.group(1))
            continue
        m = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", ln)
        if m and name:
            k = re.search(r"(latency|balanced)_kernelILi(\d+)ELi(\d+)ELi(\d+)E", name)
            if k:  # several builds of one variant (latency: both store policies): the fewest
                assert sgprs is not None, name
                key = (k.group(1), int(k.group(2)), int(k.group(3)), int(k.group(4)))
                waves = min(int(m.group(1)), sgpr_waves_per_simd(sgprs))
                occ[key] = min(occ.get(key, 99), waves)
            name = None
    assert occ, out[-2000:]
    return occ


@pytest.fixture(scope="module")
def occupancy():
    return compiled_occupancy()


def test_residency_table_matches_the_compiler(lib, occupancy):
    """The workgroups per CU the planner counts on for every latency and
    balanced variant and block size never exceed what the compiler's register
    report allows (4 SIMDs x waves per SIMD, at most 16 workgroups per CU)."""
    lib.fused_boundary_resident_workgroups.argtypes = [ctypes.c_int32] * 5 + [
        ctypes.POINTER(ctypes.c_int32)] * 2
    variants = {(8, 0): (10, 0), (16, 0): (18, 0), (8, 8): (10, 8), (8, 12): (10, 12),
                (16, 16): (18, 16)}
    lat_bound = {(10, 0): 1024, (18, 0): 256, (10, 8): 1024, (10, 12): 512, (18, 16): 256}
    checked = 0
    for (R, K), (md, me) in variants.items():
        for upw, spb in [(u, 0) for u in (0, 1, 2, 3, 4, 6, 8)] + [(1, 2)]:
            for block in range(64, 1025, 64):
                planned, device = ctypes.c_int32(-1), ctypes.c_int32()
                rc = lib.fused_boundary_resident_workgroups(R, K, upw, spb, block,
                                                            ctypes.byref(planned),
                                                            ctypes.byref(device))
                if rc == 1:
                    continue
                # the streamed balanced form is one build for every R and K
                key = (("balanced", 0, 0, 1) if spb else ("balanced", md, me, upw) if upw
                       else ("latency", md, me, lat_bound[(md, me)]))
                assert key in occupancy, key
                allowed = min(16, 4 * occupancy[key] // (block // 64))
                assert 0 <= planned.value <= allowed, (R, K, upw, block, planned.value, allowed)
                checked += 1
    assert checked > 300


def test_auto_plan_invariants_over_a_grid(lib, occupancy):
    """The automatic plan is always launchable: for every size on a broad grid the
    plan covers the row, stays within the lane bounds of its kernel variant, fits
    the workspace it was given, and keeps the per-CU limit in range.  Every
    launch whose workgroups wait for each other (split rows, balanced units) is
    resident at once on a 256-CU part: its grid is within what the compiler's
    register report lets the CUs hold (at most 16 workgroups per CU)."""
    lib.fused_boundary_get_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_size_t,
                                            ctypes.POINTER(Plan)]
    lib.fused_boundary_workspace_bytes.restype = ctypes.c_size_t

    def variant(R, K):
        few = R + 2 <= 10
        if K == 0:
            return (10, 0) if few else (18, 0)
        if few and K <= 8:
            return (10, 8)
        if few and K <= 12:
            return (10, 12)
        return (18, 16)

    def latency_bound(R, K):
        return {(10, 0): 1024, (10, 8): 1024, (10, 12): 512}.get(variant(R, K), 256)

    def resident_wgs(wps, block):
        return 256 * min(16, 4 * wps // (block // 64))

    n = waits = 0
    for T in (1, 2, 7, 16, 31, 64, 100, 128, 129, 200, 256, 257, 292, 293, 300, 320, 384, 385,
              511, 512, 513, 640, 700, 768, 769, 1000, 2048, 4095, 4096, 6000, 8192, 20000):
        for H in (8, 64, 520, 1024, 2048, 4096, 6144, 7168, 7176, 8192, 12288, 16384):
            for R, K, sh in ((8, 8, 1), (8, 0, 0), (1, 0, 0), (16, 16, 1), (0, 12, 1), (8, 10, 1),
                             (9, 0, 0)):
                for wsb in (0, lib.fused_boundary_workspace_bytes(T, H)):
                    p = Plan()
                    rc = lib.fused_boundary_get_plan(T, H, R, K, sh, wsb, ctypes.byref(p))
                    assert rc == 0, (T, H, R, K)
                    H8 = H // 8
                    what = (T, H, R, K, sh, wsb, p.block, p.vec_per_thread, p.split, p.grid,
                            p.sources_per_batch, p.workgroups_per_cu, p.units_per_wave, p.waves)
                    assert p.block % 64 == 0 and 64 <= p.block <= 1024, what
                    assert 0 <= p.workgroups_per_cu <= 16, what
                    md, me = variant(R, K)
                    if p.units_per_wave:  # balanced kernel
                        nu = -(-H8 // 64)
                        U = T * nu
                        G, nw = p.grid, p.block // 64
                        assert p.split == nu and p.waves == G * nw and G <= U, what
                        n_max = -(-U // G)
                        assert -(-n_max // nw) <= p.units_per_wave, what
                        rows_max = (n_max + nu - 2) // nu + 1
                        assert rows_max <= 16 and rows_max * K <= 64, what
                        streamed = p.sources_per_batch != 0
                        if streamed:
                            assert p.sources_per_batch == 2 and p.units_per_wave == 1, what
                        wps = occupancy[("balanced", 0, 0, 1) if streamed
                                        else ("balanced", md, me, p.units_per_wave)]
                        wpc = p.workgroups_per_cu
                        per_cu = min(resident_wgs(wps, p.block) // 256, 2 if wpc == 1 else wpc)
                        assert G <= 256 * per_cu, ("not resident", what)
                        if nu > 1 and not (U % G == 0 and (U // G) % nu == 0):
                            assert wsb >= 256 + 512 * T, what
                        waits += 1
                        n += 1
                        continue
                    assert p.grid == T * p.split, what
                    assert p.units_per_wave == 0 and p.waves == 0, what
                    if p.sources_per_batch == 0:  # latency kernel
                        assert p.vec_per_thread == 1 and p.workgroups_per_cu == 0, what
                        assert p.block <= latency_bound(R, K), what
                        assert p.split * p.block >= H8 and (p.split - 1) * p.block < H8, what
                        assert p.split <= 32, what
                        if p.split > 1:
                            assert wsb >= 256 + 512 * T, what
                            lb = latency_bound(R, K)
                            wps = occupancy[("latency", md, me, lb)]
                            assert p.grid <= resident_wgs(wps, p.block), ("not resident", what)
                            waits += 1
                    else:  # stream kernel: whole rows
                        assert p.vec_per_thread in (1, 2, 4, 8) and p.split == 1, what
                        assert p.sources_per_batch in (1, 2, 4, 8), what
                        assert p.block * p.vec_per_thread >= H8, what
                        bound = {1: 1024, 2: 1024, 4: 512, 8: 256}[p.vec_per_thread]
                        assert p.block <= bound, what
                    n += 1
    assert n > 3000 and waits > 500


def _no_gpu():
    import torch

    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu(), reason="needs a host without a GPU: the launch must fail")
def test_launch_failure_reports_hip_error(lib):
    """With no GPU the runtime refuses the launch: both fused entry points and
    both split stages return FB_HIP_ERROR with the runtime's nonzero code in
    their own error slots.  Each check runs on a fresh thread (the slots are
    thread-local and start at 0), so no earlier failure can stand in for it.
    The fake addresses are never dereferenced: nothing can run."""
    import threading

    lib.fused_boundary_last_hip_error.restype = ctypes.c_int
    lib.fused_boundary_split_last_hip_error.restype = ctypes.c_int
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.fused_boundary_split_sum.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, vp, i32, vp, vp,
                                             i64, i64, vp, vp]
    lib.fused_boundary_split_residual_rmsnorm.argtypes = [vp, vp, vp, f32, f32, i64, i64, vp, vp, vp]
    idx, w = fake(5), fake(6)

    def fused_reduce():
        return reduce_call(lib, R=2, H=64, T=4), lib.fused_boundary_last_hip_error()

    def fused_finalize():
        arr = (ctypes.c_void_p * 1)(A + 10 * SZ)
        rc = lib.fused_moe_finalize_rmsnorm(arr, 1, fake(7), 8, idx, w, 2, None, None, fake(1),
                                            fake(2), 0.0, 1e-6, 4, 64, fake(3), fake(4), None, 0,
                                            None)
        return rc, lib.fused_boundary_last_hip_error()

    def split_sum():
        arr = (ctypes.c_void_p * 2)(A + 10 * SZ, A + 11 * SZ)
        rc = lib.fused_boundary_split_sum(arr, 2, None, 0, None, None, 0, None, None, 4, 64,
                                          fake(3), None)
        return rc, lib.fused_boundary_split_last_hip_error()

    def split_norm(H):  # H=64: through the fused reduce launch; H=60: the scalar kernel
        def f():
            rc = lib.fused_boundary_split_residual_rmsnorm(fake(10), fake(1), fake(2), 0.0, 1e-6,
                                                           4, H, fake(3), fake(4), None)
            return rc, lib.fused_boundary_split_last_hip_error()
        return f

    for f in (fused_reduce, fused_finalize, split_sum, split_norm(64), split_norm(60)):
        out = []
        th = threading.Thread(target=lambda: out.append(f()))
        th.start()
        th.join()
        rc, err = out[0]
        assert rc == 3, (f, rc)
        assert err != 0, f


def test_bandwidth_probe_validation(lib):
    """The diagnostic probe checks its arguments before any runtime call: bad
    counts, sizes, vector widths, alignment and missing buffers are refused,
    and zero tokens is a no-op that succeeds.  Fake addresses are never
    dereferenced: every case returns before a launch."""
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.fused_boundary_bandwidth_probe.argtypes = [ctypes.POINTER(vp), i32, vp, i64, vp, i32,
                                                   ctypes.POINTER(vp), i32, i64, i64, i32, i32, vp]
    ok_direct = (vp * 10)(*[A + i * SZ for i in range(10)])
    outs = (vp * 2)(A + 20 * SZ, A + 21 * SZ)

    def call(direct=ok_direct, nd=10, gathered=fake(7), n=32, idx=fake(5), k=8, outputs=outs, no=2,
             T=4, H=64, vpt=4, wgcu=3):
        return lib.fused_boundary_bandwidth_probe(direct, nd, gathered, n, idx, k, outputs, no, T, H,
                                                  vpt, wgcu, None)

    INVALID = 1
    assert call(T=0) == 0
    for kw in (dict(nd=19), dict(nd=-1), dict(k=17), dict(k=-1), dict(no=3), dict(T=-1),
               dict(T=1 << 31), dict(H=0), dict(H=60), dict(vpt=3), dict(vpt=16), dict(wgcu=17),
               dict(wgcu=-1), dict(n=-1), dict(n=0), dict(gathered=None), dict(idx=None),
               dict(gathered=fake(7, 8)), dict(outputs=None), dict(direct=None),
               dict(direct=(vp * 10)(*([A + i * SZ for i in range(9)] + [A + 9 * SZ + 4]))),
               dict(outputs=(vp * 2)(A + 20 * SZ, None)), dict(H=8 * 64 * 4 * 2 + 8, vpt=1)):
        assert call(**kw) == INVALID, kw


def test_residency_probe_validation(lib):
    """The residency probe refuses a bad SGPR level, grid, block, sleep length,
    missing or misaligned output before any runtime call (fake addresses are
    never dereferenced: every case returns before a launch)."""
    lib.fused_boundary_residency_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_uint64, ctypes.c_void_p,
                                                   ctypes.c_void_p]

    def call(level=1, grid=512, block=256, ticks=2000, out=A):
        return lib.fused_boundary_residency_probe(level, grid, block, ticks, out, None)

    for kw in (dict(level=-1), dict(level=3), dict(grid=0), dict(grid=65537), dict(block=0),
               dict(block=32), dict(block=96), dict(block=1088), dict(ticks=1000001),
               dict(out=None), dict(out=A + 4)):
        assert call(**kw) == 1, kw
