"""The public header is plain C: a C99 program that includes it compiles with
warnings as errors, links against the library and calls its host-side helpers
(no GPU needed: nothing here launches)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "reduce_moe_finalize_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fused_boundary.h"

int main(void) {
  fused_boundary_plan p;
  const void* parts[1] = {0};
  memset(&p, 0, sizeof p);
  if (fused_boundary_workspace_bytes(16, 7168) != 256u + 16u * 512u) return 1;
  if (fused_boundary_get_plan(16, 7168, 8, 8, 1, fused_boundary_workspace_bytes(16, 7168), &p)
      != FB_OK) return 2;
  if (p.sources_per_batch != 0 || p.split * p.block < 7168 / 8) return 3;
  /* invalid arguments are rejected on the host, before any HIP call */
  if (fused_reduce_rmsnorm(parts, 0, 0, 0, 0.0f, 1e-6f, 4, 64, 0, 0, 0, 0, 0)
      != FB_INVALID_ARGUMENT) return 4;
  printf("%s\n", fused_boundary_status_string(FB_DECLINED));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
@pytest.mark.skipif(not os.path.exists(os.path.join(LIBDIR, "libfused_boundary.so")),
                    reason="library not built")
def test_header_is_c99_and_links_from_c(tmp_path):
    src = tmp_path / "use_header.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_header"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src),
                    "-L", LIBDIR, "-lfused_boundary", f"-Wl,-rpath,{LIBDIR}"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join(
        p for p in ("/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")) if p)
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert res.returncode == 0, (res.returncode, res.stderr)
    assert "declined" in res.stdout
