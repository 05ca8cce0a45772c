"""The C ABI from plain C: a C99 program that includes include/streamkl.h and
include/streamkl_probes.h, links against both libraries and calls entry points
that are rejected before any launch (no GPU is touched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "streaming_kl_divergence_amd")

PROGRAM = r"""
#include "streamkl.h"
#include "streamkl_probes.h"
#include <stdio.h>

int main(void) {
  const void* f = (const void*)4096;   /* non-NULL and aligned, never dereferenced */
  float* o = (float*)4096;
  int a = streamkl_fwd(f, f, f, f, 16, 16, 2, 64, 0, 0.125f, STREAMKL_BF16, NULL, o, o, NULL);
  int b = streamkl_fwd(f, f, f, f, 16, 16, 2, 96, 0, 0.125f, STREAMKL_BF16, o, o, o, NULL);
  int c = streamkl_bwd_set2(f, f, f, f, 16, 16, 2, 64, 0, 0.125f, STREAMKL_FP32, o, o, NULL, NULL, o, o,
                            STREAMKL_BWD_SEPARATE, NULL, 0, NULL);
  int d = streamkl_fwd_splitk_noalloc(f, f, f, f, 1, 4096, 2, 128, 0, -1.0f, STREAMKL_BF16, 0, o, o, o, NULL);
  size_t ws = streamkl_workspace_bytes(0, 1, 4096, 2, 128, 4, STREAMKL_BWD_AUTO);
  printf("%d %d %d %d %zu %d %d\n", a, b, c, d, ws, streamkl_bwd_select(64, 131072, 32, 128, 0),
         streamkl_probe_threads());
  printf("%s\n", streamkl_strerror(a));
  return 0;
}
"""


def test_headers_compile_as_c99_and_the_libraries_link(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("no C compiler or HIP headers")
    for lib in ("libstreamkl.so", "libstreamkl_probes.so"):
        assert os.path.exists(os.path.join(PKG, lib)), f"{lib} is not built"
    src, exe = str(tmp_path / "c_abi.c"), str(tmp_path / "c_abi")
    with open(src, "w") as f:
        f.write(PROGRAM)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src, "-o", exe,
                        "-L", PKG, "-lstreamkl", "-lstreamkl_probes", f"-Wl,-rpath,{PKG}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    codes, msg = r.stdout.splitlines()
    # NULL kl; head_dim 96; Setting 2 without kl; negative scale; 4 splits x 2 heads x 1 row x 20 B;
    # AUTO resolves to the separate kernels; 256 threads per probe workgroup
    assert codes.split() == ["-1", "-3", "-1", "-4", "160", "2", "256"], r.stdout
    assert msg == "a required pointer is NULL"
