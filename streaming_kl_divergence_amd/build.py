"""Build the HIP library libstreamkl.so for gfx950 in this package directory.

    python -m streaming_kl_divergence_amd.build

Every source is compiled with hipcc for gfx950 only.  Packed fp32 VALU
instructions are disabled (-packed-fp32-ops) and float atomics map to the
hardware instructions (-munsafe-fp-atomics).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libstreamkl.so")
SOURCES = ["fwd.hip", "bwd.hip", "bwd_both.hip", "api.cpp"]
# calibration probes (bench.py --calibrate), a library of their own
PROBES_LIB = os.path.join(PKG, "libstreamkl_probes.so")
PROBES_SOURCES = ["probes.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def flags() -> list[str]:
    # -Wno-inline-asm: the LDS-DMA helper names M0 as clobbered; the kernels
    # never use M0 otherwise (checked in the generated code)
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics", "-Wno-inline-asm",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# MFMA results stay in VGPRs: the VALU reads every score, and a result in an
# AGPR would cost one v_accvgpr_read per value.  The both-settings kernels
# (bwd_both.hip) need more registers than the VGPRs hold and leave the choice
# to the compiler, which puts their gradient accumulators in AGPRs.
EXTRA = {"fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that note is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBES_SOURCES
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBES_SOURCES], PROBES_LIB)
    if verbose:
        print(f"built {LIB} and {PROBES_LIB}")
    return LIB


if __name__ == "__main__":
    build()
