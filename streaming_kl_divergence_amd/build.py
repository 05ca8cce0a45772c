"""Build the HIP library libstreamkl.so for gfx950 in this package directory.

    python -m streaming_kl_divergence_amd.build
    python -m streaming_kl_divergence_amd.build --rev REV [--out DIR]

Every source is compiled with hipcc for gfx950 only.  Packed fp32 VALU
instructions are disabled (-packed-fp32-ops) and float atomics map to the
hardware instructions (-munsafe-fp-atomics).

--rev builds the library from the sources of a git revision (with the flags
below) into DIR (default _build/rev-REV/libstreamkl.so beside this file), for
timing two builds against each other in one process (bench.py --ab).
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


def flags(include: str = os.path.join(ROOT, "include"), csrc: str = CSRC) -> list[str]:
    # -Wno-inline-asm: the LDS-DMA helper names M0 as clobbered; the kernels
    # never use M0 otherwise (checked in the generated code)
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics", "-Wno-inline-asm",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", include, "-I", csrc]


# MFMA results stay in VGPRs: the VALU reads every score, and a result in an
# AGPR would cost one v_accvgpr_read per value.  The both-settings kernels
# (bwd_both.hip) need more registers than the VGPRs hold and leave the choice
# to the compiler, which puts their gradient accumulators in AGPRs.
EXTRA = {"fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, csrc: str = CSRC, include: str = os.path.join(ROOT, "include"), build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [hipcc(), *flags(include, csrc), *EXTRA.get(src, []), "-c", os.path.join(csrc, src), "-o", obj]
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


def build_revision(rev: str, out_dir: str | None = None, verbose: bool = True) -> str:
    """libstreamkl.so from the library sources of git revision `rev` (the
    files under csrc/ and include/streamkl.h), compiled with the flags above."""
    def git(*args: str, text: bool = True):
        return subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=text, check=True).stdout
    sha = git("rev-parse", "--short=12", rev).strip()
    out_dir = out_dir or os.path.join(BUILD, f"rev-{sha}")
    src_dir, inc_dir = os.path.join(out_dir, "csrc"), os.path.join(out_dir, "include")
    os.makedirs(src_dir, exist_ok=True)
    os.makedirs(inc_dir, exist_ok=True)
    rel = os.path.relpath(CSRC, ROOT)
    for path in git("ls-tree", "--name-only", sha, rel + "/").split():
        with open(os.path.join(src_dir, os.path.basename(path)), "wb") as f:
            f.write(git("show", f"{sha}:{path}", text=False))
    with open(os.path.join(inc_dir, "streamkl.h"), "wb") as f:
        f.write(git("show", f"{sha}:include/streamkl.h", text=False))
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, src_dir, inc_dir, out_dir), SOURCES))
    lib = os.path.join(out_dir, "libstreamkl.so")
    _link(objs, lib)
    if verbose:
        print(f"built {lib} from {rev} ({sha})")
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="Build libstreamkl.so (and the probes library) for gfx950.")
    ap.add_argument("--rev", help="build the library from this git revision's sources instead")
    ap.add_argument("--out", help="output directory for --rev")
    a = ap.parse_args()
    if a.rev:
        build_revision(a.rev, a.out)
    else:
        build()
