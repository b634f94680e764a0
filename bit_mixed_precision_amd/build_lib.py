"""Build libtq.so (host packer + HIP kernels for gfx950) in the package folder.

Run ``python -m bit_mixed_precision_amd.build_lib`` or call ``build()``.  Host
C++ is compiled with g++ (IEEE fp64, no contraction); device code with hipcc
for gfx950 only, with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wextra",
              "-I", INCLUDE, "-I", CSRC, "-pthread"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument",
             "-I", INCLUDE, "-I", CSRC]


def _sources():
    host = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    dev = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    return host, dev


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libtq.so; always rebuilds.  Returns the path."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    host, dev = _sources()
    cmds, objs = [], []
    for f in host:
        o = os.path.join(BUILD, f + ".o")
        cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in dev:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    # -z defs: a kernel whose host stub was not emitted fails here, not at load time
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-Wl,-z,defs", *objs,
          "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
