"""Build libtq.so (host packer + HIP kernels for gfx950) in the package folder.

Run ``python -m bit_mixed_precision_amd.build_lib`` or call ``build()``.  Host
C++ is compiled with g++ (IEEE fp64, no contraction); device code with hipcc
for gfx950 only, with packed-fp32 instructions disabled.

``build(sanitize=True)`` (``--sanitize``) writes a checking variant to
``_build/sanitize/libtq.so`` instead: the host C++ and the host side of every
HIP source (argument checks, kernel choice, launches) built with AddressSanitizer
and UndefinedBehaviorSanitizer by clang (so that one sanitizer runtime serves
both), device code unchanged.  Load it with the environment variable
``TQ_LIBRARY`` pointing at it and clang's ASan runtime preloaded
(``sanitizer_env()`` gives both).
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
SAN_BUILD = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libtq.so")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]

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


def _hip_san_flags():
    # host side only: each -fsanitize= right after -Xarch_host, device code untouched
    out = []
    for f in SAN_FLAGS:
        out += ["-Xarch_host", f]
    return out


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every source and link libtq.so; always rebuilds.  Returns the path
    (the sanitizer variant's when ``sanitize``)."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out_dir = SAN_BUILD if sanitize else BUILD
    os.makedirs(out_dir, exist_ok=True)
    host, dev = _sources()
    cmds, objs = [], []
    for f in host:
        o = os.path.join(out_dir, f + ".o")
        if sanitize:
            cmds.append([CLANGXX, *HOST_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        else:
            cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in dev:
        o = os.path.join(out_dir, f + ".o")
        extra = _hip_san_flags() if sanitize else []
        cmds.append([HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    target = SAN_LIB if sanitize else LIB
    tmp = target + ".tmp"
    if sanitize:
        # the sanitizer runtime comes from the preloaded library at run time,
        # so its symbols stay undefined here (no -z defs)
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp])
    else:
        # -z defs: a kernel whose host stub was not emitted fails here, not at load time
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-Wl,-z,defs",
              *objs, "-o", tmp])
    os.replace(tmp, target)
    if verbose:
        print("built", target)
    return target


def sanitizer_env(base=None) -> dict:
    """Environment that loads the sanitizer variant: TQ_LIBRARY, clang's ASan
    runtime preloaded (it carries the UBSan handlers too), leak checks off
    (the Python interpreter keeps its allocations until exit)."""
    import glob
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise RuntimeError("clang's ASan runtime not found under /opt/rocm/llvm")
    env = dict(os.environ if base is None else base)
    env.update({"TQ_LIBRARY": SAN_LIB, "LD_PRELOAD": rt[-1],
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    return env


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv, sanitize="--sanitize" in sys.argv)
