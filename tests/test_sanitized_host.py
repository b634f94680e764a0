"""The host code of libtq.so under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the sanitizer variant of the library (host C++ and the host side of the
HIP sources instrumented, device code unchanged) and runs the CPU tests of the
packers and of the C ABI against it in a child process with clang's ASan
runtime preloaded.  Any out-of-bounds access, use after free or undefined
behaviour (signed overflow, bad shift, misaligned access ...) aborts the child.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_packers_and_abi_under_sanitizers():
    sys.path.insert(0, ROOT)
    from bit_mixed_precision_amd import build_lib
    lib = build_lib.build(sanitize=True)
    env = build_lib.sanitizer_env()
    out = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_pack.py"), os.path.join(ROOT, "tests", "test_abi.py")],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = out.stdout[-3000:] + out.stderr[-3000:]
    assert out.returncode == 0, tail
    assert "passed" in out.stdout and "ERROR: AddressSanitizer" not in out.stderr, tail
    assert "runtime error" not in out.stderr, tail  # UBSan reports
    # the child really ran the instrumented build
    probe = subprocess.run(
        [sys.executable, "-c", "import bit_mixed_precision_amd.binding as b; print(b._LIB_PATH)"],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.stdout.strip() == lib, probe.stdout + probe.stderr
