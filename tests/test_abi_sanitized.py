"""The C ABI's host-side code (argument validation, workspace sizing, the
segment plans, the allocation-free entry point's size check) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

abi.cpp and noalloc.cpp are compiled with the sanitizers on their host code
only (-Xarch_host; the gfx950 device code is untouched) and linked with the
library's other objects into a separate copy of the library; the host ABI
tests (tests/test_abi_host.py, error paths only: nothing is launched) then run
against that copy with the sanitizer runtime preloaded.  Any finding aborts
the run and fails this test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "state_space_sequence_03_amd", "csrc")


def test_abi_host_checks_under_sanitizers(tmp_path):
    from state_space_sequence_03_amd import build
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts or not os.path.exists(build.hipcc()):
        pytest.skip("no hipcc or no sanitizer runtime in this image")
    others = [os.path.join(build.BUILD, os.path.splitext(s)[0] + ".o") for s in build.SOURCES
              if s not in ("abi.cpp", "noalloc.cpp")]
    if not all(os.path.exists(o) for o in others):
        build.build(verbose=False)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    for src in ("abi.cpp", "noalloc.cpp"):
        obj = str(tmp_path / (src + ".o"))
        flags = [f for f in build.FLAGS if f != "-O3"] + ["-O1", "-g"]
        r = subprocess.run([build.hipcc()] + flags + san + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    lib = str(tmp_path / "libmamba3_ssm.so")
    r = subprocess.run([build.hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC"] + san[:4] +
                       ["-shared-libsan", "-o", lib] + objs + others, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_PRELOAD=rts[-1], M3_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    # the sanitized copy is the one the binding loads
    probe = ("from state_space_sequence_03_amd import ops; ops.lib(); "
             "m = open('/proc/self/maps').read(); "
             f"assert {lib!r} in m and 'libclang_rt.asan' in m, 'sanitized library not loaded'")
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
