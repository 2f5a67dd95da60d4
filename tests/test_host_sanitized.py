"""The library's host layer (argument validation, size and overflow checks,
dispatch limits, workspace sizing, error messages) built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code (the device
code is compiled as usual, uninstrumented), then driven through every CPU
test of the C ABI (tests/test_abi.py, the plain C consumer included) in a
child process with the sanitizer runtime preloaded.  No GPU is involved:
none of these calls reaches a launch."""
import glob
import os
import re
import subprocess
import sys

import pytest

import vocab_argmax_amd as vpa
from vocab_argmax_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# "-s": a sanitizer report goes to stderr, which pytest's capture would hide
CHILD = """
import sys
import pytest
import vocab_argmax_amd as vpa
vpa.LIB_PATH = sys.argv[1]
vpa._lib = None
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", sys.argv[2]]))
"""


def _asan_runtime():
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "lib", "clang")
    found = sorted(glob.glob(os.path.join(llvm, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def test_abi_checks_under_asan_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    sanitize = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"):
        sanitize += ["-Xarch_host", flag]
    objs = []
    for src in _build.SOURCES:
        obj = tmp_path / (src + ".o")
        flags = [f for f in _build.compile_flags() if f != "-O3"]
        subprocess.run([_build.hipcc(), *flags, "-O1", "-g", *sanitize, "-c",
                        os.path.join(_build.CSRC, src), "-o", str(obj)], check=True,
                       capture_output=True)
        objs.append(str(obj))
    lib = tmp_path / "libvpa.so"                 # the name the C consumer test links with
    # the runtime's directory as the library's run path, so that the C
    # consumer's link step (gcc) finds the library's sanitizer dependency
    subprocess.run([_build.hipcc(), f"--offload-arch={_build.ARCH}", "-shared", "-fPIC",
                    "-shared-libasan", *sanitize[:4], *objs,
                    f"-Wl,-rpath,{os.path.dirname(runtime)}", "-o", str(lib)], check=True,
                   capture_output=True)
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               PYTHONPATH=os.pathsep.join([ROOT, HERE, os.environ.get("PYTHONPATH", "")]))
    res = subprocess.run([sys.executable, "-c", CHILD, str(lib), os.path.join(HERE, "test_abi.py")],
                         capture_output=True, text=True, env=env, timeout=900, cwd=ROOT)
    out = res.stdout + res.stderr
    reports = [ln for ln in out.splitlines()
               if "runtime error" in ln or "ERROR: AddressSanitizer" in ln or "SUMMARY:" in ln]
    assert not reports, "\n".join(reports[:20])
    assert res.returncode == 0, out[-4000:]
    passed = re.search(r"(\d+) passed", res.stdout)
    assert passed and int(passed.group(1)) >= 40 and "failed" not in res.stdout, \
        res.stdout[-2000:]
    # the child really loaded the sanitized build
    assert str(lib) != vpa.LIB_PATH
