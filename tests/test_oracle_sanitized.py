"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
every pin cleanly (CPU only; the sanitizer runtimes are preloaded into a
child Python process)."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    src = os.path.join(os.path.dirname(oracle.__file__), "vpa_ref.c")
    lib = tmp_path / "liboracle_asan.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=gnu99", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared",
                    "-fPIC", src, "-o", str(lib)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", LD_PRELOAD=f"{asan} {ubsan}")
    res = subprocess.run([sys.executable, os.path.join(HERE, "pin_runner.py"), str(lib)],
                         capture_output=True, text=True, env=env, timeout=900)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = res.stdout.split("\n")
    assert all(ln.startswith("ok ") for ln in lines if ln.strip()), res.stdout
    assert sum(1 for ln in lines if ln.startswith("ok ")) >= 12
