"""Compile the CPU oracle (oracle/vpa_ref.c) into oracle/libvpa_ref.so with gcc.

Test infrastructure only: the oracle is the checker, never the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "vpa_ref.c")
LIB = os.path.join(HERE, "libvpa_ref.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB, strict: bool = True) -> str:
    # -fno-fast-math and no -ffinite-math: the oracle relies on IEEE NaN
    # comparisons; -O2 keeps the scalar loops fast enough for the CPU baseline.
    tmp = f"{lib}.{os.getpid()}.tmp"   # concurrent builders never share a temporary
    cmd = ["gcc", "-O2", "-std=gnu99", "-Wall", "-Wextra", "-fno-fast-math",
           "-shared", "-fPIC", src, "-o", tmp] + (["-Werror"] if strict else [])
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
