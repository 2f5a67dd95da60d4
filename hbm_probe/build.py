"""Build hbm_probe/libvpa_probe.so (HIP, gfx950) from hbm_probe/read_probe.hip.

    python -m hbm_probe.build          # or: hbm_probe.build.build()

The probe is a measurement aid of the benchmark, built with the same hipcc
flags as the argmax library but into its own shared object.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "read_probe.hip")
LIB = os.path.join(HERE, "libvpa_probe.so")


def build(verbose: bool = False) -> str:
    from vocab_argmax_amd import _build as lib_build
    obj = os.path.join(HERE, "read_probe.o")
    cmd = [lib_build.hipcc(), *lib_build.compile_flags([f"-I{HERE}"]), "-c", SRC, "-o", obj]
    link = [lib_build.hipcc(), f"--offload-arch={lib_build.ARCH}", "-shared", "-fPIC", obj,
            "-o", LIB + ".tmp"]
    for c in (cmd, link):
        if verbose:
            print(" ".join(c), flush=True)
        res = subprocess.run(c, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed:\n{res.stdout}\n{res.stderr}")
    os.replace(LIB + ".tmp", LIB)
    os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
