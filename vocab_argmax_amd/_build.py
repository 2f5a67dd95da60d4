"""Build libvpa.so (HIP, gfx950) in-tree with hipcc, and the binding's
CPython marshalling module _vpa_call with the host C compiler.

    python -m vocab_argmax_amd._build          # or: vocab_argmax_amd._build.build()

Sources are compiled in parallel into vocab_argmax_amd/_build/ and linked into
vocab_argmax_amd/libvpa.so.  Packed-fp32 instructions are disabled for the
device code (the path has no float arithmetic; the flag keeps it that way).
_vpa_call (csrc/pycall.c) does not link the library: the binding hands it the
entry points of the libvpa.so it has loaded.
"""
import os
import shutil
import subprocess
import sysconfig
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvpa.so")
SOURCES = ["api.hip", "block_stats.hip", "chunk_stats.hip", "reduce.hip"]
ARCH = "gfx950"
PYCALL = os.path.join(PKG, "_vpa_call" + sysconfig.get_config_var("EXT_SUFFIX"))


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set ROCM_PATH")


def compile_flags(extra=()):
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra]


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags(extra_flags), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        return obj

    def link(objs, out):
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
        os.replace(out + ".tmp", out)

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    link(objs, LIB)
    build_pycall(verbose)
    return LIB


def build_pycall(verbose: bool = False) -> str:
    """Compile csrc/pycall.c into the _vpa_call extension module."""
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no host C compiler (gcc / cc) for _vpa_call")
    cmd = [cc, "-O2", "-std=gnu11", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
           f"-I{sysconfig.get_paths()['include']}", f"-I{INCLUDE}",
           os.path.join(CSRC, "pycall.c"), "-o", PYCALL + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"_vpa_call failed to build:\n{res.stdout}\n{res.stderr}")
    os.replace(PYCALL + ".tmp", PYCALL)
    return PYCALL


if __name__ == "__main__":
    print(build(verbose=True))
