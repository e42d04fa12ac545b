"""Builds libfpd.so (the C-ABI library of hand-written gfx950 kernels) in
place, next to the Python binding.  Every source is compiled as HIP for
gfx950 only; packed fp32 arithmetic is disabled for device code."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
SOURCES = ["api.cpp", "layout.cpp", "gemm.hip", "attention.hip", "elementwise.hip", "lmhead.hip",
           "accept.hip", "codec.hip", "profile.cpp"]
OUT = os.path.join(PKG, "libfpd.so")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


FLAGS = ["-x", "hip", "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-ffp-contract=fast-honor-pragmas"]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *FLAGS, "-c", os.path.join(HERE, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libfpd.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
