"""Compile libsegkv.so (all HIP sources, gfx950) next to this file."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsegkv.so")
SOURCES = ["host.hip", "pages.hip", "relocate.hip", "attention.hip", "decode.hip", "importance.hip", "ffn.hip",
           "dense.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsegkv)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 into one shared library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-result", "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature: harmless
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out, file=sys.stderr)
    # a kernel whose host-side stub was silently dropped links into an
    # unloadable library: refuse it here rather than at import time
    nm = subprocess.run(["nm", "-D", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if " U " in l and "device_stub" in l]
    if missing:
        raise RuntimeError("kernel launch stubs missing from libsegkv.so: " + ", ".join(missing))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
