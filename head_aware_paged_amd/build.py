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


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (each flag applies to
# the host pass only; the device code is built as usual). The library then
# needs the ASan runtime preloaded into the process that loads it.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that a sanitized build must be run with."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True):
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("clang ASan runtime not found under " + root)


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile every HIP source for gfx950 into one shared library; returns its
    path. sanitize=True builds the host code with ASan/UBSan (at -O1)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O1" if sanitize else "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-result", "-o", tmp] + (HOST_SANITIZE + ["-g"] if sanitize else []) + \
        [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature: harmless
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + log)
    if verbose and log.strip():
        print(log, file=sys.stderr)
    # a kernel whose host-side stub was silently dropped links into an
    # unloadable library: refuse it here rather than at import time
    nm = subprocess.run(["nm", "-D", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if " U " in l and "device_stub" in l]
    if missing:
        raise RuntimeError("kernel launch stubs missing from libsegkv.so: " + ", ".join(missing))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
