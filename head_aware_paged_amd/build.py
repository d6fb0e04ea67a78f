"""Compile libsegkv.so (all HIP sources, gfx950) next to this file."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsegkv.so")
DEBUG_LIB = os.path.join(HERE, "libsegkv_debug.so")  # SEGKV_DEBUG: device-side bounds checks
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


# Per-source extra flags (none at present; the hook keeps a flag that one
# kernel file needs from reaching the others).
DEVICE_FLAGS = {}


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False, debug: bool = False) -> str:
    """Compile every HIP source for gfx950 (one object each, in parallel) and
    link them into one shared library; returns its path. sanitize=True builds
    the host code with ASan/UBSan (at -O1); debug=True defines SEGKV_DEBUG
    (device-side bounds checks reported as SEGKV_ERR_DEVICE_CHECK)."""
    import concurrent.futures
    import tempfile
    base = [hipcc(), "--offload-arch=gfx950", "-O1" if sanitize else "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"] + \
        (HOST_SANITIZE + ["-g"] if sanitize else []) + (["-DSEGKV_DEBUG"] if debug else [])
    tmpdir = tempfile.mkdtemp(prefix="segkv_build_")

    def compile_one(src):
        obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
        cmd = base + DEVICE_FLAGS.get(src, []) + ["-c", "-o", obj, os.path.join(CSRC, src)]
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    link = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] +
                          (HOST_SANITIZE if sanitize else []) + [o for o, _ in results],
                          capture_output=True, text=True)
    res = [r for _, r in results] + [link]
    log = "\n".join(l for r in res for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature: harmless
    shutil.rmtree(tmpdir, ignore_errors=True)
    if any(r.returncode != 0 for r in res):
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
    print(build(out=DEBUG_LIB, debug=True))
