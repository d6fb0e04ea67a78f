"""CPU: the library's host code (layout validation, planning, argument checks)
under AddressSanitizer and UndefinedBehaviorSanitizer. A sanitized build of
libsegkv goes to a temporary directory, and the ABI and plan-size tests run
against it in a child process with the ASan runtime preloaded; any report
aborts that process. No GPU is touched: every call in those tests returns on
the host."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

hb = pytest.importorskip("head_aware_paged_amd.build")


def test_abi_under_asan_ubsan(tmp_path):
    try:
        hb.hipcc()
        rt = hb.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = hb.build(out=str(tmp_path / "libsegkv_asan.so"), sanitize=True)
    env = dict(os.environ, SEGKV_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_plan_sizes.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(res.stdout[-3000:], res.stderr[-3000:])
    assert res.returncode == 0
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr
