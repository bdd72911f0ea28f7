"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU).

The host pass of every source is rebuilt with both sanitizers into a
temporary directory (no device code: nothing in that library can launch a
kernel), and a child interpreter with the ASan runtime preloaded runs every
check of tests/test_abi_host.py against it: the argument validation and its
error messages, the size queries, the tiling rule, the capacity verdict, the
zero-sized calls and the no-allocation entry's refusals.  Any invalid access,
overflow or undefined operation in that host code ends the child with a
sanitizer report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
import ctypes, os, sys
sys.path.insert(0, os.environ["MOE_ROOT"])
assert hasattr(ctypes.CDLL(None), "__asan_report_load8")      # the runtime is live in this process
import quantized_moe_routed_router_amd as m
m.LIB_PATH = os.environ["MOE_SANITIZED_LIB"]
assert m.lib()._name == m.LIB_PATH
from tests import test_abi_host as t
names = sorted(n for n in dir(t) if n.startswith("test_"))
for n in names:
    getattr(t, n)()
    print("passed", n, flush=True)
assert "torch" not in sys.modules
print("host checks passed:", len(names), flush=True)
"""


def _have_hipcc():
    from quantized_moe_routed_router_amd import build
    return os.path.exists(build.HIPCC) or shutil.which(build.HIPCC) is not None


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc is not installed")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    from quantized_moe_routed_router_amd import build
    lib = build.build_host_sanitized(str(tmp_path))
    # the library really is instrumented: it calls into both runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms
    env = dict(os.environ, MOE_ROOT=ROOT, MOE_SANITIZED_LIB=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([sys.executable, "-c", DRIVER], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    report = r.stdout[-3000:] + r.stderr[-6000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    n = sum(1 for l in r.stdout.splitlines() if l.startswith("passed test_"))
    assert n >= 7 and f"host checks passed: {n}" in r.stdout, report
