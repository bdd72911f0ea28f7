"""Build libmoe.so (gfx950 only) in-tree with hipcc.

    python -m quantized_moe_routed_router_amd.build   [-j N] [--verbose]
    python -m quantized_moe_routed_router_amd.build --host-sanitized DIR

Every source under csrc/ is compiled to an object in _build/ and linked into
quantized_moe_routed_router_amd/libmoe.so.  Always rebuilds.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=fast-honor-pragmas",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build: the host code of every source (argument
# validation, workspace carving, launch set-up) with AddressSanitizer and
# UndefinedBehaviorSanitizer; the device code is built as usual, without
# them.  Each -fsanitize= applies to the host pass only.
SANITIZE_HOST = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime that the sanitized library needs
    preloaded into the (uninstrumented) interpreter."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found (hipcc printed {path!r})")
    return path


def build_host_sanitized(out_dir: str, jobs: int = 8) -> str:
    os.makedirs(out_dir, exist_ok=True)
    flags = [*FLAGS, "-g", *SANITIZE_HOST]

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host, sanitized) failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(one, sources()))
    lib = os.path.join(out_dir, "libmoe_host_sanitized.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *SANITIZE_HOST, "-shared-libsan",
                        *objs, "-o", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}{r.stderr}")
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--host-sanitized", metavar="DIR",
                    help="instead: the host code only, with ASan + UBSan, into DIR")
    a = ap.parse_args(argv)
    if a.host_sanitized:
        print(build_host_sanitized(a.host_sanitized, a.j))
    else:
        print(build(a.j, a.verbose))


if __name__ == "__main__":
    main()
