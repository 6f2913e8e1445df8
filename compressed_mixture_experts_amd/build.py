"""Build the HIP libraries (gfx950 only) in-tree with hipcc.

    python -m compressed_mixture_experts_amd.build [--jobs N] [--no-host-sanitize]

Outputs, next to this file:
  libbmoe.so          the product library (include/bmoe.h, bmoe_trace.h, bmoe_grad.h,
                      bmoe_train.h)
  libbmoe_debug.so    the same plus the test hooks of include/bmoe_debug.h
                      (api.hip compiled with -DBMOE_DEBUG_EXPORTS)
  libbmoe_hostsan.so  the debug library with its host code (argument checks,
                      planning, packing) built under AddressSanitizer and
                      UndefinedBehaviorSanitizer; the device code is unchanged.
                      Used only by the CPU ABI tests, run with the sanitizer
                      runtime preloaded (tests/test_abi_sanitized.py).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbmoe.so")
LIB_DEBUG = os.path.join(PKG, "libbmoe_debug.so")
LIB_HOSTSAN = os.path.join(PKG, "libbmoe_hostsan.so")
# kernels and their host launchers, shared by every library
KERNEL_SOURCES = ["route.hip", "gemm.hip", "butterfly.hip", "butterfly_in.hip", "butterfly_mid.hip",
                  "butterfly_out.hip", "fused.hip", "fused_mfma.hip", "prep.hip", "gemm_fp4.hip",
                  "butterfly_split.hip", "butterfly_bwd.hip", "substrate_grad.hip", "combine_bwd.hip",
                  "router_bwd.hip", "gelu_bwd.hip", "butterfly_rot.hip", "train.hip"]
DEBUG_SOURCES = ["butterfly_dbg.hip"]   # kernels reached only from the test hooks

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # never emit packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# host-only sanitizers: each flag goes to the host compilation alone
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(job) -> str:
    src, obj, extra = job
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(out: str, objs, extra=()) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stderr}")
    os.replace(tmp, out)


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime hipcc's clang links against (to
    preload into an uninstrumented interpreter), or '' when absent."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else ""


def build(jobs: int = 8, verbose: bool = False, host_sanitize: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    obj = lambda name: os.path.join(BUILD, name)  # noqa: E731
    jobs_list = [(s, obj(os.path.splitext(s)[0] + ".o"), []) for s in KERNEL_SOURCES + DEBUG_SOURCES]
    jobs_list.append(("api.hip", obj("api.o"), []))
    jobs_list.append(("api.hip", obj("api_debug.o"), ["-DBMOE_DEBUG_EXPORTS"]))
    if host_sanitize:
        jobs_list.append(("api.hip", obj("api_hostsan.o"), ["-DBMOE_DEBUG_EXPORTS", *HOST_SANITIZE]))
    # the api objects first: they take longest
    jobs_list.sort(key=lambda j: not j[0].startswith("api"))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_compile, jobs_list))
    kern = [obj(os.path.splitext(s)[0] + ".o") for s in KERNEL_SOURCES]
    dbg = [obj(os.path.splitext(s)[0] + ".o") for s in DEBUG_SOURCES]
    _link(LIB, [obj("api.o"), *kern])
    _link(LIB_DEBUG, [obj("api_debug.o"), *kern, *dbg])
    if host_sanitize:
        _link(LIB_HOSTSAN, [obj("api_hostsan.o"), *kern, *dbg],
              ["-Xarch_host", "-fsanitize=address,undefined", "-shared-libsan"])
    if verbose:
        print(f"built {LIB}, {LIB_DEBUG}" + (f", {LIB_HOSTSAN}" if host_sanitize else ""))
    return LIB


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--no-host-sanitize", action="store_true",
                    help="skip libbmoe_hostsan.so (the sanitized host build for the CPU ABI tests)")
    args = ap.parse_args()
    build(args.jobs, verbose=True, host_sanitize=not args.no_host_sanitize)
    return 0


if __name__ == "__main__":
    sys.exit(main())
