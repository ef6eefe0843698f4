"""Build libbeam_moe.so in-tree: every HIP translation unit for gfx950 with
hipcc, then one shared library.

Flags:
  -Xclang -target-feature -Xclang -packed-fp32-ops
      no packed fp32 instructions anywhere;
  -ffp-contract=off for router.hip, fp8.hip and mxfp4.hip
      the routing specification and the activation quantiser round every
      binary32 operation separately.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbeam_moe.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

SOURCES = ["api.cpp", "router.hip", "permute.hip", "experts_grouped.hip",
           "experts_stream.hip", "experts_f32.hip", "combine.hip", "fp8.hip",
           "mxfp4.hip"]
NO_CONTRACT = {"router.hip", "fp8.hip", "mxfp4.hip"}

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _host(flags):
    # host-only flags (e.g. sanitizers): each behind -Xarch_host so the GPU
    # code is compiled exactly as in the regular build
    return [f for fl in flags for f in ("-Xarch_host", fl)]


def _compile(src: str, verbose: bool, build_dir: str, host_flags=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = ["hipcc", *COMMON, *_host(host_flags)]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    if src in NO_CONTRACT:
        cmd += ["-ffp-contract=off"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    out = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if out and verbose:
        print(out)
    return obj


def build(verbose: bool = False, lib: str = None, build_dir: str = None,
          host_flags=()) -> str:
    """Compile every source and link the library (default: in-tree).  `lib`,
    `build_dir` and `host_flags` serve instrumented host builds, e.g. the
    sanitizer runs of tests/sanitize.py."""
    lib = lib or LIB
    build_dir = build_dir or BUILD
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, host_flags), SOURCES))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC",
           *_host(host_flags), "-o", lib + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
