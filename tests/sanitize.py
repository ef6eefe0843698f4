"""Host sanitizer runs of the CPU test suite.

1. The oracle (plain C) built by gcc with AddressSanitizer and
   UndefinedBehaviorSanitizer (errors fatal), loaded in place of the regular
   build through BEAM_ORACLE_LIB, under the whole `-m "not gpu"` suite.
2. The HIP library built by hipcc with the same sanitizers on its host code
   only (every flag behind -Xarch_host; the gfx950 code is compiled as
   usual), loaded through BEAM_MOE_LIB, under the tests that call its host
   entry points (descriptor validation, workspace sizing, argument errors,
   exported symbols): tests/test_abi.py.

Python itself is not instrumented, so each run preloads the sanitizer
runtime of the compiler that built the library under test (gcc's libasan,
clang's libclang_rt.asan) and turns leak detection off (the interpreter's
own allocations would be reported).  No GPU is used.

    python tests/sanitize.py          # builds under /tmp, exits non-zero on failure
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]
ENV_COMMON = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:symbolize=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _run(env_extra, args, label):
    env = dict(os.environ)
    env.update(ENV_COMMON)
    env.update(env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", *args]
    print(f"[{label}] {' '.join(f'{k}={v}' for k, v in env_extra.items())} {' '.join(cmd)}",
          flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env)
    print(f"[{label}] exit {r.returncode}", flush=True)
    return r.returncode


def main() -> int:
    from oracle import build as ob
    from group_limited_routing_sigmoid_amd import build as pb

    tmp = tempfile.mkdtemp(prefix="beam_san_")
    rc = 0

    # 1. oracle under gcc ASan + UBSan, whole CPU suite
    olib = ob.compile_to(ob.SRC, os.path.join(tmp, "libbeam_oracle_san.so"), extra=SAN,
                         verbose=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    rc |= _run({"LD_PRELOAD": libasan, "BEAM_ORACLE_LIB": olib}, ["tests"], "oracle")

    # 2. library host code under clang ASan + UBSan, the host-side ABI tests
    llib = pb.build(verbose=False, lib=os.path.join(tmp, "libbeam_moe_san.so"),
                    build_dir=os.path.join(tmp, "build"), host_flags=SAN)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        print("clang ASan runtime not found", flush=True)
        return 1
    rc |= _run({"LD_PRELOAD": rt[-1], "BEAM_MOE_LIB": llib},
               [os.path.join("tests", "test_abi.py")], "library")
    print("sanitizer runs:", "green" if rc == 0 else "FAILED", flush=True)
    return rc


if __name__ == "__main__":
    sys.exit(main())
