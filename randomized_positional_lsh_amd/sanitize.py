"""Host-code sanitizer run of libplpsh: AddressSanitizer and
UndefinedBehaviorSanitizer on the host C++ (argument validation, the hash
draw, the staging ring, the Lanczos driver), on the CPU.

Builds a second copy of the library under _build/asan/ in which the host
sources (api.cpp, sampler.cpp) carry -fsanitize=address,undefined on their
host compilation only (the device code is built as usual and never runs
here), then runs the C-ABI tests of tests/test_abi_cpu.py against it with
the sanitizer runtime preloaded into the Python process.  Any report aborts
the run with a non-zero status.

Usage: python randomized_positional_lsh_amd/sanitize.py
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, HERE)

import build as B  # noqa: E402

OUT = os.path.join(B.BUILD, "asan")
LIB = os.path.join(OUT, "libplpsh.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan", "-g"]


def runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm")
    return hits[-1]


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src, extra in B.SOURCES.items():
        obj = os.path.join(OUT, src + ".o")
        flags = extra + (HOST_SAN if src.endswith(".cpp") else [])
        cmd = [B.hipcc(), *B.COMMON, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-fsanitize=address,undefined", "-fno-gpu-sanitize", "-o", LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking the sanitizer build failed:\n" + r.stdout + r.stderr)
    return LIB


def main() -> int:
    lib = build()
    env = dict(os.environ)
    env["PLPSH_LIBRARY"] = lib
    env["LD_PRELOAD"] = runtime()
    # Python's own allocations are never freed at exit: leak reports off;
    # everything else (buffer overflows, use after free, undefined behaviour) aborts
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_cpu.py")]
    print("sanitizer build:", lib, flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
