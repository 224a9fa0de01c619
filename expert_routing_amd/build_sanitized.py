"""Host-sanitized build of the library for CPU tests of the ABI layer's validation.

    python expert_routing_amd/build_sanitized.py

abi.hip (argument checks, exact capacity, sizing, workspace layout, the replica plan) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (each
-fsanitize flag goes to the host compilation through -Xarch_host; the kernels are built as
usual) and linked with the normal objects of the other sources into
_build/libmoe_san.so. The sanitizer runtime is not linked into the Python interpreter, so a
process that loads this library preloads it: see runtime_env().
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import build as B  # noqa: E402

OUT = os.path.join(B.BUILD_DIR, "libmoe_san.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime_library() -> str | None:
    """Path of the ASan runtime (with the UBSan handlers) of the ROCm clang, or None."""
    clang = os.path.join(os.path.dirname(B.HIPCC), "..", "lib", "llvm", "bin", "clang")
    try:
        r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                           capture_output=True, text=True)
    except OSError:
        return None
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def runtime_env(lib: str = OUT) -> dict:
    """Environment for a child process that loads the sanitized library."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime_library() or ""
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["EXPERT_ROUTING_AMD_LIB"] = lib
    return env


def build_sanitized(verbose: bool = False) -> str:
    B.build()   # the other sources' objects, up to date
    obj = os.path.join(B.BUILD_DIR, "abi_san.o")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    r = subprocess.run([B.HIPCC, *flags, "-c", os.path.join(B.CSRC, "abi.hip"), "-o", obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on abi.hip:\n{r.stderr}")
    objs = [obj] + [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o")
                    for s in B.SOURCES if s != "abi.hip"]
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN,
                        "-Xarch_host", "-shared-libsan", *objs, "-o", OUT],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build_sanitized(verbose=True)
