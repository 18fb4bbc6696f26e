"""Host-only build of the C ABI layer under AddressSanitizer and
UndefinedBehaviorSanitizer.

Compiles causal_linear_attention_02_amd/csrc/la_api.cpp (the library's
validation, planning and workspace carving) with tests/sanitize/abi_stubs.cpp
(dispatchers that launch nothing) into _build/sanitize/liblinattn_abi_asan.so.
The sanitizers instrument host code only: each sanitizer flag is passed to
the host pass alone. Test infrastructure; tests/test_abi_sanitized.py runs
tests/test_abi.py against the result.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "causal_linear_attention_02_amd")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "liblinattn_abi_asan.so")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"

HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The clang AddressSanitizer runtime that the built library needs preloaded."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-shared-libsan", *HOST_SANITIZE,
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(PKG, 'csrc')}",
           os.path.join(PKG, "csrc", "la_api.cpp"), os.path.join(HERE, "abi_stubs.cpp"), "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{r.stdout}\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
