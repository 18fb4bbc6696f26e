"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/sanitize/build_abi_sanitized.py builds la_api.cpp (validation,
planning, workspace carving) with stub dispatchers that launch nothing, its
host code instrumented. tests/test_abi.py then runs against that build in a
child process with the sanitizer runtime preloaded; any report fails it.
"""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))

import build_abi_sanitized as sb  # noqa: E402

pytestmark = pytest.mark.skipif(shutil.which(sb.HIPCC) is None and not os.path.exists(sb.HIPCC),
                                reason="hipcc not available")

PROBE = r"""
import ctypes, os
import causal_linear_attention_02_amd as la
assert la.library_path == os.environ["LINATTN_LIBRARY"], la.library_path
ctypes.CDLL(None).__asan_init          # the runtime is in the process
print("sanitized ABI library loaded")
"""


def _env(lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=sb.runtime(), LINATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_abi_suite_is_sanitizer_clean():
    lib = sb.build()
    env = _env(lib)
    root = os.path.dirname(HERE)
    p = subprocess.run([sys.executable, "-c", PROBE], cwd=root, env=env, capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0 and "sanitized ABI library loaded" in p.stdout, p.stdout + p.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], cwd=root, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
