"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU): every source of libnsa.so is compiled again
with the sanitizers on its host code only (the gfx950 device code is built as
usual and never runs here), and tests/test_abi_host.py, which drives the
argument validation, workspace planning and status strings of every entry
point with no GPU, runs in a child process against that library with the
sanitizer runtime preloaded.  A memory error or undefined operation (an
out-of-range enum, a signed overflow in a size check) aborts the child with a
report; the test requires a clean, passing run.  The build (about a minute)
is kept in _build/asan and redone only when a source or header changes."""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

from long_context_dynamic_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libnsa_sanitized.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        return None
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _sources():
    return sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))


def _stale():
    if not os.path.exists(LIB):
        return True
    deps = _sources() + glob.glob(os.path.join(B.CSRC, "*.h")) + glob.glob(os.path.join(B.INCLUDE, "*.h"))
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(LIB)


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    r = subprocess.run([B.HIPCC, *B.CFLAGS, *SAN, "-c", src, "-o", obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return obj


def _build():
    os.makedirs(OUT, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", LIB + ".tmp"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    os.replace(LIB + ".tmp", LIB)


RUNNER = """
import sys
sys.path.insert(0, sys.argv[1])
from long_context_dynamic_amd import nsa
nsa._LIB_PATH = sys.argv[2]          # the sanitized build in place of libnsa.so
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", sys.argv[3]]))
"""


@pytest.mark.skipif(not os.path.exists(B.HIPCC) or _runtime() is None, reason="hipcc or the ASan runtime missing")
def test_host_library_is_clean_under_address_and_ub_sanitizers():
    if _stale():
        _build()
    env = dict(os.environ, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0",  # the interpreter and torch keep memory to the end
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", RUNNER, ROOT, LIB, os.path.join(ROOT, "tests", "test_abi_host.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    print(r.stdout[-2000:])
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout
