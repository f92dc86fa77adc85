"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The host side of libpkv (argument validation, split planning, the
multiplexing policy, the mux round's host logic) is rebuilt with both
sanitizers on its host code only (the gfx950 device code is compiled as
usual), and the host-only tests of the boundary run against that build in a
child process with the sanitizer runtime preloaded: an out-of-bounds access,
a use after free or undefined behaviour on those paths ends the child with a
report.  A planted heap overflow in a small library built the same way shows
that the set-up catches such a mistake.  CPU only (hipcc cross-compiles; no
call reaches a device).
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT
from decode_paged_kv_amd import build

# sanitizers for the host pass only: each flag right after -Xarch_host
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
HOST_TESTS = ["tests/test_abi_cpu.py", "tests/test_mux_policy_cpu.py", "tests/test_stall_free_cpu.py"]

PLANTED = r"""
#include <cstdlib>
extern "C" int planted_overflow(int n) {
  int* a = static_cast<int*>(std::malloc(n * sizeof(int)));
  for (int i = 0; i <= n; ++i) a[i] = i;   // one past the end
  int s = a[0];
  std::free(a);
  return s;
}
"""


def _asan_runtime():
    clang = shutil.which("clang") or "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    runtime = _asan_runtime()
    if not os.path.exists(hipcc) or runtime is None:
        pytest.skip("hipcc or the AddressSanitizer runtime is not available")
    d = tmp_path_factory.mktemp("san")

    def comp(src):
        obj = str(d / (os.path.basename(src) + ".o"))
        res = subprocess.run([hipcc, "-x", "hip", *build.HIPCC_FLAGS, *SAN_FLAGS, "-c", src, "-o", obj],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, build.sources()))
    lib = str(d / "libpkv_sanitized.so")
    res = subprocess.run([hipcc, f"--offload-arch={build.ARCH}", "-shared", "-fPIC", *SAN_FLAGS, *objs, "-o", lib],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]

    planted_src = d / "planted.cpp"
    planted_src.write_text(PLANTED)
    planted = str(d / "libplanted.so")
    res = subprocess.run([hipcc, "-x", "c++", "-O1", "-shared", "-fPIC", *SAN_FLAGS, str(planted_src), "-o", planted],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]

    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               PKV_LIB_PATH=lib)
    return env, planted


def test_planted_heap_overflow_is_reported(sanitized):
    env, planted = sanitized
    code = f"import ctypes; ctypes.CDLL({planted!r}).planted_overflow(8)"
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr


def test_host_tests_pass_against_the_sanitized_library(sanitized):
    env, _ = sanitized
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *HOST_TESTS],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
