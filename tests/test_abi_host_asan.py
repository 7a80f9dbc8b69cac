"""The host-only ABI tests again, against a build of the library whose host code is
compiled with AddressSanitizer (no GPU: only argument checks and status codes run).

The sanitizer build goes to _build/asan (rebuilt when a source is newer); the tests
run in a child process with the compiler's ASan runtime preloaded and the binding
pointed at that build, and any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

from block_sparse_long_osk_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc_available():
    try:
        build.hipcc()
        build.asan_runtime()
        return True
    except (RuntimeError, OSError):
        return False


pytestmark = pytest.mark.skipif(not _hipcc_available(), reason="hipcc or its ASan runtime is not installed")


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    srcs += [os.path.join(build.INCLUDE, f) for f in os.listdir(build.INCLUDE)]
    return any(os.path.getmtime(f) > t for f in srcs)


@pytest.fixture(scope="module")
def asan_env():
    lib = build.ASAN_LIB_PATH
    if _stale(lib):
        build.build_host_asan()
    env = dict(os.environ)
    env.update(COSA_OSK_LIBRARY=lib, LD_PRELOAD=build.asan_runtime(),
               # the interpreter itself is not instrumented and keeps its allocations
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    return env


def _run(cmd, env):
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    return res.returncode, out


def test_host_abi_checks_under_asan(asan_env):
    rc, out = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                    os.path.join("tests", "test_abi_host.py")], asan_env)
    assert rc == 0, out[-4000:]
    assert " passed" in out


def test_the_sanitized_build_is_what_runs(asan_env):
    code = ("from block_sparse_long_osk_amd import binding; binding.lib(); "
            "maps = open('/proc/self/maps').read(); "
            "print('asan' if 'libclang_rt.asan' in maps else 'no-asan', binding.LIB_PATH in maps)")
    rc, out = _run([sys.executable, "-c", code], asan_env)
    assert rc == 0, out
    assert out.split()[-2:] == ["asan", "True"], out
