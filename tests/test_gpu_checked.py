"""The small-shape prefill parity tests and the largest-batch test again, against the
bounds-checked build of the library (libcosa_osk_checked.so, built by build() with
COSA_OSK_CHECKED), on an MI355X.

In that build the prefill kernels test the index invariants they rely on -- schedule
positions, order-mask and page-table columns, physical page ids, output rows -- and count
each violation in the workspace health word.  The tests run in one child process with the
binding pointed at the checked library and COSA_OSK_HEALTH_CHECK naming a record file,
which makes every prefill call read the health word back, require 0 and add a line to the
record (tests/conftest.py); the record shows that the checks ran.  The full-size
workloads, the mask builders (which have no such checks) and the graph-capture test (which
cannot synchronise inside a capture) are left out.
"""
import os
import re
import subprocess
import sys

import pytest

from block_sparse_long_osk_amd import build

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FILES = ["test_gpu_parity.py", "test_gpu_edges.py", "test_gpu_paging.py", "test_gpu_union.py",
         "test_gpu_block128.py", "test_gpu_unmapped_pages.py", "test_gpu_scale.py", "test_gpu_schedule.py",
         "test_gpu_limits.py"]
DESELECT = ("not full_size and not cfg1_full and not builder and not kap and not validator "
            "and not rejects")


def log(*a):
    print("[gpu-test]", *a, flush=True)


@pytest.fixture(scope="module")
def checked_env(tmp_path_factory):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib = build.CHECKED_LIB_PATH
    assert os.path.exists(lib), f"{lib} is missing: build() makes it next to libcosa_osk.so"
    env = dict(os.environ)
    record = str(tmp_path_factory.mktemp("health") / "calls.txt")
    env.update(COSA_OSK_LIBRARY=lib, COSA_OSK_HEALTH_CHECK=record)
    return env


def _run(cmd, env, timeout):
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    return res.returncode, res.stdout + res.stderr


def test_the_checked_build_is_what_runs(checked_env):
    code = ("from block_sparse_long_osk_amd import binding; binding.lib(); "
            "print(binding.LIB_PATH, binding.LIB_PATH in open('/proc/self/maps').read())")
    rc, out = _run([sys.executable, "-c", code], checked_env, 120)
    assert rc == 0, out[-4000:]
    assert out.split()[-2:] == [build.CHECKED_LIB_PATH, "True"], out[-4000:]


def test_prefill_parity_under_the_checked_build(checked_env):
    files = [os.path.join("tests", f) for f in FILES]
    log("checked library:", checked_env["COSA_OSK_LIBRARY"])
    rc, out = _run([sys.executable, "-u", "-m", "pytest", "-q", "-x", "-m", "gpu", "-p", "no:cacheprovider",
                    "--timeout", "120", "--timeout-method", "thread", "-k", DESELECT] + files, checked_env, 300)
    tail = out[-4000:]
    log(tail.strip().splitlines()[-1] if tail.strip() else "(no output)")
    assert rc == 0, tail
    m = re.search(r"(\d+) passed", out)
    assert m and " failed" not in out, tail
    passed = int(m.group(1))
    with open(checked_env["COSA_OSK_HEALTH_CHECK"]) as f:
        calls = f.read().splitlines()
    log(f"{passed} tests passed, {len(calls)} prefill calls with a zero health word")
    assert passed >= 43, tail
    assert len(calls) >= passed, "the health check did not run on every test"
