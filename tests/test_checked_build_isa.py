"""The bounds checks of the checked build are in every prefill kernel of it, and none of
them is in the default build: the gfx950 assembly of osk_prefill.hip, compiled as the
library compiles it, with and without COSA_OSK_CHECKED.  The prefill kernels use no
global atomic except the health-word count of a failed check, so the default build's
prefill kernels must have none and every prefill kernel of the checked build some.
(No GPU: hipcc cross-compiles.)"""
import os
import re
import subprocess
import tempfile

import pytest

from block_sparse_long_osk_amd import build


def _hipcc_available():
    try:
        build.hipcc()
        return True
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not _hipcc_available(), reason="hipcc is not installed")

KERNEL = re.compile(r"^(_ZN8cosa_osk\d+osk_prefill_(?:ring|b128)_kernel\w*):", re.M)
ATOMIC = re.compile(r"^\s+(?:global|buffer|flat)_atomic\w*", re.M)


def _atomics_per_kernel(asm):
    counts = {}
    for m in KERNEL.finditer(asm):
        end = asm.find(".Lfunc_end", m.start())
        assert end > 0
        counts[m.group(1)] = len(ATOMIC.findall(asm, m.start(), end))
    return counts


def test_checks_are_in_the_checked_build_only():
    with tempfile.TemporaryDirectory() as tmp:
        outs = {"default": os.path.join(tmp, "default.s"), "checked": os.path.join(tmp, "checked.s")}
        procs = {k: subprocess.Popen(build.device_asm_cmd("osk_prefill.hip", path,
                                                          ("COSA_OSK_CHECKED",) if k == "checked" else ()),
                                     stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
                 for k, path in outs.items()}
        for k, p in procs.items():
            log, _ = p.communicate(timeout=600)
            assert p.returncode == 0, log[-3000:]
        counts = {k: _atomics_per_kernel(open(path).read()) for k, path in outs.items()}
    assert counts["default"].keys() == counts["checked"].keys()
    assert len(counts["default"]) >= 30, sorted(counts["default"])  # 34 instantiations
    assert all(n == 0 for n in counts["default"].values()), counts["default"]
    assert all(n > 0 for n in counts["checked"].values()), counts["checked"]
