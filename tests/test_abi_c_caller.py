"""The library's C ABI from a plain C11 program (tests/c_abi_host_caller.c), built with
gcc against include/cosa_osk.h and linked to the built library: its host-only checks
pass, and the sizes and mask widths it prints are those the Python binding returns for
the same arguments.  No GPU is touched."""
import os
import shutil
import subprocess

import pytest

from block_sparse_long_osk_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or not os.path.exists(binding.LIB_PATH) or not os.path.isdir(ROCM_INCLUDE),
    reason="gcc, the ROCm headers or the built library are missing")


def test_c_program_calls_the_abi(tmp_path):
    exe = str(tmp_path / "c_abi_host_caller")
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_host_caller.c"),
           "-L", libdir, "-l:" + os.path.basename(binding.LIB_PATH), "-Wl,-rpath," + libdir, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    got = dict(line.split() for line in run.stdout.splitlines())

    dims = binding.CosaOskDims(num_seqs=1, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
                               total_q_tokens=131072, total_qblocks=2048, max_pages_per_seq=2048,
                               num_phys_pages=2048, max_mask_len=int(got["order_mask_width"]), sm_scale=0.0,
                               block_size=64, q_stride_tok=32 * 128, q_stride_head=128, o_stride_tok=32 * 128,
                               o_stride_head=128, kv_stride_page=8 * 64 * 128, kv_stride_head=64 * 128,
                               kv_stride_tok=128)
    assert int(got["workspace"]) == binding.cosa_osk_workspace_bytes(dims)
    assert int(got["builder_workspace"]) == binding.cosa_build_order_mask_workspace_bytes(dims)
    assert int(got["order_mask_width"]) == binding.cosa_order_mask_width(2048, 0.1)
    assert int(got["kap_mask_width"]) == binding.cosa_kap_mask_width(2048, binding.COSA_KAP_FRACTION, 0.1)
    assert int(got["union_mask_width"]) == binding.cosa_union_mask_width(2048, 4, 0.1)
