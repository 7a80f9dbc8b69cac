"""Build libcosa_osk.so (HIP kernels for gfx950 + the C-ABI layer) in-tree with hipcc.

    python -m block_sparse_long_osk_amd.build
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libcosa_osk.so")
SOURCES = ["osk_prefill.hip", "mask_builder.hip", "kap.hip", "api.cpp"]
# measurement-only microbenchmarks (attainable MFMA and HBM read rates), a library of their own
CALIB_LIB_PATH = os.path.join(PKG, "libcosa_calib.so")
CALIB_SOURCES = ["calib.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link both shared libraries; returns the
    attention library's path."""
    _link(SOURCES, LIB_PATH, verbose)
    _link(CALIB_SOURCES, CALIB_LIB_PATH, verbose)
    return LIB_PATH


def _link(sources, lib_path, verbose):
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU forms stay off in all device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA results in VGPRs: the softmax reads S with plain VALU ops and AGPRs
           # serve as spill space instead of holding S and O behind copy instructions
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in sources]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib_path)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
