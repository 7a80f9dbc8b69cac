"""Build libcosa_osk.so (HIP kernels for gfx950 + the C-ABI layer) in-tree with hipcc.

    python -m block_sparse_long_osk_amd.build               # the library, its checked variant, the calibration one
    python -m block_sparse_long_osk_amd.build --host-asan   # host-sanitizer build under _build/asan
    python -m block_sparse_long_osk_amd.build --checked     # the bounds-checked library alone
"""
import concurrent.futures
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
# Bounds-checked variant of the attention library (same sources and ABI, built with
# COSA_OSK_CHECKED): the prefill kernels test their index invariants -- schedule
# positions, mask and page-table columns, physical page ids, output rows -- and count each
# violation in the workspace health word.  Load it in place of the default library by
# pointing COSA_OSK_LIBRARY at it.
CHECKED_LIB_PATH = os.path.join(PKG, "libcosa_osk_checked.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the attention library, its bounds-checked
    variant and the calibration library (three hipcc processes side by side); returns the
    attention library's path."""
    jobs = [(SOURCES, LIB_PATH, {}), (SOURCES, CHECKED_LIB_PATH, {"extra": ["-DCOSA_OSK_CHECKED"]}),
            (CALIB_SOURCES, CALIB_LIB_PATH, {})]
    with concurrent.futures.ThreadPoolExecutor(len(jobs)) as pool:
        futs = [pool.submit(_link, src, lib, verbose, **kw) for src, lib, kw in jobs]
        for f in futs:
            f.result()
    return LIB_PATH


# Host AddressSanitizer build of the attention library, for the host-only ABI tests
# (argument checks and status codes; no kernel is launched from it).  The device code
# is compiled as usual; only the host side is instrumented.
ASAN_LIB_PATH = os.path.join(ROOT, "_build", "asan", "libcosa_osk.so")


def asan_runtime() -> str:
    """The compiler's ASan runtime, to be preloaded into the process that loads the
    host-sanitizer build."""
    base = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("the compiler's ASan runtime was not found")


def build_host_asan(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(ASAN_LIB_PATH), exist_ok=True)
    _link(SOURCES, ASAN_LIB_PATH, verbose, opt="-O1",
          extra=["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"])
    return ASAN_LIB_PATH


def build_checked(verbose: bool = False) -> str:
    _link(SOURCES, CHECKED_LIB_PATH, verbose, extra=["-DCOSA_OSK_CHECKED"])
    return CHECKED_LIB_PATH


# code-generation flags of every device compile
DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-std=c++17",
    # packed fp32 VALU forms stay off in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax reads S with plain VALU ops and AGPRs
    # serve as spill space instead of holding S and O behind copy instructions
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # the page gathers set M0 (the LDS destination of global_load_lds) inside inline
    # assembly and list it as clobbered on purpose; the compiler warns about every
    # inlined copy of that statement
    "-Wno-inline-asm",
]


def device_asm_cmd(source, out_path, defines=()):
    """The hipcc command that writes the gfx950 assembly of one source file, compiled
    exactly as in the library (for inspecting what a build contains)."""
    return ([hipcc(), "-O3"] + DEVICE_FLAGS + ["--cuda-device-only", "-S", "-Wno-unused-result",
                                               "-I", INCLUDE, "-I", CSRC]
            + ["-D" + d for d in defines] + [os.path.join(CSRC, source), "-o", out_path])


def _link(sources, lib_path, verbose, opt="-O3", extra=()):
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), opt] + DEVICE_FLAGS + ["-fPIC", "-shared", "-Wno-unused-result", "-I", INCLUDE,
                                           "-I", CSRC] + list(extra)
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
    if "--host-asan" in sys.argv:
        print(build_host_asan(verbose="-v" in sys.argv))
    elif "--checked" in sys.argv:
        print(build_checked(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
