"""MI355X-native ordered-skipping block-sparse prefill attention.

The computation lives in libcosa_osk.so (HIP kernels for gfx950 behind a C ABI,
declared in include/cosa_osk.h); `binding` exposes its entry points under the
same names, `runner` uploads inputs and allocates outputs with torch, and
`inputs` draws the seeded synthetic workloads.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "binding", "runner"]


def __getattr__(name):
    if name in ("binding", "runner", "build"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
