"""TANGO / WANGO gated-aggregation block forward on MI355X (gfx950).

The compute lives in libtango.so (hand-written HIP kernels behind the C ABI of
include/tango.h); this package holds its Python binding, the seeded workload
generator and the build script.
"""
from . import workload  # noqa: F401
from ._lib import TangoError, LIB_PATH, EXPORTS  # noqa: F401

__all__ = ["workload", "TangoError", "LIB_PATH", "EXPORTS", "api"]


def __getattr__(name):
    # the binding imports torch; load it on first use
    if name == "api":
        import importlib
        return importlib.import_module(".api", __name__)
    raise AttributeError(name)
