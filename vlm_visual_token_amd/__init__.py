"""InternVL visual-token compression connector on AMD Instinct MI355X (gfx950).

The computation lives in libivc.so (C ABI in include/ivc.h, HIP kernels in
csrc/); ``ivc`` is its ctypes binding and ``Connector`` a small owner of a
handle and workspace.  Build with ``python -m vlm_visual_token_amd.build``.
"""
from . import ivc  # noqa: F401

__all__ = ["ivc", "Connector"]


def __getattr__(name):
    if name == "Connector":
        from .connector import Connector
        return Connector
    raise AttributeError(name)
