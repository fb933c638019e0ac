"""ConvRot quantized linear on MI355X (gfx950): grouped-Hadamard rotation + INT8/INT4
quantization + integer MFMA GEMM, behind the C-ABI library ``libconvrot.so``.

Submodules are imported lazily so that ``workloads`` can be used without loading the
HIP library.
"""
import importlib

__all__ = ["convrot", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
