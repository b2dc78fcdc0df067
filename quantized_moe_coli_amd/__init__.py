"""colibrì routed-expert MoE layer on MI355X (gfx950).

``quantized_moe_coli_amd.binding`` is the thin Python binding over the C-ABI
library ``libcoli_moe.so`` (HIP kernels for gfx950); it fails loudly if the
library is not built.  ``quantized_moe_coli_amd.inputs`` holds the seeded
synthetic input generators.  Attribute access on the package (for example
``quantized_moe_coli_amd.coli_moe_forward``) loads the binding on first use.
"""
import importlib

__version__ = "0.1.0"
_SUBMODULES = ("binding", "inputs", "build")


def __getattr__(name):
    if name in _SUBMODULES:
        return importlib.import_module("." + name, __name__)
    if name.startswith("__"):
        raise AttributeError(name)
    return getattr(importlib.import_module(".binding", __name__), name)
