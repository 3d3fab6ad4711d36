"""Routed Mixture-of-Experts SwiGLU layer (forward) for MI355X / gfx950.

The compute lives in libmoe.so (hand-written HIP kernels behind a C ABI,
include/moe.h); `sparse_mixture_experts_12_amd.ops` is its thin Python
binding.  Importing the binding fails loudly when the library is not built.
"""
import importlib


def __getattr__(name):
    if name == "ops":
        return importlib.import_module("._lib", __name__)
    raise AttributeError(name)
