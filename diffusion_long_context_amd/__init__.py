"""MI355X (gfx950) chunk-sparse attention path of Prefilling-dLLM.

The work happens in ``libpdllm.so`` (HIP kernels behind the C ABI of
``include/pdllm.h``); ``_lib`` is its ctypes binding for torch tensors.
Importing the binding fails loudly if the library was not built.
"""
__all__ = ["ops"]


def __getattr__(name):
    if name == "ops":
        from . import _lib
        return _lib
    raise AttributeError(name)
