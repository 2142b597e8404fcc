"""libkvq: decode-step attention over a compressed (INT8/INT4/INT2 + bf16) VLM
KV cache, for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/kvq.h``); ``kvq`` is a thin ctypes binding
with the same call names.  ``synth`` draws the seeded synthetic workloads.
"""
import importlib

__all__ = ["kvq", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
