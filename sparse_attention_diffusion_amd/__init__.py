"""Re-ttention-style ultra-sparse attention for DiT denoising on MI355X (gfx950).

The compute path is a HIP library with a C ABI (``include/rettn.h``); the
Python module ``rettn`` is its thin ctypes binding.  ``synth`` draws the seeded
synthetic workloads and ``configs`` names them.
"""
import importlib

__all__ = ["configs", "synth", "rettn"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
