"""Re-ttention-style ultra-sparse attention for DiT denoising on MI355X (gfx950).

The compute path is a HIP library with a C ABI (``include/rettn.h``); the
Python module ``rettn`` is its thin ctypes binding.  ``synth`` draws the seeded
synthetic workloads and ``configs`` names them.
"""
__all__ = ["configs", "synth", "rettn"]


def __getattr__(name):
    if name == "rettn":
        from . import rettn
        return rettn
    raise AttributeError(name)
