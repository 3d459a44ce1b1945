"""MI355X-native spatiotemporal self-attention forward for video diffusion
transformers: a C-ABI HIP library for gfx950 and a thin ctypes binding.

``inputs`` (seeded synthetic workloads) imports nothing from the binding, so
it can be used without the built library.  The attention entry points live in
``binding`` and load the library on first use; they raise if it is missing.
"""

import importlib

__all__ = ["inputs", "binding"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
