"""MI355X (gfx950) JEPA ViT encoder forward pass.

The compute lives in libjepa_mi355x.so (hand-written HIP kernels behind the C
ABI of include/jepa_mi355x.h).  This package holds its Python binding
(`_lib`, one function per C entry point), a small owning wrapper
(`Encoder`), the build step (`build`) and the seeded synthetic workloads
(`synth`).  Importing the binding fails loudly if the library is not built.
"""
from __future__ import annotations


def __getattr__(name):
    # the binding loads lazily, so `synth` and `build` import without a library
    if name in ("Encoder", "lib"):
        from . import _lib
        from .encoder import Encoder
        return {"Encoder": Encoder, "lib": _lib}[name]
    raise AttributeError(name)
