"""libarl2: one ARL2 ("Attend Locally, Remember Linearly") hybrid attention
layer on MI355X (gfx950), behind the C ABI of include/arl2.h.

``hybrid_softmax_gated_amd.binding`` is the ctypes binding (same names as the
C entry points); ``hybrid_softmax_gated_amd.layer`` holds a small helper that
lets torch allocate the state and workspace; ``hybrid_softmax_gated_amd.stack``
the bookkeeping of an attention-only stack mixing the layer with softmax
key/value-cache layers. Importing any of them requires the built library
(``python -m hybrid_softmax_gated_amd.build``).
"""
import importlib

__all__ = ["binding", "layer", "stack", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
