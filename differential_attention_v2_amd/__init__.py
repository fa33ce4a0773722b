"""MI355X-native Differential Attention V2 forward pass.

The computation lives in ``libdiffattn.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/diffattn.h``); ``binding`` is a thin ctypes
layer over it.  Importing this package does not load the library: the first call
does, and raises if it was never built.
"""
__version__ = "0.1.0"

from .binding import (  # noqa: F401
    DiffAttnError, decode, decode_workspace, load_library, prefill, v1_lambda,
)
