"""MI355X-native sparse Mixture-of-Experts feed-forward layer (forward pass).

The compute runs in libmoe (hand-written HIP for gfx950, C ABI declared in
include/libmoe.h); ``_lib`` is its ctypes binding and ``MoELayer`` sequences
one layer call.  Importing ``_lib`` or ``MoELayer`` fails if the library has
not been built (``python -m sparse_mixture_experts_moe_amd.build``).
"""

__all__ = ["MoELayer", "lib"]


def __getattr__(name):
    if name == "MoELayer":
        from .layer import MoELayer
        return MoELayer
    if name == "lib":
        from . import _lib
        return _lib
    raise AttributeError(name)
