"""MI355X (gfx950) quantized Llama forward with Q8_0 weights.

The compute runs in hand-written HIP kernels inside ``libq8l.so`` behind the C
ABI declared in ``include/q8l.h``; ``q8l`` is its ctypes binding and
``Q8Model`` a convenience wrapper that places a model's tensors in device
memory (torch), binds them and drives forward / generate.
"""

from __future__ import annotations

from . import q8l
from .q8l import (Q8LError, Q8L_OK, STATUS_NAMES, q8l_config)

__all__ = ["q8l", "Q8LError", "Q8L_OK", "STATUS_NAMES", "q8l_config", "Q8Model"]


def __getattr__(name):
    if name == "Q8Model":
        from .model import Q8Model
        return Q8Model
    raise AttributeError(name)
