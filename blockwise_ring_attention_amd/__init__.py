"""MI355X-native ring-member share of exact blockwise softmax attention.

The compute lives in ``libringattn.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/ring_attn.h``); ``_lib`` binds it with ctypes and
``share`` runs whole ring shares through it.  Importing this package does not
load the library; the first call does, and raises if it was never built.
"""
from .configs import CONFIGS, ShareConfig  # noqa: F401

__all__ = ["CONFIGS", "ShareConfig"]
