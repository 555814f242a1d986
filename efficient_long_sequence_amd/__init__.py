"""MI355X-native MiTA (Mixture-of-Top-k Attention) forward pass.

The compute path is the HIP library ``libmita.so`` (C ABI in include/mita.h);
:mod:`efficient_long_sequence_amd.mita` is its Python binding.
"""
from . import configs, synth  # noqa: F401

__all__ = ["configs", "synth"]
