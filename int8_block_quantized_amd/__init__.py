"""MI355X-native per-block (32x32) INT8 data flow (Jetfire-style linear layer).

The compute path is the HIP library ``libjetfire.so`` (C ABI declared in
``include/jetfire.h``); ``int8_block_quantized_amd.jetfire`` is its thin
ctypes binding.  The binding is imported lazily so that ``inputs`` (the seeded
generators) can be used without loading the device library.
"""
from __future__ import annotations

import importlib

__all__ = ["jetfire", "inputs", "quantize_block", "requant_block", "gemm_i8_blockscaled", "gelu_i8"]

_BINDING_NAMES = {"quantize_block", "requant_block", "gemm_i8_blockscaled", "gelu_i8"}


def __getattr__(name):
    if name in ("jetfire", "inputs"):
        return importlib.import_module(f"{__name__}.{name}")
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(f"{__name__}.jetfire"), name)
    raise AttributeError(name)
