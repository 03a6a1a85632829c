"""MI355X-native forward pass of a stack of post-LN transformer encoder
layers with causal and key-padding masking (library name: tfl).

The compute path is the HIP library ``libtfl.so`` (C ABI in include/tfl.h);
``binding`` is its ctypes binding and ``synth`` draws seeded inputs.
"""
from .binding import (AUDIT_LIB_PATH, DTYPE_CODES, LAYER_KEYS, LIB_PATH, PATHS, STAGES, SYMBOLS, Encoder, Handle, TflError,
                      load_library, make_config, plan_for, to_device, to_numpy_f64)

__all__ = ["AUDIT_LIB_PATH", "DTYPE_CODES", "LAYER_KEYS", "LIB_PATH", "PATHS", "STAGES", "SYMBOLS", "Encoder", "Handle", "TflError",
           "load_library", "make_config", "plan_for", "to_device", "to_numpy_f64"]
