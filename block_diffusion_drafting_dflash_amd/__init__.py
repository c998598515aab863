"""DFlash drafting hot path for AMD Instinct MI355X (gfx950).

The drafting step lives in ``libdflash.so`` (hand-written HIP kernels behind
the C ABI in ``include/dflash.h``); this package is its ctypes binding.
"""
from .binding import (DFlash, DFlashError, Config, Weights, load_library,
                      load_harness, make_config, kv_cache_bytes,
                      verify_greedy, verify_sampling, synth_target, fp8_to_bf16,
                      target_forward, read_probe, LIB_PATH,
                      HARNESS_PATH,
                      LIB_SYMBOLS, HARNESS_SYMBOLS)

__all__ = ["DFlash", "DFlashError", "Config", "Weights", "load_library",
           "load_harness", "make_config", "kv_cache_bytes", "verify_greedy",
           "verify_sampling",
           "synth_target", "fp8_to_bf16", "target_forward", "read_probe",
           "LIB_PATH", "HARNESS_PATH", "LIB_SYMBOLS",
           "HARNESS_SYMBOLS"]
