"""Lossless BF16 exponent coding on AMD MI355X (gfx950).

The codec of ZipCCL ("Key idea and contribution", technique 1) as HIP kernels
behind the C ABI in include/zc.h; ``Plan`` is the thin ctypes binding.
``workloads`` draws the seeded synthetic inputs.
"""
from .binding import (EXPORTS, LIB_PATH, Plan, ZcError, check_buffer, lib, prefer_compressed,
                      reduce_native)

__all__ = ["EXPORTS", "LIB_PATH", "Plan", "ZcError", "check_buffer", "lib", "prefer_compressed",
           "reduce_native"]
