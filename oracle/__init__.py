"""CPU oracle for lossless BF16 exponent coding -- TEST INFRASTRUCTURE ONLY.

This package wraps the plain C oracle (``zco.c``) with numpy-friendly
helpers.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its
binding) never does, and shares no code with it.

Method source: ZipCCL (SIGCOMM scribe notes), "Key idea and contribution",
first technique -- exponent window from the tensor's standard deviation,
3-bit codes for frequent exponents, full exponents kept separately for the
rest, about 11 bits per value.  Stream layout: see ``zco.c``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libzco.so")
_lib = None

MAGIC = 0x3142435A
GROUP = 2048
FMT_MAGIC, FMT_WINDOW, FMT_SHAPE, FMT_SIZE = 0x01, 0x02, 0x04, 0x08
FMT_TABLE, FMT_COUNT, FMT_PAD = 0x10, 0x20, 0x40
FLAG_RAW = 0x01          # header flags: a raw stream
OPT_RAW_FALLBACK = 0x01  # compress option: raw when the coded stream is longer


def lib():
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "zco.c")
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src)):
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        dp = ctypes.POINTER(ctypes.c_double)
        L.zco_c0.restype = ctypes.c_double
        L.zco_bf16_to_f64.argtypes = [u16p, ctypes.c_size_t, dp]
        L.zco_pairwise_sum.argtypes = [dp, ctypes.c_size_t]
        L.zco_pairwise_sum.restype = ctypes.c_double
        L.zco_sigma.argtypes = [u16p, ctypes.c_size_t, dp, dp, u64p, dp]
        L.zco_window.argtypes = [ctypes.c_double]
        L.zco_window.restype = ctypes.c_int
        for name in ("zco_code_off", "zco_sm_off", "zco_esc_off",
                     "zco_max_stream_bytes"):
            f = getattr(L, name)
            f.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
            f.restype = ctypes.c_uint64
        L.zco_compress.argtypes = [u16p, ctypes.c_uint64, ctypes.c_uint32,
                                   ctypes.c_int, u8p, ctypes.c_uint64, u64p]
        L.zco_compress.restype = ctypes.c_int
        L.zco_compress_ex.argtypes = [u16p, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_int, ctypes.c_uint32, u8p,
                                      ctypes.c_uint64, u64p]
        L.zco_compress_ex.restype = ctypes.c_int
        L.zco_decompress.argtypes = [u8p, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_uint32, u16p]
        L.zco_decompress.restype = ctypes.c_uint32
        L.zco_round_bf16.argtypes = [ctypes.c_float]
        L.zco_round_bf16.restype = ctypes.c_uint16
        L.zco_decompress_reduce.argtypes = [
            ctypes.POINTER(u8p), u64p, ctypes.c_uint32, ctypes.c_uint64,
            ctypes.c_uint32, u16p]
        L.zco_decompress_reduce.restype = ctypes.c_uint32
        _lib = L
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("BF16 data must be passed as uint16 bit patterns")
    return x


def c0() -> float:
    return lib().zco_c0()


def bf16_to_f64(x):
    x = _u16(x)
    out = np.empty(x.size, dtype=np.float64)
    lib().zco_bf16_to_f64(_ptr(x, ctypes.c_uint16), x.size,
                          _ptr(out, ctypes.c_double))
    return out


def pairwise_sum(a) -> float:
    a = np.ascontiguousarray(a, dtype=np.float64)
    return lib().zco_pairwise_sum(_ptr(a, ctypes.c_double), a.size)


def sigma(x):
    """Return (S1, S2, n_finite, var, L) of one tensor of BF16 bits."""
    x = _u16(x)
    S1, S2, var = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    n = ctypes.c_uint64()
    lib().zco_sigma(_ptr(x, ctypes.c_uint16), x.size, ctypes.byref(S1),
                    ctypes.byref(S2), ctypes.byref(n), ctypes.byref(var))
    return S1.value, S2.value, n.value, var.value, window(var.value)


def window(var: float) -> int:
    return lib().zco_window(float(var))


def code_off(N, C=65536):
    return lib().zco_code_off(N, C)


def sm_off(N, C=65536):
    return lib().zco_sm_off(N, C)


def esc_off(N, C=65536):
    return lib().zco_esc_off(N, C)


def max_stream_bytes(N, C=65536):
    return lib().zco_max_stream_bytes(N, C)


def compress(x, C=65536, L=None, raw_fallback=False) -> bytes:
    """Compress one tensor of BF16 bits; L forces the window (1..248);
    raw_fallback stores the words as they are when coding would not shrink
    them."""
    x = _u16(x)
    cap = max(max_stream_bytes(x.size, C), 64 + 2 * x.size)
    out = np.zeros(cap, dtype=np.uint8)
    n = ctypes.c_uint64()
    rc = lib().zco_compress_ex(_ptr(x, ctypes.c_uint16), x.size, C,
                               -1 if L is None else int(L),
                               OPT_RAW_FALLBACK if raw_fallback else 0,
                               _ptr(out, ctypes.c_uint8), cap, ctypes.byref(n))
    if rc != 0:
        raise ValueError(f"zco_compress failed with {rc}")
    return out[: n.value].tobytes()


def decompress_status(stream, N, C=65536):
    """Return (rejection bits, decoded uint16 array)."""
    s = np.frombuffer(bytes(stream), dtype=np.uint8).copy()
    if s.size == 0:
        s = np.zeros(1, dtype=np.uint8)
        length = 0
    else:
        length = s.size
    out = np.zeros(max(N, 1), dtype=np.uint16)
    bad = lib().zco_decompress(_ptr(s, ctypes.c_uint8), length, N, C,
                               _ptr(out, ctypes.c_uint16))
    return bad, out[:N]


def decompress(stream, N, C=65536):
    bad, out = decompress_status(stream, N, C)
    if bad:
        raise ValueError(f"stream rejected, bits 0x{bad:02x}")
    return out


def round_bf16(f: float) -> int:
    return lib().zco_round_bf16(ctypes.c_float(f))


def decompress_reduce(streams, N, C=65536):
    """Decode each stream, sum in shard order in fp32, round to BF16."""
    arrs = [np.frombuffer(bytes(s), dtype=np.uint8).copy() for s in streams]
    u8p = ctypes.POINTER(ctypes.c_uint8)
    ptrs = (u8p * len(arrs))(*[_ptr(a, ctypes.c_uint8) for a in arrs])
    lens = np.array([a.size for a in arrs], dtype=np.uint64)
    out = np.zeros(max(N, 1), dtype=np.uint16)
    bad = lib().zco_decompress_reduce(ptrs, _ptr(lens, ctypes.c_uint64),
                                      len(arrs), N, C,
                                      _ptr(out, ctypes.c_uint16))
    if bad:
        raise ValueError(f"stream rejected, bits 0x{bad:02x}")
    return out[:N]


def parse_header(stream):
    """Header fields of a stream as a dict (little-endian)."""
    b = bytes(stream[:64])
    le = lambda o, n: int.from_bytes(b[o:o + n], "little")
    return dict(magic=le(0, 4), version=le(4, 2), L=b[6], flags=b[7],
                N=le(8, 8), C=le(16, 4), K=le(20, 4), E=le(24, 8),
                total=le(32, 8), code_off=le(40, 8), sm_off=le(48, 8),
                esc_off=le(56, 8))
