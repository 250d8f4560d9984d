"""ctypes binding of libzc.so (the C ABI in include/zc.h).

Argument marshalling only: every step of the codec runs in the HIP kernels of
libzc.so.  torch is used for device memory and the current HIP stream.  There
is no fallback: if the library is missing or cannot load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzc.so")

ZC_OK, ZC_ERR_INVALID_ARG, ZC_ERR_CAPACITY = 0, 1, 2
ZC_ERR_UNSUPPORTED, ZC_ERR_FORMAT, ZC_ERR_HIP = 3, 4, 5
FMT_BITS = {0x01: "magic", 0x02: "window", 0x04: "shape", 0x08: "size",
            0x10: "table", 0x20: "count", 0x40: "pad"}

# Every symbol include/zc.h declares.
EXPORTS = (
    "zc_version", "zc_status_string", "zc_plan_create", "zc_plan_create_ex",
    "zc_plan_destroy", "zc_plan_num_segments", "zc_plan_chunk_elems", "zc_plan_flags",
    "zc_plan_input_offset",
    "zc_plan_input_elems", "zc_plan_stream_offset", "zc_plan_max_stream_bytes",
    "zc_plan_code_offset", "zc_plan_escape_offset",
    "zc_plan_out_bytes", "zc_plan_workspace_bytes", "zc_plan_decode_workspace_bytes",
    "zc_compress",
    "zc_compress_window", "zc_compress_split", "zc_compress_timed", "zc_decompress",
    "zc_decompress_reduce",
    "zc_read_status", "zc_read_sigma", "zc_prefer_compressed", "zc_reduce_native",
    "zc_compress_static", "zc_static_workspace_bytes",
)


class ZcError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {status_string(code)} ({code})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libzc.so, raising if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, u64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
    P = ctypes.POINTER
    L.zc_version.restype = ctypes.c_int
    L.zc_status_string.argtypes = [ctypes.c_int]
    L.zc_status_string.restype = ctypes.c_char_p
    L.zc_plan_create.argtypes = [u32, P(u64), u32, P(vp)]
    L.zc_plan_create_ex.argtypes = [u32, P(u64), u32, u32, P(vp)]
    L.zc_plan_destroy.argtypes = [vp]
    L.zc_plan_destroy.restype = None
    for name, rt in (("zc_plan_num_segments", u32), ("zc_plan_chunk_elems", u32),
                     ("zc_plan_flags", u32),
                     ("zc_plan_input_elems", u64), ("zc_plan_out_bytes", u64),
                     ("zc_plan_workspace_bytes", u64), ("zc_plan_decode_workspace_bytes", u64)):
        f = getattr(L, name)
        f.argtypes = [vp]
        f.restype = rt
    for name in ("zc_plan_input_offset", "zc_plan_stream_offset",
                 "zc_plan_max_stream_bytes", "zc_plan_code_offset", "zc_plan_escape_offset"):
        f = getattr(L, name)
        f.argtypes = [vp, u32]
        f.restype = u64
    L.zc_compress.argtypes = [vp, vp, vp, u64, vp, vp, u64, vp]
    L.zc_compress_window.argtypes = [vp, vp, vp, u64, vp, u32, vp, u64, vp]
    L.zc_compress_timed.argtypes = [vp, vp, vp, u64, vp, vp, u64, vp, P(ctypes.c_float)]
    L.zc_compress_split.argtypes = [vp, vp, vp, u64, vp, vp, u64, vp, vp]
    L.zc_decompress.argtypes = [vp, vp, u64, vp, vp, u64, vp]
    L.zc_decompress_reduce.argtypes = [vp, P(vp), u32, u64, vp, vp, u64, vp]
    L.zc_read_status.argtypes = [vp, vp, vp, P(u32)]
    L.zc_reduce_native.argtypes = [P(vp), u32, u64, vp, vp]
    L.zc_compress_static.argtypes = [vp, vp, vp, u64, vp, vp]
    L.zc_static_workspace_bytes.argtypes = []
    L.zc_static_workspace_bytes.restype = u64
    L.zc_prefer_compressed.argtypes = [u64, u64, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_double, P(ctypes.c_double)]
    L.zc_prefer_compressed.restype = ctypes.c_int
    L.zc_read_sigma.argtypes = [vp, vp, u32, vp, P(ctypes.c_double),
                                P(ctypes.c_double), P(u64), P(ctypes.c_double),
                                P(u32)]
    for name in ("zc_plan_create", "zc_plan_create_ex", "zc_compress", "zc_compress_window", "zc_compress_timed",
                 "zc_compress_split",
                 "zc_decompress", "zc_decompress_reduce", "zc_read_status",
                 "zc_read_sigma", "zc_reduce_native", "zc_compress_static"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(code: int) -> str:
    return lib().zc_status_string(code).decode()


def prefer_compressed(raw_bytes: int, compressed_bytes: int, compress_us: float,
                      decompress_us: float, link_GBps: float):
    """(send compressed?, break-even link GB/s) from measured sizes and times."""
    be = ctypes.c_double()
    r = lib().zc_prefer_compressed(int(raw_bytes), int(compressed_bytes), float(compress_us),
                                   float(decompress_us), float(link_GBps), ctypes.byref(be))
    return bool(r), be.value


def _check(rc: int, what: str):
    if rc != ZC_OK:
        raise ZcError(rc, what)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def check_buffer(t, what: str, elem_size: int | None = None, min_elems: int = 0,
                 min_bytes: int = 0):
    """Raise ZcError(ZC_ERR_INVALID_ARG / ZC_ERR_CAPACITY) unless t is a
    contiguous tensor on a GPU with the given element size and at least
    min_elems elements and min_bytes bytes.  The C ABI takes bare pointers,
    so the sizes it cannot see are checked here, before any call."""
    if not getattr(t, "is_cuda", False):
        raise ZcError(ZC_ERR_INVALID_ARG, f"{what}: not a GPU tensor")
    if not t.is_contiguous():
        raise ZcError(ZC_ERR_INVALID_ARG, f"{what}: not contiguous")
    if elem_size is not None and t.element_size() != elem_size:
        raise ZcError(ZC_ERR_INVALID_ARG,
                      f"{what}: {t.element_size()}-byte elements, {elem_size} expected")
    if t.numel() < min_elems or _nbytes(t) < min_bytes:
        raise ZcError(ZC_ERR_CAPACITY, f"{what}: {t.numel()} elements, {_nbytes(t)} bytes "
                                       f"(needs {min_elems} elements, {min_bytes} bytes)")


def reduce_native(shards, out, stream=None):
    """Enqueue the native (uncompressed) fixed-order fp32 sum of BF16 shards
    (16-bit tensors of equal length) into out, rounded as decompress_reduce
    rounds."""
    if not 1 <= len(shards) <= 16:
        raise ZcError(ZC_ERR_INVALID_ARG, "reduce_native: 1..16 shards")
    n = shards[0].numel()
    for i, t in enumerate(shards):
        check_buffer(t, f"shard {i}", 2, n)
    check_buffer(out, "out", 2, n)
    arr = (ctypes.c_void_p * len(shards))(*[t.data_ptr() for t in shards])
    _check(lib().zc_reduce_native(arr, len(shards), n, _ptr(out), _stream(stream)),
           "zc_reduce_native")


PLAN_RAW_FALLBACK = 0x1  # ZC_PLAN_RAW_FALLBACK


class Plan:
    """A codec plan: segment sizes and chunk size, plus its device tables.
    raw_fallback: compress stores a segment as a raw stream (its words after
    the header) when the coded stream would be longer."""

    def __init__(self, segment_elems, chunk_elems: int = 65536, raw_fallback: bool = False):
        sizes = [int(n) for n in segment_elems]
        arr = (ctypes.c_uint64 * len(sizes))(*sizes)
        h = ctypes.c_void_p()
        flags = PLAN_RAW_FALLBACK if raw_fallback else 0
        _check(lib().zc_plan_create_ex(len(sizes), arr, chunk_elems, flags, ctypes.byref(h)),
               "zc_plan_create_ex")
        self._h = h
        self.segment_elems = sizes
        self.chunk_elems = lib().zc_plan_chunk_elems(h)
        self.flags = lib().zc_plan_flags(h)

    def close(self):
        if getattr(self, "_h", None):
            lib().zc_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # geometry -----------------------------------------------------------
    @property
    def num_segments(self) -> int:
        return lib().zc_plan_num_segments(self._h)

    @property
    def input_elems(self) -> int:
        return lib().zc_plan_input_elems(self._h)

    @property
    def out_bytes(self) -> int:
        return lib().zc_plan_out_bytes(self._h)

    @property
    def workspace_bytes(self) -> int:
        return lib().zc_plan_workspace_bytes(self._h)

    @property
    def decode_workspace_bytes(self) -> int:
        """Workspace bytes the decoders need (status words and a stand-in)."""
        return lib().zc_plan_decode_workspace_bytes(self._h)

    def input_offset(self, s: int) -> int:
        return lib().zc_plan_input_offset(self._h, s)

    def stream_offset(self, s: int) -> int:
        return lib().zc_plan_stream_offset(self._h, s)

    def max_stream_bytes(self, s: int) -> int:
        return lib().zc_plan_max_stream_bytes(self._h, s)

    def code_offset(self, s: int) -> int:
        """Offset of segment s's code planes from its stream start."""
        return lib().zc_plan_code_offset(self._h, s)

    def escape_offset(self, s: int) -> int:
        """Offset of segment s's escape region from its stream start."""
        return lib().zc_plan_escape_offset(self._h, s)

    # buffers (torch allocation only) -------------------------------------
    def empty_input(self, device="cuda"):
        import torch
        return torch.zeros(max(self.input_elems, 1), dtype=torch.int16, device=device)

    def empty_output(self, device="cuda"):
        import torch
        return torch.empty(self.out_bytes, dtype=torch.uint8, device=device)

    def empty_workspace(self, device="cuda", decode_only: bool = False):
        import torch
        n = self.decode_workspace_bytes if decode_only else self.workspace_bytes
        return torch.empty(n, dtype=torch.uint8, device=device)

    def empty_sizes(self, device="cuda"):
        import torch
        return torch.zeros(self.num_segments, dtype=torch.int64, device=device)

    # codec calls ----------------------------------------------------------
    def _check_compress(self, x, out, stream_bytes, ws):
        check_buffer(x, "input", 2, self.input_elems)
        check_buffer(out, "output", 1)
        check_buffer(stream_bytes, "stream_bytes", 8, self.num_segments)
        check_buffer(ws, "workspace", 1)

    def _check_decode(self, out, ws):
        check_buffer(out, "output", 2, self.input_elems)
        check_buffer(ws, "workspace", 1)

    def compress(self, x, out, stream_bytes, ws, window: int | None = None, stream=None):
        """Enqueue compression of x (BF16 bits, 16-bit dtype) into out."""
        self._check_compress(x, out, stream_bytes, ws)
        if window is None:
            rc = lib().zc_compress(self._h, _ptr(x), _ptr(out), _nbytes(out),
                                   _ptr(stream_bytes), _ptr(ws), _nbytes(ws),
                                   _stream(stream))
            _check(rc, "zc_compress")
        else:
            rc = lib().zc_compress_window(self._h, _ptr(x), _ptr(out), _nbytes(out),
                                          _ptr(stream_bytes), int(window), _ptr(ws),
                                          _nbytes(ws), _stream(stream))
            _check(rc, "zc_compress_window")

    def compress_static(self, x, out, stream_bytes, stream=None):
        """Enqueue compress() with the library's own device array as the
        workspace (zc_compress_static: allocates nothing; calls on one GPU
        must not overlap)."""
        check_buffer(x, "input", 2, self.input_elems)
        check_buffer(out, "output", 1)
        check_buffer(stream_bytes, "stream_bytes", 8, self.num_segments)
        rc = lib().zc_compress_static(self._h, _ptr(x), _ptr(out), _nbytes(out),
                                      _ptr(stream_bytes), _stream(stream))
        _check(rc, "zc_compress_static")

    def compress_split(self, x, out, stream_bytes, ws, fixed_ready, stream=None):
        """Enqueue compress() and record fixed_ready (a torch.cuda.Event that
        has been recorded once, so it exists) as soon as the headers, chunk
        tables, code planes, sign+mantissa bytes and sizes are final."""
        self._check_compress(x, out, stream_bytes, ws)
        rc = lib().zc_compress_split(self._h, _ptr(x), _ptr(out), _nbytes(out),
                                     _ptr(stream_bytes), _ptr(ws), _nbytes(ws),
                                     _stream(stream), ctypes.c_void_p(fixed_ready.cuda_event))
        _check(rc, "zc_compress_split")

    def compress_timed(self, x, out, stream_bytes, ws, stream=None):
        """Compress as compress() and wait for it; returns the three kernels'
        times in microseconds (encoder pass, window, escape placement), from
        HIP events recorded on the stream between them."""
        self._check_compress(x, out, stream_bytes, ws)
        us = (ctypes.c_float * 3)()
        rc = lib().zc_compress_timed(self._h, _ptr(x), _ptr(out), _nbytes(out),
                                     _ptr(stream_bytes), _ptr(ws), _nbytes(ws),
                                     _stream(stream), us)
        _check(rc, "zc_compress_timed")
        return [float(v) for v in us]

    def decompress(self, comp, out, ws, capacity: int | None = None, stream=None):
        """Enqueue decoding of the packed streams in comp into out; capacity
        (default: all of comp) is the readable bytes the kernels are told of."""
        cap = _nbytes(comp) if capacity is None else int(capacity)
        check_buffer(comp, "compressed input", 1, 0, cap)
        self._check_decode(out, ws)
        rc = lib().zc_decompress(self._h, _ptr(comp), cap, _ptr(out), _ptr(ws),
                                 _nbytes(ws), _stream(stream))
        _check(rc, "zc_decompress")

    def decompress_reduce(self, streams, out, ws, capacity: int, stream=None):
        """Enqueue decode + fixed-order fp32 sum of single-segment streams
        (each tensor holds at least `capacity` bytes)."""
        for i, t in enumerate(streams):
            check_buffer(t, f"stream {i}", 1, 0, int(capacity))
        self._check_decode(out, ws)
        arr = (ctypes.c_void_p * len(streams))(*[s.data_ptr() for s in streams])
        rc = lib().zc_decompress_reduce(self._h, arr, len(streams), int(capacity),
                                        _ptr(out), _ptr(ws), _nbytes(ws),
                                        _stream(stream))
        _check(rc, "zc_decompress_reduce")

    def read_status(self, ws, stream=None) -> int:
        """Synchronise and return the rejection bits of the last decode."""
        bits = ctypes.c_uint32()
        rc = lib().zc_read_status(self._h, _ptr(ws), _stream(stream), ctypes.byref(bits))
        if rc not in (ZC_OK, ZC_ERR_FORMAT):
            _check(rc, "zc_read_status")
        return bits.value

    def read_sigma(self, ws, s: int = 0, stream=None):
        """Synchronise and return (S1, S2, n, var, L) of segment s."""
        S1, S2, var = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        n, L = ctypes.c_uint64(), ctypes.c_uint32()
        _check(lib().zc_read_sigma(self._h, _ptr(ws), s, _stream(stream),
                                   ctypes.byref(S1), ctypes.byref(S2), ctypes.byref(n),
                                   ctypes.byref(var), ctypes.byref(L)), "zc_read_sigma")
        return S1.value, S2.value, n.value, var.value, L.value
