"""The C-ABI library builds for gfx950, loads, and exports every symbol that
include/zc.h declares.  No compute call here needs a GPU: only argument
checks that return before any HIP call."""
import ctypes
import os
import re

import pytest

from lossless_bf16_exponent_zc_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "zc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(zc_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from lossless_bf16_exponent_zc_amd import build
        build.build()
    return binding.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 29
    assert sorted(binding.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert lib.zc_version() == 1
    assert binding.status_string(0) == "ok"
    assert binding.status_string(4) == "stream rejected"


def test_plan_argument_errors_need_no_gpu(lib):
    h = ctypes.c_void_p()
    sizes = (ctypes.c_uint64 * 2)(1000, 2000)
    assert lib.zc_plan_create(2, sizes, 1000, ctypes.byref(h)) == binding.ZC_ERR_UNSUPPORTED
    assert lib.zc_plan_create(2, sizes, 1024, ctypes.byref(h)) == binding.ZC_ERR_UNSUPPORTED
    assert lib.zc_plan_create(2, sizes, 131072, ctypes.byref(h)) == binding.ZC_ERR_UNSUPPORTED
    assert lib.zc_plan_create(0, sizes, 0, ctypes.byref(h)) == binding.ZC_ERR_INVALID_ARG
    big = (ctypes.c_uint64 * 1)(1 << 32)
    assert lib.zc_plan_create(1, big, 0, ctypes.byref(h)) == binding.ZC_ERR_UNSUPPORTED
    # plan flags: only the raw fallback is defined
    assert lib.zc_plan_create_ex(2, sizes, 0, 0x2, ctypes.byref(h)) == binding.ZC_ERR_INVALID_ARG
    assert lib.zc_plan_create_ex(2, sizes, 1000, 0x1, ctypes.byref(h)) == binding.ZC_ERR_UNSUPPORTED
    assert lib.zc_plan_flags(None) == 0
    assert lib.zc_compress(None, None, None, 0, None, None, 0, None) == binding.ZC_ERR_INVALID_ARG
    assert lib.zc_decompress(None, None, 0, None, None, 0, None) == binding.ZC_ERR_INVALID_ARG


def test_reduce_native_argument_errors_need_no_gpu(lib):
    P = ctypes.c_void_p
    shards = (P * 2)(None, None)
    assert lib.zc_reduce_native(None, 1, 8, None, None) == binding.ZC_ERR_INVALID_ARG
    assert lib.zc_reduce_native(shards, 0, 8, None, None) == binding.ZC_ERR_INVALID_ARG
    assert lib.zc_reduce_native(shards, 17, 8, None, None) == binding.ZC_ERR_INVALID_ARG
    assert lib.zc_reduce_native(shards, 2, 8, None, None) == binding.ZC_ERR_INVALID_ARG
    # misaligned shard (never dereferenced: the check returns first)
    odd = (P * 1)(P(0x1002))
    assert lib.zc_reduce_native(odd, 1, 8, P(0x1000), None) == binding.ZC_ERR_INVALID_ARG
    assert lib.zc_plan_decode_workspace_bytes(None) == 0


class _FakeTensor:
    """Stands in for a torch tensor: the checks read only these fields."""

    def __init__(self, n, esize, cuda=True, contiguous=True):
        self._n, self._e, self.is_cuda, self._c = n, esize, cuda, contiguous

    def numel(self):
        return self._n

    def element_size(self):
        return self._e

    def is_contiguous(self):
        return self._c


@pytest.mark.parametrize("bad,code", [
    (dict(x=_FakeTensor(99, 2)), binding.ZC_ERR_CAPACITY),        # too few values
    (dict(x=_FakeTensor(100, 4)), binding.ZC_ERR_INVALID_ARG),     # 4-byte elements
    (dict(x=_FakeTensor(100, 2, cuda=False)), binding.ZC_ERR_INVALID_ARG),
    (dict(x=_FakeTensor(100, 2, contiguous=False)), binding.ZC_ERR_INVALID_ARG),
    (dict(sizes=_FakeTensor(1, 4)), binding.ZC_ERR_INVALID_ARG),   # sizes are u64
    (dict(sizes=_FakeTensor(0, 8)), binding.ZC_ERR_CAPACITY),
    (dict(out=_FakeTensor(1000, 1, cuda=False)), binding.ZC_ERR_INVALID_ARG),
    (dict(ws=_FakeTensor(1000, 1, contiguous=False)), binding.ZC_ERR_INVALID_ARG),
])
def test_binding_checks_buffers_before_compress(monkeypatch, bad, code):
    monkeypatch.setattr(binding.Plan, "input_elems", property(lambda self: 100))
    monkeypatch.setattr(binding.Plan, "num_segments", property(lambda self: 1))
    p = object.__new__(binding.Plan)
    p._h = None
    args = dict(x=_FakeTensor(100, 2), out=_FakeTensor(1000, 1), sizes=_FakeTensor(1, 8),
                ws=_FakeTensor(1000, 1))
    args.update(bad)
    with pytest.raises(binding.ZcError) as e:
        p._check_compress(args["x"], args["out"], args["sizes"], args["ws"])
    assert e.value.code == code


def test_binding_checks_buffers_before_decode(monkeypatch):
    monkeypatch.setattr(binding.Plan, "input_elems", property(lambda self: 100))
    p = object.__new__(binding.Plan)
    p._h = None
    ok_out, ws = _FakeTensor(100, 2), _FakeTensor(4096, 1)
    p._check_decode(ok_out, ws)  # passes
    for out, code in ((_FakeTensor(99, 2), binding.ZC_ERR_CAPACITY),
                      (_FakeTensor(100, 1), binding.ZC_ERR_INVALID_ARG),
                      (_FakeTensor(100, 2, cuda=False), binding.ZC_ERR_INVALID_ARG)):
        with pytest.raises(binding.ZcError) as e:
            p._check_decode(out, ws)
        assert e.value.code == code
    # a capacity beyond the compressed buffer would let the kernels read past it
    with pytest.raises(binding.ZcError) as e:
        binding.check_buffer(_FakeTensor(1000, 1), "compressed input", 1, 0, 1001)
    assert e.value.code == binding.ZC_ERR_CAPACITY
    binding.check_buffer(_FakeTensor(1000, 1), "compressed input", 1, 0, 1000)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libzc.so"))
    with pytest.raises(ImportError):
        binding.lib()


def test_prefer_compressed_cost_model(lib):
    # 64M BF16 values (134,217,728 raw bytes) at ratio ~1.27, 73 us to
    # compress and 47 us to decompress: compression pays below
    # (raw - compressed) / 120 us
    raw, comp = 134217728, 105900000
    ok, be = binding.prefer_compressed(raw, comp, 73.0, 47.0, 50.0)
    assert ok and abs(be - (raw - comp) / 120e3) < 1e-9
    assert binding.prefer_compressed(raw, comp, 73.0, 47.0, be * 1.01)[0] is False
    assert binding.prefer_compressed(raw, comp, 73.0, 47.0, be * 0.99)[0] is True
    # no saving: never compressed, break-even 0
    assert binding.prefer_compressed(raw, raw, 1.0, 1.0, 0.001) == (False, 0.0)
    assert binding.prefer_compressed(raw, raw + 5, 0.0, 0.0, 1.0) == (False, 0.0)
    # free codec: any saving pays on any link
    ok, be = binding.prefer_compressed(raw, comp, 0.0, 0.0, 1e6)
    assert ok and be == float("inf")
    # invalid arguments
    assert binding.prefer_compressed(raw, comp, 1.0, 1.0, 0.0)[0] is False
    assert binding.prefer_compressed(raw, comp, -1.0, 1.0, 10.0)[0] is False
