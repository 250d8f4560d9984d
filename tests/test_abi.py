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
    assert len(names) == 25
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
