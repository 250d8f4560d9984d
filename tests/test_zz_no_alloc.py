"""zc_compress_static, the entry point that allocates nothing: its workspace
is the library's own device array.  Through the C ABI it must give the
streams and sizes zc_compress gives with a caller's workspace, call after
call, on plans of different sizes (each call leaves the array's contents to
the next), and refuse plans whose workspace exceeds the array."""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import Plan, ZcError, lib, workloads as W

from conftest import assert_same_bytes
from gpu_util import pack_inputs, say

pytestmark = pytest.mark.gpu


def _both(segs, chunk):
    plan = Plan([s.size for s in segs], chunk)
    x = pack_inputs(plan, segs)
    ref_out, ref_sz, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    plan.compress(x, ref_out, ref_sz, ws)
    out, sz = plan.empty_output(), plan.empty_sizes()
    out.fill_(0xA5)
    sz.fill_(-1)
    plan.compress_static(x, out, sz)
    torch.cuda.synchronize()
    sizes = sz.cpu().numpy()
    assert np.array_equal(sizes, ref_sz.cpu().numpy())
    o, r = out.cpu().numpy(), ref_out.cpu().numpy()
    for s, seg in enumerate(segs):
        a = plan.stream_offset(s)
        got = o[a:a + int(sizes[s])].tobytes()
        assert_same_bytes(got, r[a:a + int(sizes[s])].tobytes(), f"segment {s}")
        assert got == oracle.compress(seg, C=chunk), s
    return plan


def test_static_workspace_matches_compress_call_after_call():
    assert lib().zc_static_workspace_bytes() == 80 << 20
    big = [W.gradient(1_500_000, seed=41), np.zeros(0, np.uint16), W.small(300_001, seed=42)]
    small = [W.small(70_001, seed=43)]
    say("  first call: 3 segments, 1.8M values")
    _both(big, 65536)
    say("  second call: 1 segment, 70,001 values (another plan, smaller)")
    _both(small, 8192)
    say("  third call: the first plan again, after the other plan used the array")
    _both(big, 65536)


def test_static_workspace_refuses_large_plans():
    plan = Plan([100_000_000])
    assert plan.workspace_bytes > lib().zc_static_workspace_bytes()
    # refused on the plan's size, before any buffer is looked at
    assert lib().zc_compress_static(plan._h, None, None, 0, None, None) == 2  # ZC_ERR_CAPACITY
    with pytest.raises(ZcError):
        plan.compress_static(plan.empty_input(), plan.empty_output(), plan.empty_sizes())
