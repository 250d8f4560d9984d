"""GPU parity of the window prediction: the encoder's first pass codes every
segment with the window the workspace recorded on the previous call, and
segments whose window turns out different are coded again.  Whatever the
workspace holds (fresh zeros, garbage, another tensor's windows), every
stream must be byte-identical to the oracle's and the statistics identical.
"""
import numpy as np
import pytest

import oracle
from lossless_bf16_exponent_zc_amd import Plan
from lossless_bf16_exponent_zc_amd import workloads as W

from gpu_util import gpu_compress, gpu_decompress, say

pytestmark = pytest.mark.gpu


def scaled(x: np.ndarray, binades: int) -> np.ndarray:
    """Shift every normal value's exponent by `binades` (kept within the
    normal range), which moves the window by the same amount."""
    e = (x >> 7) & 0xFF
    normal = (e >= 1) & (e <= 254)
    ne = np.clip(e.astype(np.int32) + binades, 1, 254).astype(np.uint16)
    y = np.where(normal, (x & 0x807F) | (ne << 7), x)
    return y.astype(np.uint16)


def check(segs, plan, ws, chunk=65536, window=None):
    streams, _, out, _ = gpu_compress(segs, chunk, window, plan=plan, ws=ws)
    for s, (seg, st) in enumerate(zip(segs, streams)):
        ref = oracle.compress(seg, C=chunk, L=window)
        assert st == ref, f"segment {s}: stream differs (len {len(st)} vs {len(ref)})"
        if window is None:
            assert plan.read_sigma(ws, s) == oracle.sigma(seg), s
    bits, dec = gpu_decompress(plan, out)
    assert bits == 0, hex(bits)
    for seg, d in zip(segs, dec):
        assert np.array_equal(seg, d)


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x7B])
def test_fresh_workspace(fill):
    x = W.gradient(5 * 65536 + 999, seed=21)
    plan = Plan([x.size])
    ws = plan.empty_workspace()
    ws.fill_(fill)
    say(f"  workspace filled with {fill:#x}: first call, then repeat")
    check([x], plan, ws)
    check([x], plan, ws)


def test_window_moves_between_calls():
    x = W.gradient(3 * 65536 + 4321, seed=22)
    plan = Plan([x.size])
    ws = plan.empty_workspace()
    ws.zero_()
    for b in (0, 9, 9, -5, 0, 40, 40):
        say(f"  exponents shifted by {b}")
        check([scaled(x, b)], plan, ws)


def test_large_segment_recoded_by_many_workgroups():
    # 5M values: 306 encoder items, recoded by 20 window workgroups
    x = W.gradient(5 * (1 << 20) + 3333, seed=24)
    plan = Plan([x.size])
    ws = plan.empty_workspace()
    ws.zero_()
    for b in (0, 0, -7, 0):
        say(f"  exponents shifted by {b}")
        check([scaled(x, b)], plan, ws)


def test_some_segments_mispredicted():
    segs = [W.gradient(70000 + 4096 * i, seed=30 + i) for i in range(6)]
    segs.insert(2, np.zeros(0, np.uint16))
    plan = Plan([s.size for s in segs], 16384)
    ws = plan.empty_workspace()
    ws.zero_()
    check(segs, plan, ws, chunk=16384)
    moved = [scaled(s, 3) if i % 2 else s for i, s in enumerate(segs)]
    say("  odd segments shifted by 3 binades")
    check(moved, plan, ws, chunk=16384)
    check(moved, plan, ws, chunk=16384)


def test_fixed_window_between_derived_calls():
    x = W.gradient(2 * 65536 + 17, seed=23)
    plan = Plan([x.size])
    ws = plan.empty_workspace()
    ws.zero_()
    check([x], plan, ws)
    check([x], plan, ws, window=200)
    check([x], plan, ws)
    check([x], plan, ws, window=oracle.sigma(x)[4])
    check([x], plan, ws)
