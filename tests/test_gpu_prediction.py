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

from conftest import assert_same_bytes
from gpu_util import gpu_compress, gpu_decompress, say, stat_bits

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
        assert_same_bytes(st, ref, f"segment {s}")
        if window is None:
            assert stat_bits(plan.read_sigma(ws, s)) == stat_bits(oracle.sigma(seg)), s
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


def test_split_event_fixed_regions_final():
    # copies taken on another stream right after the split event must equal
    # the finished streams: headers, chunk tables, code planes, sm bytes and
    # sizes are final at the event (first call mispredicted: the window kernel
    # codes again before the event)
    import torch
    segs = [W.gradient(200000 + 777 * i, seed=40 + i) for i in range(3)]
    plan = Plan([s.size for s in segs])
    from gpu_util import pack_inputs
    x = pack_inputs(plan, segs)
    out, sizes, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    ws.zero_()
    side = torch.cuda.Stream()
    for call in range(3):
        out.fill_(0xA5)
        torch.cuda.synchronize()
        ev = torch.cuda.Event()
        ev.record()
        plan.compress_split(x, out, sizes, ws, ev)
        early = []
        with torch.cuda.stream(side):
            side.wait_event(ev)
            early_sizes = sizes.clone()
            for s in range(len(segs)):
                so = plan.stream_offset(s)
                k = -(-segs[s].size // plan.chunk_elems)
                head = 64 + 4 * (k + 1)  # header and chunk table
                early.append((out[so:so + head].clone(),
                              out[so + plan.code_offset(s):so + plan.escape_offset(s)].clone()))
        torch.cuda.synchronize()
        assert torch.equal(early_sizes, sizes), call
        for s, seg in enumerate(segs):
            so = plan.stream_offset(s)
            ref = oracle.compress(seg)
            assert_same_bytes(out[so:so + int(sizes[s])].cpu().numpy().tobytes(), ref, f"call {call}, segment {s}")
            h, f = early[s]
            assert torch.equal(h, out[so:so + h.numel()]), (call, s, "header/table")
            assert torch.equal(f, out[so + plan.code_offset(s):so + plan.escape_offset(s)]), (call, s)


def test_many_small_chunks():
    # 2048-value chunks over 32M values: 16,385 chunks (the chunk table goes
    # through its table-resident path, 64+ chunks per thread) and 16,385
    # moment blocks (8 rounds in the window kernel's reduction); fresh
    # workspace (the window kernel codes again), then the predicted path
    x = W.gradient((1 << 25) + 555, seed=25)
    plan = Plan([x.size], 2048)
    ws = plan.empty_workspace()
    ws.zero_()
    for _ in range(2):
        check([x], plan, ws, chunk=2048)
