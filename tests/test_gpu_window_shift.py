"""GPU parity of the one-step recode: when the window the encoder's first
pass used (the previous call's) is one step from the tensor's own, the
tail derives the new code planes and escapes from the first pass's output
instead of coding the input again.  Every stream must be byte-identical to
the oracle's, whatever the shift's direction, the group's fill (a ragged
last group, groups with more than 512 escapes, whole groups of escapes,
Inf and NaN), the chunk size, and at the ends of the window's range
(1 <-> 2, 247 <-> 248); shifts of two or more take the full recode.
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
    """Every normal value's exponent moved by `binades` (kept within the
    normal range), which moves the window by about as much."""
    e = (x >> 7) & 0xFF
    normal = (e >= 1) & (e <= 254)
    ne = np.clip(e.astype(np.int32) + binades, 1, 254).astype(np.uint16)
    return np.where(normal, (x & 0x807F) | (ne << 7), x).astype(np.uint16)


def window(x: np.ndarray) -> int:
    return int(oracle.sigma(x)[4])


def after(prev, segs, chunk):
    """Compress `prev` (so the workspace predicts its windows), then `segs`
    on the same plan and workspace; every stream of the second call against
    the oracle's, the statistics, and the round trip."""
    plan = Plan([s.size for s in segs], chunk)
    ws = plan.empty_workspace()
    ws.zero_()
    gpu_compress(prev, chunk, plan=plan, ws=ws)
    for s, p in enumerate(prev):
        if p.size:
            assert plan.read_sigma(ws, s)[4] == window(p), s
    streams, _, out, _ = gpu_compress(segs, chunk, plan=plan, ws=ws)
    for s, (seg, st) in enumerate(zip(segs, streams)):
        assert_same_bytes(st, oracle.compress(seg, C=chunk), f"segment {s}")
        assert stat_bits(plan.read_sigma(ws, s)) == stat_bits(oracle.sigma(seg)), s
    bits, dec = gpu_decompress(plan, out)
    assert bits == 0, hex(bits)
    for seg, d in zip(segs, dec):
        assert np.array_equal(seg, d)


def one_step_pair(x):
    """(tensor one window step above x, one step below), found by moving
    the exponents: normally one binade, but the values clipped at the ends
    of the range can make it two."""
    L = window(x)
    up = next(scaled(x, b) for b in (1, 2, 3) if window(scaled(x, b)) == L + 1)
    down = next(scaled(x, -b) for b in (1, 2, 3) if window(scaled(x, -b)) == L - 1)
    return up, down


@pytest.mark.parametrize("chunk", [2048, 16384, 65536])
def test_one_step_both_directions(chunk):
    x = W.gradient(3 * 65536 + 2048 * 5 + 777, seed=61)  # a ragged last group
    up, down = one_step_pair(x)
    say(f"  chunk {chunk}: window {window(x)}, first pass one step above, then one below")
    after([up], [x], chunk)    # coded with L + 1 first: the recode moves down
    after([down], [x], chunk)  # coded with L - 1 first: the recode moves up


def test_one_step_many_escapes():
    # groups with more than 512 escapes (half the values zero, so the staged
    # run spans more than two dwords per lane), a chunk of zeros only (every
    # value an escape), and Inf / NaN values (always escapes)
    rng = np.random.default_rng(62)
    x = W.gradient(4 * 65536 + 3001, seed=62)
    x[rng.random(x.size) < 0.5] = 0
    x[65536:2 * 65536] = 0
    x[rng.integers(0, x.size, 40)] = 0x7F80
    x[rng.integers(0, x.size, 40)] = 0xFFC1
    up, down = one_step_pair(x)
    say(f"  window {window(x)}: half the values zero, one chunk all zero, Inf and NaN")
    after([up], [x], 65536)
    after([down], [x], 65536)


def with_window(x, target):
    """x with its exponents moved so that its window is `target`."""
    for b in range(-200, 200):
        y = scaled(x, b)
        if window(y) == target:
            return y
    raise AssertionError(f"no shift of the test tensor has window {target}")


@pytest.mark.parametrize("lo,hi", [(1, 2), (247, 248)])
def test_one_step_at_the_ends(lo, hi):
    x = W.gradient(2 * 65536 + 123, seed=63)
    a, b = with_window(x, lo), with_window(x, hi)
    say(f"  windows {lo} and {hi}: each coded first with the other's")
    after([b], [a], 65536)
    after([a], [b], 65536)


def test_mixed_segments():
    # one plan: segments whose first pass was one step up, one step down,
    # right (a hit), two steps off (the full recode), and an empty one
    base = [W.gradient(70000 + 9000 * i, seed=64 + i) for i in range(5)]
    base[3] = np.zeros(0, np.uint16)
    prev = []
    for i, s in enumerate(base):
        if i == 0:
            prev.append(one_step_pair(s)[0])
        elif i == 1:
            prev.append(one_step_pair(s)[1])
        elif i == 4:
            prev.append(scaled(s, 2))
        else:
            prev.append(s)
    say("  segments: first pass one step up, one down, a hit, empty, two steps")
    after(prev, base, 16384)
