"""Seeded random plans on the GPU against the oracle.

Each plan draws its segment count (1..8), segment sizes (empty, tiny,
ragged, several chunks), chunk size (2048..65536), the raw-fallback flag
and each segment's values (workloads.mixed: Gaussian of a random scale,
with or without injected zeros, subnormals, Inf and NaN, or uniform bit
patterns) from one seed.  Every stream must be byte-identical to the
oracle's on a garbage-filled workspace (windows not predicted) and again on
the same workspace (predicted); statistics of coded segments bit-identical;
round trips exact.  Single-segment plans also run the fused reduce of the
segment's stream with a second one against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import Plan
from lossless_bf16_exponent_zc_amd import workloads as W

from gpu_util import gpu_compress, gpu_decompress, gpu_reduce, say, stat_bits

pytestmark = pytest.mark.gpu


def draw_plan(seed):
    rng = np.random.default_rng(seed)
    nseg = int(rng.integers(1, 9))
    chunk = 1 << int(rng.integers(11, 17))
    raw = bool(rng.random() < 0.3)
    sizes = []
    for _ in range(nseg):
        r = rng.random()
        if r < 0.1:
            sizes.append(0)
        elif r < 0.3:
            sizes.append(int(rng.integers(1, 200)))
        elif r < 0.6:
            sizes.append(int(rng.integers(200, 20000)))
        else:
            sizes.append(int(rng.integers(20000, 300000)))
    segs = [W.mixed(n, seed * 100 + i) for i, n in enumerate(sizes)]
    return segs, chunk, raw


@pytest.mark.parametrize("seed", range(24))
def test_random_plan(seed):
    segs, chunk, raw = draw_plan(seed)
    say(f"  seed {seed}: {len(segs)} segment(s) {[s.size for s in segs]}, chunk {chunk}, raw {raw}")
    plan = Plan([s.size for s in segs], chunk, raw_fallback=raw)
    ws = plan.empty_workspace()
    ws.fill_(0x5C)
    refs = [oracle.compress(s, C=chunk, raw_fallback=raw) for s in segs]
    for call in ("fresh", "predicted"):
        streams, plan, out, ws = gpu_compress(segs, chunk, plan=plan, ws=ws)
        for i, (a, b) in enumerate(zip(streams, refs)):
            assert a == b, f"{call}: segment {i} of {len(segs)} differs ({len(a)} vs {len(b)} bytes)"
        for i, (seg, b) in enumerate(zip(segs, refs)):
            if oracle.parse_header(b)["flags"] == 0:
                assert stat_bits(plan.read_sigma(ws, i)) == stat_bits(oracle.sigma(seg)), (call, i)
    bits, dec = gpu_decompress(plan, out)
    assert bits == 0, hex(bits)
    for seg, d in zip(segs, dec):
        assert np.array_equal(seg, d)
    if len(segs) == 1 and segs[0].size:
        n = segs[0].size
        other = oracle.compress(W.mixed(n, seed + 7777), C=chunk, raw_fallback=raw)
        rbits, got = gpu_reduce([refs[0], other], n, chunk)
        assert rbits == 0
        assert np.array_equal(got, oracle.decompress_reduce([refs[0], other], n, C=chunk))
