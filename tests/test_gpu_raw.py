"""GPU parity of raw streams: plans with the raw fallback against the oracle.

A raw stream stores a tensor's words after the 64-byte header (flags 1).
Compression picks it, for plans made with the raw fallback, when the coded
stream would be longer.  This is the ZipCCL notes' switch between the
compressed and the native path by compression benefit ("Key idea and
contribution", third technique), taken per stream.  Bar: streams
byte-identical to oracle.compress(..., raw_fallback=True); decompression and
decompress-reduce bit-exact over raw and coded streams alike.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import Plan, workloads as W
from lossless_bf16_exponent_zc_amd.binding import ZcError

from gpu_util import (gpu_compress, gpu_decompress, gpu_reduce, pack_inputs, say,
                      streams_to_packed)

pytestmark = pytest.mark.gpu


def uniform(n, seed):
    """Uniform bit patterns (no Inf/NaN): about 97% of exponents escape."""
    x = np.random.default_rng(seed).integers(0, 65536, n, dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80
    return x


def check_raw(segs, chunk=65536, window=None, plan=None, ws=None):
    say(f"  raw-fallback compress {len(segs)} segment(s), sizes {[s.size for s in segs][:6]}, "
        f"chunk {chunk}, L {window}")
    plan = plan or Plan([s.size for s in segs], chunk, raw_fallback=True)
    streams, plan, out, ws = gpu_compress(segs, chunk, window, plan=plan, ws=ws)
    kinds = []
    for s, (seg, st) in enumerate(zip(segs, streams)):
        ref = oracle.compress(seg, C=chunk, L=window, raw_fallback=True)
        if st != ref:
            a, b = np.frombuffer(st, np.uint8), np.frombuffer(ref, np.uint8)
            m = min(a.size, b.size)
            diff = np.nonzero(a[:m] != b[:m])[0]
            raise AssertionError(f"segment {s}: len {a.size} vs {b.size}, first diffs "
                                 f"{diff[:10].tolist()}, header {oracle.parse_header(st)} vs "
                                 f"{oracle.parse_header(ref)}")
        kinds.append(oracle.parse_header(st)["flags"])
    bits, dec = gpu_decompress(plan, out)
    assert bits == 0, hex(bits)
    for seg, d in zip(segs, dec):
        assert np.array_equal(seg, d)
    return kinds, streams, plan, ws


@pytest.mark.parametrize("n,chunk", [(1, 2048), (7, 2048), (1000, 2048), (2047, 65536),
                                     (5000, 2048), (65536, 65536), (3 * 65536 + 12345, 65536),
                                     (5 * 8192 + 3, 8192)])
def test_zeros_and_uniform_go_raw(n, chunk):
    kinds, *_ = check_raw([np.zeros(n, np.uint16), uniform(n, n)], chunk)
    assert kinds == [1, 1]


def test_empty_segment_is_a_bare_header():
    kinds, streams, *_ = check_raw([np.zeros(0, np.uint16), W.small(70001, seed=2)])
    assert kinds == [1, 0] and len(streams[0]) == 64


@pytest.mark.parametrize("n,kind", [(1, 1), (1500, 1), (2048, 0), (4096, 0), (3 * 2048 + 5, 1),
                                    (65536, 0), (200003, 0)])
def test_gradient_tensors_pick_the_shorter(n, kind):
    # the coded form's fixed regions take 2816 bytes per started 2048-value
    # group: tiny tensors, and a last group of 5 values, tip it to raw
    kinds, *_ = check_raw([W.gradient(n, seed=n)], 2048)
    assert kinds == [kind]


@pytest.mark.parametrize("extra", [0, 1])
def test_break_even_with_a_fixed_window(extra):
    # window 127: 1.0 codes, 0x0001 escapes; 4928 escapes in 8192 values tie
    N, E = 8192, 4928 + extra
    x = np.full(N, 0x3F80, dtype=np.uint16)
    x[np.random.default_rng(3).permutation(N)[:E]] = 0x0001
    kinds, streams, *_ = check_raw([x], 8192, window=127)
    assert kinds == [extra] and len(streams[0]) == 16448


def test_mixed_segments_in_one_launch():
    segs = [W.gradient(70000, seed=1), np.zeros(5000, np.uint16), uniform(3000, 4),
            np.zeros(0, np.uint16), W.gradient(1, seed=5), W.gradient(200000, seed=6),
            uniform(2 * 65536 + 9, 7)]
    kinds, *_ = check_raw(segs, 65536)
    assert kinds == [0, 1, 1, 1, 1, 0, 1]


def test_prediction_across_raw_and_coded_calls():
    # one workspace: coded, then raw (the window moves: the window kernel
    # codes the segment again and its last workgroup picks raw), then coded
    n = 5 * 65536 + 99
    plan = Plan([n], 65536, raw_fallback=True)
    ws = plan.empty_workspace()
    for i, x in enumerate([W.gradient(n, seed=10), np.zeros(n, np.uint16), uniform(n, 11),
                           W.gradient(n, seed=12), W.gradient(n, seed=12)]):
        say(f"  call {i}")
        kinds, *_ = check_raw([x], 65536, plan=plan, ws=ws)
        assert kinds == [[0, 1, 1, 0, 0][i]]


def test_split_refuses_raw_fallback_plans():
    n = 70000
    plan = Plan([n], raw_fallback=True)
    x = pack_inputs(plan, [W.gradient(n, seed=1)])
    ev = torch.cuda.Event()
    ev.record()  # the event exists: the refusal is the plan's flag
    with pytest.raises(ZcError):
        plan.compress_split(x, plan.empty_output(), plan.empty_sizes(), plan.empty_workspace(), ev)


@pytest.mark.parametrize("nshards", [3, 8, 12])
def test_reduce_over_raw_and_coded_shards(nshards):
    n = 70000 + 17
    sh = W.shards(n=n, nshards=nshards)
    for s in range(1, nshards, 3):  # every third shard is near-uniform: raw
        sh[s] = uniform(n, 100 + s)
    streams = [oracle.compress(s, raw_fallback=True) for s in sh]
    flags = [oracle.parse_header(t)["flags"] for t in streams]
    assert 0 in flags and 1 in flags
    say(f"  reduce {nshards} shards, raw {flags}")
    bits, got = gpu_reduce(streams, n)
    assert bits == 0, hex(bits)
    assert np.array_equal(got, oracle.decompress_reduce(streams, n))


def test_raw_header_rejections_match_the_oracle():
    N = 3000
    x = uniform(N, 5)
    s = oracle.compress(x, C=2048, raw_fallback=True)
    assert oracle.parse_header(s)["flags"] == 1
    plan = Plan([N], 2048)
    muts = [s, s[:-1]]
    for off, xor in [(0, 1), (4, 2), (6, 5), (7, 3), (8, 1), (16, 1), (20, 1), (24, 1), (32, 1),
                     (40, 1), (48, 16), (56, 1)]:
        b = bytearray(s)
        b[off] ^= xor
        muts.append(bytes(b))
    for i, m in enumerate(muts):
        obits, _ = oracle.decompress_status(m, N, 2048)
        gbits, dec = gpu_decompress(plan, streams_to_packed(plan, [m]), capacity=len(m))
        say(f"  mutant {i}: oracle 0x{obits:02x} gpu 0x{gbits:02x}")
        assert (obits == 0) == (gbits == 0), i
        if obits == 0:
            assert np.array_equal(dec[0], x)
        elif i > 1 and obits != oracle.FMT_MAGIC:  # one field changed: the same bit
            assert gbits == obits, i


def test_reduce_raw_header_rejections_match_the_oracle():
    # the fused reduce's own header check on raw streams: each mutant as both
    # shards, at its exact length as the capacity
    N = 3000
    x = uniform(N, 5)
    s = oracle.compress(x, C=2048, raw_fallback=True)
    muts = [s, s[:-1]]
    for off, xor in [(0, 1), (4, 2), (6, 5), (7, 3), (8, 1), (16, 1), (20, 1), (24, 1), (32, 1),
                     (40, 1), (48, 16), (56, 1)]:
        b = bytearray(s)
        b[off] ^= xor
        muts.append(bytes(b))
    for i, m in enumerate(muts):
        obits, _ = oracle.decompress_status(m, N, 2048)
        gbits, got = gpu_reduce([m, m], N, 2048, capacity=len(m))
        say(f"  reduce mutant {i}: oracle 0x{obits:02x} gpu 0x{gbits:02x}")
        assert (obits == 0) == (gbits == 0), i
        if obits == 0:
            assert np.array_equal(got, oracle.decompress_reduce([m, m], N, 2048))
        elif i > 1 and obits != oracle.FMT_MAGIC:  # one field changed: the same bit
            assert gbits == obits, i


def test_large_raw_tensor():
    # 2^22 zeros plus a ragged tail: the placement kernel's raw copy over 64 chunks
    n = (1 << 22) + 5
    kinds, *_ = check_raw([np.zeros(n, np.uint16)])
    assert kinds == [1]
