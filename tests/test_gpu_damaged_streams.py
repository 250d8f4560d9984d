"""GPU decoders against the oracle on damaged streams: seeded single-byte
changes spread over every region of a stream (header, chunk table, group
table, code planes, sign+mantissa bytes, escape exponents) and truncations,
at three chunk sizes.  The oracle rejects a whole stream; the GPU decides
per group.  Either both reject or neither does, and an accepted stream
decodes to the oracle's values (a changed code or exponent byte usually
leaves a valid stream with other values).  The fused reduce is held to the
same with a valid stream beside the damaged one.
"""
import numpy as np
import pytest

import oracle
from lossless_bf16_exponent_zc_amd import Plan
from lossless_bf16_exponent_zc_amd import workloads as W

from gpu_util import gpu_decompress, gpu_reduce, say, streams_to_packed

pytestmark = pytest.mark.gpu


def damaged(s: bytes, n_changes: int, seed: int):
    """(description, stream) pairs: one byte changed (XOR with a random
    non-zero value) in each region in turn, and a few truncations."""
    h = oracle.parse_header(s)
    K = h["K"]
    regions = [
        ("header", 0, 64),
        ("chunk table", 64, 64 + 4 * (K + 1)),
        ("group table", 64 + 4 * (K + 1), h["code_off"]),
        ("code planes", h["code_off"], h["sm_off"]),
        ("sign+mantissa", h["sm_off"], h["esc_off"]),
        ("escapes", h["esc_off"], len(s)),
    ]
    regions = [r for r in regions if r[2] > r[1]]
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_changes):
        name, lo, hi = regions[i % len(regions)]
        off = int(rng.integers(lo, hi))
        b = bytearray(s)
        b[off] ^= int(rng.integers(1, 256))
        out.append((f"{name} byte {off}", bytes(b)))
    for cut in (1, 3, 64, int(rng.integers(1, len(s)))):
        out.append((f"truncated by {cut}", s[:len(s) - cut]))
    return out


CASES = [  # (values, chunk)
    (5 * 65536 + 777, 65536),
    (3 * 16384 + 2048 + 5, 16384),
    (7 * 2048 + 300, 2048),
]


@pytest.mark.parametrize("n,chunk", CASES)
def test_damaged_streams_decode(n, chunk):
    x = W.gradient(n, seed=71 + chunk % 7)
    s = oracle.compress(x, C=chunk)
    plan = Plan([n], chunk)
    muts = damaged(s, 90, seed=chunk)
    rejected = 0
    for i, (what, m) in enumerate(muts):
        obits, odec = oracle.decompress_status(m, n, chunk)
        packed = streams_to_packed(plan, [m])
        gbits, dec = gpu_decompress(plan, packed, capacity=len(m))
        assert (obits == 0) == (gbits == 0), (i, what, hex(obits), hex(gbits))
        if obits == 0:
            assert np.array_equal(dec[0], odec), (i, what)
        else:
            rejected += 1
        if i % 30 == 29:
            say(f"  chunk {chunk}: {i + 1} damaged streams, {rejected} rejected by both")
    say(f"  chunk {chunk}: {len(muts)} damaged streams, {rejected} rejected by both")


@pytest.mark.parametrize("n,chunk", CASES[::2])
def test_damaged_streams_reduce(n, chunk):
    x = W.gradient(n, seed=81)
    y = W.gradient(n, seed=82)
    s, t = oracle.compress(x, C=chunk), oracle.compress(y, C=chunk)
    # truncations are left out here: one capacity covers both streams, so a
    # truncated stream would be read past its cut (the decode test covers
    # them, each stream with its own length as the capacity)
    muts = [(w, m) for w, m in damaged(s, 42, seed=chunk + 1) if len(m) == len(s)]
    for i, (what, m) in enumerate(muts):
        cap = max(len(m), len(t))
        obits, _ = oracle.decompress_status(m, n, chunk)
        gbits, got = gpu_reduce([t, m], n, chunk, capacity=cap)
        assert (obits == 0) == (gbits == 0), (i, what, hex(obits), hex(gbits))
        if obits == 0:
            assert np.array_equal(got, oracle.decompress_reduce([t, m], n, chunk)), (i, what)
    say(f"  chunk {chunk}: {len(muts)} damaged shards beside a valid one")
