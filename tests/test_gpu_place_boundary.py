"""GPU parity at the placement's LDS-buffer edge.

A placement workgroup gathers its chunk's escape run in LDS at the run's
final alignment modulo 16 and stores it in whole 16-byte blocks when
(offset mod 16) + run length fits the buffer (19,584 bytes for chunks of
32,768 and 65,536 values); a longer run goes out group by group from the
staging slots instead.  These tests build chunks whose runs end exactly at
that edge, one byte before and one byte past it, for several alignments,
and check the streams byte by byte against the oracle on the held-
prediction, failed-prediction and caller-fixed-window paths.

The values: every value not chosen to escape has exponent 127 (magnitude
in [1, 2)), which the window of such a tensor always holds; the escapes are
zeros (exponent 0), placed at seeded positions, so each chunk's escape
count is exactly what the test asks for.
"""
import numpy as np
import pytest

import oracle
from lossless_bf16_exponent_zc_amd import Plan

from conftest import assert_same_bytes
from gpu_util import gpu_compress, gpu_decompress, say

pytestmark = pytest.mark.gpu

BUF = 19584  # the gather buffer of 32,768- and 65,536-value chunks


def build(chunk, counts, seed):
    """One segment of len(counts) chunks; chunk k holds counts[k] zeros."""
    rng = np.random.default_rng(seed)
    n = chunk * len(counts)
    sign = rng.integers(0, 2, n).astype(np.uint16) << 15
    mant = rng.integers(0, 128, n).astype(np.uint16)
    x = (sign | (127 << 7) | mant).astype(np.uint16)
    for k, c in enumerate(counts):
        pos = rng.choice(chunk, size=c, replace=False) + k * chunk
        x[pos] = 0
    return x


def chunk_escapes(stream, k):
    tab = np.frombuffer(stream, np.uint32, count=k + 1, offset=64)
    return np.diff(tab.astype(np.int64))


CASES = []
for C in (32768, 65536):
    for off in (0, 1, 7, 15):
        for d in (-1, 0, 1):
            CASES.append((C, off, d))


@pytest.mark.parametrize("C,off,d", CASES)
def test_run_at_buffer_edge(C, off, d):
    # chunk 0 leaves the run of chunk 1 at offset `off` mod 16 (its escape
    # count is 16 q + off); chunk 1's run ends d bytes past the buffer's end
    c0 = 16 * 97 + off
    c1 = BUF - off + d
    counts = [c0, c1, 300]
    x = build(C, counts, seed=C + 16 * off + d + 1)
    ref = oracle.compress(x, C=C)
    assert list(chunk_escapes(ref, len(counts))) == counts  # the construction holds
    L = oracle.parse_header(ref)["L"]
    assert L <= 127 <= L + 6
    say(f"  C={C} off={off} d={d}: escapes per chunk {counts}, window {L}")
    plan = Plan([x.size], C)
    ws = plan.empty_workspace()
    ws.fill_(0x3D)
    # a first call on another tensor, so the next call's prediction fails
    other = (x ^ 0x0080).astype(np.uint16)  # exponent 127 -> 126 and 0 -> 1: another window or other escapes
    gpu_compress([other], C, plan=plan, ws=ws)
    for call in ("after another tensor", "predicted"):
        streams, _, out, _ = gpu_compress([x], C, plan=plan, ws=ws)
        assert_same_bytes(streams[0], ref, f"{call}")
        bits, dec = gpu_decompress(plan, out)
        assert bits == 0 and np.array_equal(dec[0], x), call
    streams, _, _, _ = gpu_compress([x], C, window=L, plan=plan, ws=ws)
    assert_same_bytes(streams[0], oracle.compress(x, C=C, L=L), "caller-fixed window")
