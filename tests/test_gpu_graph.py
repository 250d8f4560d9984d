"""GPU parity under HIP graph capture: compress, decompress and the fused
decompress-and-sum launch only kernels (no allocation, copy, fill or host
synchronisation), so a caller can capture them once and replay them.  Each
replay runs on new input written into the captured buffers, with eager work
and synchronisations between replays, and must give the oracle's streams and
the eager calls' outputs, also when the window moves between replays (the
captured encoder then codes again on the device), at several chunk sizes and
with a window fixed by the caller.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import Plan
from lossless_bf16_exponent_zc_amd import workloads as W

from conftest import assert_same_bytes
from gpu_util import pack_inputs, say, to_device

pytestmark = pytest.mark.gpu

SIZES = [300_000, 2 * 65536 + 77, 4096, 1]


def shifted(x: np.ndarray, binades: int) -> np.ndarray:
    """Move every normal value's exponent by `binades` (kept normal)."""
    e = (x >> 7) & 0xFF
    normal = (e >= 1) & (e <= 254)
    ne = np.clip(e.astype(np.int32) + binades, 1, 254).astype(np.uint16)
    return np.where(normal, (x & 0x807F) | (ne << 7), x).astype(np.uint16)


def inputs(replay: int):
    shift = [0, 12, 12, -7, 0][replay]
    return [shifted(W.gradient(n, seed=100 + 10 * replay + s), shift)
            for s, n in enumerate(SIZES)]


def streams_of(plan, out, sizes):
    sz = sizes.cpu().numpy()
    host = out.cpu().numpy()
    return [host[plan.stream_offset(s):plan.stream_offset(s) + int(sz[s])].tobytes()
            for s in range(plan.num_segments)]


@pytest.mark.parametrize("chunk,window", [(65536, None), (2048, None), (16384, 130)])
def test_captured_round_trip_replays(chunk, window):
    plan = Plan(SIZES, chunk)
    x = plan.empty_input()
    out, sizes, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    y, ws_d = plan.empty_input(), plan.empty_workspace()
    out_e, sizes_e, ws_e = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    y_e, ws_de = plan.empty_input(), plan.empty_workspace()
    for t in (ws, ws_d, ws_e, ws_de):
        t.zero_()

    x.copy_(pack_inputs(plan, inputs(0)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        plan.compress(x, out, sizes, ws, window=window)
        plan.decompress(out, y, ws_d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.compress(x, out, sizes, ws, window=window)
        plan.decompress(out, y, ws_d)
    torch.cuda.synchronize()

    for r in range(5):
        segs = inputs(r)
        say(f"  replay {r}: sizes {SIZES}, chunk {chunk}, window {window}, shift {[0, 12, 12, -7, 0][r]}")
        x.copy_(pack_inputs(plan, segs))
        out.fill_(0xA5)
        y.fill_(0x5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()

        plan.compress(x, out_e, sizes_e, ws_e, window=window)  # eager, between replays
        plan.decompress(out_e, y_e, ws_de)
        torch.cuda.synchronize()

        got = streams_of(plan, out, sizes)
        assert_same_bytes(got, streams_of(plan, out_e, sizes_e), f"replay {r}: graph and eager streams")
        for s, seg in enumerate(segs):
            assert_same_bytes(got[s], oracle.compress(seg, C=chunk, L=window), f"replay {r}, segment {s}")
        assert plan.read_status(ws_d) == 0
        for s, n in enumerate(SIZES):
            o = plan.input_offset(s)
            assert torch.equal(y[o:o + n], x[o:o + n]), f"replay {r}, segment {s}: graph round trip"
            assert torch.equal(y_e[o:o + n], x[o:o + n]), f"replay {r}, segment {s}: eager round trip"


def test_captured_reduce_replays():
    n, P = 5 * 65536 + 321, 5
    plan = Plan([n])
    cap = (oracle.max_stream_bytes(n) + 255) // 256 * 256
    bufs = [torch.zeros(cap, dtype=torch.uint8, device="cuda") for _ in range(P)]
    y, ws = plan.empty_input(), plan.empty_workspace()
    y_e, ws_e = plan.empty_input(), plan.empty_workspace()

    def load(r):
        shards = [W.gradient(n, seed=300 + 10 * r + p) for p in range(P)]
        streams = [oracle.compress(s) for s in shards]
        for b, st in zip(bufs, streams):
            b.zero_()
            b[:len(st)] = torch.from_numpy(np.frombuffer(st, dtype=np.uint8).copy()).cuda()
        return streams

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.decompress_reduce(bufs, y, ws, capacity=cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.decompress_reduce(bufs, y, ws, capacity=cap)
    torch.cuda.synchronize()

    for r in range(4):
        say(f"  reduce replay {r}: {P} shards of {n}")
        streams = load(r)
        y.fill_(0x5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        plan.decompress_reduce(bufs, y_e, ws_e, capacity=cap)
        torch.cuda.synchronize()
        want = to_device(oracle.decompress_reduce(streams, n))
        assert plan.read_status(ws) == 0
        assert torch.equal(y[:n], want), f"replay {r}: graph sum differs from the oracle"
        assert torch.equal(y_e[:n], want), f"replay {r}: eager sum differs from the oracle"
