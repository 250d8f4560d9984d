"""GPU parity with calls in flight together.  The C ABI lets calls that share
no workspace overlap (zc.h, conventions); here two plans, each with its own
workspace, compress, decompress and reduce on two streams with nothing
synchronising them, so their kernels can run side by side on the device.
The compress tail's waits between workgroups of one launch (window parts,
verdict, chunk counts) only ever wait on lower-indexed workgroups of the
same launch, which another launch's workgroups cannot hold back forever;
every stream must still be byte-identical to the oracle's, every round trip
exact and every reduce equal to the oracle's fixed-order sum.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import Plan
from lossless_bf16_exponent_zc_amd import workloads as W

from conftest import assert_same_bytes
from gpu_util import pack_inputs, say, stat_bits
from test_gpu_prediction import scaled

pytestmark = pytest.mark.gpu


def gate(*streams):
    """Hold the streams until a short spin kernel on another stream ends
    (about a millisecond), so that the work enqueued on them next is all
    queued before any of it starts: launched from Python one call at a
    time, the kernels would otherwise each end before the next is queued."""
    g = torch.cuda.Stream()
    with torch.cuda.stream(g):
        torch.cuda._sleep(2_000_000)
        ev = torch.cuda.Event()
        ev.record(g)
    for s in streams:
        s.wait_event(ev)


class Side:
    """One plan with its own buffers and workspace, used on one stream."""

    def __init__(self, variants, chunk):
        # variants: list of segment lists, all with the same segment sizes
        self.variants = variants
        self.chunk = chunk
        self.plan = Plan([s.size for s in variants[0]], chunk)
        self.x = [pack_inputs(self.plan, segs) for segs in variants]
        self.ref = [[oracle.compress(s, C=chunk) for s in segs] for segs in variants]
        self.out = self.plan.empty_output()
        self.sizes = self.plan.empty_sizes()
        self.ws = self.plan.empty_workspace()
        self.ws.fill_(0x5B)  # garbage: the first call's prediction is whatever it reads
        self.y = self.plan.empty_input()
        self.stream = torch.cuda.Stream()

    def prepare(self):
        # on the default stream; the caller synchronises before any launch
        self.out.fill_(0xA5)
        self.y.fill_(0x5A5A)

    def launch(self, v):
        with torch.cuda.stream(self.stream):
            self.plan.compress(self.x[v], self.out, self.sizes, self.ws)
            self.plan.decompress(self.out, self.y, self.ws)

    def check(self, v, what):
        plan, segs = self.plan, self.variants[v]
        assert plan.read_status(self.ws, stream=self.stream) == 0, what
        sz = self.sizes.cpu().numpy()
        host = self.out.cpu().numpy()
        y = self.y.cpu().numpy().view(np.uint16)
        for s, seg in enumerate(segs):
            off = plan.stream_offset(s)
            assert_same_bytes(host[off:off + int(sz[s])].tobytes(), self.ref[v][s], f"{what}, segment {s}")
            io = plan.input_offset(s)
            assert np.array_equal(y[io:io + seg.size], seg), (what, s)


def test_two_streams_compress_decompress():
    # side A: one segment whose window moves one binade every call (every
    # call after the first codes each chunk again in the tail); side B:
    # three segments of other sizes and a smaller chunk, whose prediction
    # holds after the first call
    a0 = W.gradient(6_000_003, seed=3)
    A = Side([[a0], [scaled(a0, 1)]], 65536)
    b = [W.mixed(1_500_000, 11), W.gradient(2_500_001, seed=4), W.small(700_001, seed=5)]
    B = Side([b], 16384)
    for call in range(4):
        va = call % 2
        say(f"call {call}: side A variant {va}, side B")
        A.prepare()
        B.prepare()
        torch.cuda.synchronize()
        gate(A.stream, B.stream)
        A.launch(va)
        B.launch(0)
        torch.cuda.synchronize()
        A.check(va, f"A call {call}")
        B.check(0, f"B call {call}")
        assert stat_bits(A.plan.read_sigma(A.ws, 0)) == stat_bits(oracle.sigma(A.variants[va][0])), call
        for s, seg in enumerate(b):
            assert stat_bits(B.plan.read_sigma(B.ws, s)) == stat_bits(oracle.sigma(seg)), (call, s)


def test_reduce_beside_compress():
    # two fused reduces of 8 shards in a row on one stream while a compress
    # that misses its prediction, then a decompress, run on another
    n = 1_048_579
    sh = W.shards(n=n, nshards=8)
    streams = [oracle.compress(t) for t in sh]
    want = oracle.decompress_reduce(streams, n)
    cap = (max(len(t) for t in streams) + 255) // 256 * 256
    dev = [torch.zeros(cap, dtype=torch.uint8, device="cuda") for _ in streams]
    for d, t in zip(dev, streams):
        d[:len(t)] = torch.from_numpy(np.frombuffer(t, np.uint8).copy()).cuda()
    rplan = Plan([n])
    rws = rplan.empty_workspace(decode_only=True)
    ry = rplan.empty_input()
    rs = torch.cuda.Stream()
    a0 = W.gradient(4_194_305, seed=6)
    A = Side([[a0], [scaled(a0, -1)]], 65536)
    for call in range(3):
        say(f"call {call}: reduce beside compress")
        va = call % 2
        ry.fill_(0x5A5A)
        A.prepare()
        torch.cuda.synchronize()
        gate(A.stream, rs)
        with torch.cuda.stream(rs):
            rplan.decompress_reduce(dev, ry, rws, capacity=cap)
        A.launch(va)
        with torch.cuda.stream(rs):
            rplan.decompress_reduce(dev, ry, rws, capacity=cap)
        torch.cuda.synchronize()
        assert rplan.read_status(rws, stream=rs) == 0, call
        assert np.array_equal(ry[:n].cpu().numpy().view(np.uint16), want), call
        A.check(va, f"A call {call}")
