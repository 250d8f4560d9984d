"""Helpers for GPU tests: run the HIP library through its C ABI on host data."""
import sys

import numpy as np
import torch

from lossless_bf16_exponent_zc_amd import Plan


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def stat_bits(stats):
    """(S1, S2, n, var, L) with the floats as their IEEE bit patterns, so
    that a comparison also tells +0.0 from -0.0."""
    S1, S2, n, var, L = stats
    f = lambda v: int(np.float64(v).view(np.uint64))
    return (f(S1), f(S2), int(n), f(var), int(L))


def to_device(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def pack_inputs(plan: Plan, segs) -> torch.Tensor:
    x = plan.empty_input()
    for s, seg in enumerate(segs):
        if seg.size:
            off = plan.input_offset(s)
            x[off:off + seg.size] = to_device(seg)
    return x


def gpu_compress(segs, chunk=65536, window=None, plan=None, ws=None):
    """Compress a list of uint16 arrays (one per segment) on the GPU.
    Returns (list of stream bytes, plan, packed device output)."""
    plan = plan or Plan([s.size for s in segs], chunk)
    x = pack_inputs(plan, segs)
    out = plan.empty_output()
    out.fill_(0xA5)  # garbage, so bytes the kernels forget to write show up
    sizes = plan.empty_sizes()
    ws = plan.empty_workspace() if ws is None else ws
    plan.compress(x, out, sizes, ws, window=window)
    torch.cuda.synchronize()
    sz = sizes.cpu().numpy()
    host = out.cpu().numpy()
    streams = [host[plan.stream_offset(s):plan.stream_offset(s) + int(sz[s])].tobytes()
               for s in range(len(segs))]
    return streams, plan, out, ws


def gpu_decompress(plan, comp: torch.Tensor, ws=None, capacity=None):
    ws = plan.empty_workspace() if ws is None else ws
    y = plan.empty_input()
    y.fill_(0x5A5A)
    plan.decompress(comp, y, ws, capacity=capacity)
    bits = plan.read_status(ws)
    yh = y.cpu().numpy().view(np.uint16)
    segs = [yh[plan.input_offset(s):plan.input_offset(s) + n].copy()
            for s, n in enumerate(plan.segment_elems)]
    return bits, segs


def streams_to_packed(plan: Plan, streams) -> torch.Tensor:
    """Place host stream bytes at the plan's stream offsets on the device."""
    buf = np.zeros(plan.out_bytes, dtype=np.uint8)
    for s, b in enumerate(streams):
        off = plan.stream_offset(s)
        buf[off:off + len(b)] = np.frombuffer(b, dtype=np.uint8)
    return torch.from_numpy(buf).cuda()


def gpu_reduce(streams, n, chunk=65536, capacity=None):
    """Decode + sum single-segment host streams on the GPU.  capacity: the
    readable bytes the kernels are told of (default: the longest stream,
    rounded up to 256); the buffers are allocated rounded up to 256."""
    plan = Plan([n], chunk)
    cap = capacity if capacity is not None else (max(len(s) for s in streams) + 255) // 256 * 256
    alloc = (max([cap] + [len(s) for s in streams]) + 255) // 256 * 256
    dev = []
    for b in streams:
        t = torch.zeros(alloc, dtype=torch.uint8, device="cuda")
        t[:len(b)] = torch.from_numpy(np.frombuffer(b, dtype=np.uint8).copy()).cuda()
        dev.append(t)
    ws = plan.empty_workspace()
    y = plan.empty_input()
    y.fill_(0x5A5A)
    plan.decompress_reduce(dev, y, ws, capacity=cap)
    bits = plan.read_status(ws)
    return bits, y.cpu().numpy().view(np.uint16)[:n].copy()
