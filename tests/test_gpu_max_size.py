"""The largest segment a plan accepts: 2^32 - 1 values (the plan refuses
2^32, test_abi).  Every 32-bit boundary of the layout is crossed here: group
and chunk indices, escape offsets, stream offsets past 4 GiB, the window's
moment tree over 262,144 blocks (64 reduction rounds).

The oracle cannot compress 4.3 billion values in a test's time, so the
stream is checked against it where it can answer exactly and against the
format's closed forms elsewhere:

* the window statistics (S1, S2, n, var, L), bit for bit, from the oracle's
  sigma over the whole tensor;
* header fields and region offsets against the oracle's closed forms;
* the chunk table against escape counts per chunk taken with plain torch
  integer ops from the definition (exponent outside [L, L+6]);
* five chunks (first, second, middle, the last full one, the partial last
  one), whose code planes, sign+mantissa bytes, group-table entries and
  escape bytes must equal those of the oracle's stream of that chunk alone
  under the same window (a chunk's coding depends only on its values and L);
* the round trip, bit-exact, on the device;
* the decompress-reduce of the stream with itself (x + x in fp32 is 2x,
  exact for finite BF16 values, rounds back to the BF16 of 2x).

Both compress calls are checked: the first, on a fresh workspace, codes the
tensor a second time in the window kernel (its window was not predicted);
the second takes the predicted path; the streams must be identical.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import Plan
from lossless_bf16_exponent_zc_amd import workloads as W

from conftest import assert_same_bytes
from gpu_util import say, stat_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N = (1 << 32) - 1
C = 65536
G_PER_C = C // 2048


def u32s(t):
    return np.frombuffer(t.cpu().numpy().tobytes(), dtype="<u4")


def test_largest_segment():
    say(f"  drawing {N:,} values on the device")
    plan = Plan([N], C)
    x = plan.empty_input()
    x[:N] = W.gaussian_device(N, seed=3)
    x[N:] = 0
    out, sizes, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    ws.fill_(0x7B)  # a fresh, garbage-filled workspace: the window is not predicted
    plan.compress(x, out, sizes, ws)
    torch.cuda.synchronize()
    total = int(sizes.cpu()[0])
    first = out[:total].clone()
    plan.compress(x, out, sizes, ws)  # predicted window
    torch.cuda.synchronize()
    assert int(sizes.cpu()[0]) == total
    assert torch.equal(out[:total], first), "predicted and re-coded streams differ"
    del first
    say(f"  compressed to {total:,} bytes (ratio {2 * N / total:.4f}), both calls identical")

    host = x[:N].cpu().numpy().view(np.uint16)
    say("  oracle sigma over the whole tensor")
    ref = oracle.sigma(host)
    got = plan.read_sigma(ws)
    assert stat_bits(got) == stat_bits(ref), (got, ref)
    L = int(ref[4])

    h = oracle.parse_header(out[:64].cpu().numpy().tobytes())
    K = (N + C - 1) // C
    assert (h["magic"], h["version"], h["L"], h["flags"]) == (0x3142435A, 1, L, 0)
    assert (h["N"], h["C"], h["K"]) == (N, C, K)
    assert h["code_off"] == oracle.code_off(N, C) and h["sm_off"] == oracle.sm_off(N, C)
    assert h["esc_off"] == oracle.esc_off(N, C) and h["total"] == total
    assert total == h["esc_off"] + h["E"]

    say("  escape counts per chunk from the definition")
    e = x[:N].to(torch.int32)
    e >>= 7
    e &= 0xFF  # the biased exponent (the sign bit drops out of the low byte)
    esc = (e < L) | (e > L + 6)
    del e
    full = (K - 1) * C
    per_chunk = torch.cat([esc[:full].view(K - 1, C).sum(dim=1), esc[full:].sum().view(1)])
    del esc
    table = u32s(out[64:64 + 4 * (K + 1)]).astype(np.int64)
    expect = np.concatenate([[0], np.cumsum(per_chunk.cpu().numpy())])
    assert np.array_equal(table, expect)
    assert int(expect[-1]) == h["E"]

    gtab_off = 64 + 4 * (K + 1)
    for k in (0, 1, K // 2, K - 2, K - 1):
        lo, hi = k * C, min(N, (k + 1) * C)
        sub = oracle.compress(host[lo:hi], C=C, L=L)
        sh = oracle.parse_header(sub)
        gs = (hi - lo + 2047) // 2048
        g0 = k * G_PER_C
        pairs = (
            (h["code_off"] + 768 * g0, sh["code_off"], 768 * gs, "codes"),
            (h["sm_off"] + 2048 * g0, sh["sm_off"], 2048 * gs, "sign+mantissa"),
            (gtab_off + 2 * g0, 64 + 8, 2 * gs, "group table"),
            (h["esc_off"] + int(table[k]), sh["esc_off"], sh["E"], "escapes"),
        )
        for a, b, n, what in pairs:
            mine = out[a:a + n].cpu().numpy().tobytes()
            assert_same_bytes(mine, sub[b:b + n], f"chunk {k}: {what}")
        assert int(table[k + 1] - table[k]) == sh["E"]
    say("  sampled chunks identical to the oracle's")
    del host

    y = plan.empty_input()
    plan.decompress(out, y, ws)
    assert plan.read_status(ws) == 0
    assert torch.equal(y[:N], x[:N]), "round trip not exact"
    say("  round trip exact")

    y.fill_(0x5A5A)
    plan.decompress_reduce([out], y, ws, capacity=out.numel())
    assert plan.read_status(ws) == 0
    assert torch.equal(y[:N], x[:N]), "one-stream reduce is not the identity"
    plan.decompress_reduce([out, out], y, ws, capacity=out.numel())
    assert plan.read_status(ws) == 0
    twice = (x[:N].view(torch.bfloat16).float() * 2).to(torch.bfloat16).view(torch.int16)
    assert torch.equal(y[:N], twice), "x + x differs from 2x"
    say("  reduce over one and two streams exact")
