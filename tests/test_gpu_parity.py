"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Bar: compressed streams byte-identical to the oracle's, window statistics
bit-identical, decompression and decompress-reduce bit-exact.  Inputs are the
seeded generators of lossless_bf16_exponent_zc_amd.workloads at sizes the
oracle finishes in seconds, spanning several chunks and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
from lossless_bf16_exponent_zc_amd import workloads as W

from conftest import assert_same_bytes
from gpu_util import (gpu_compress, gpu_decompress, gpu_reduce, say, stat_bits,
                      streams_to_packed)

pytestmark = pytest.mark.gpu


def check_segments(segs, chunk=65536, window=None):
    say(f"  compress {len(segs)} segment(s), sizes {[s.size for s in segs][:6]}..., chunk {chunk}, L {window}")
    streams, plan, out, ws = gpu_compress(segs, chunk, window)
    for s, (seg, st) in enumerate(zip(segs, streams)):
        ref = oracle.compress(seg, C=chunk, L=window)
        if st != ref:
            a = np.frombuffer(st, np.uint8)
            b = np.frombuffer(ref, np.uint8)
            m = min(a.size, b.size)
            diff = np.nonzero(a[:m] != b[:m])[0]
            raise AssertionError(
                f"segment {s}: stream differs: len {a.size} vs {b.size}, first diffs at "
                f"{diff[:10].tolist()} header {oracle.parse_header(st)} vs {oracle.parse_header(ref)}")
        if window is None:
            got, o = plan.read_sigma(ws, s), oracle.sigma(seg)
            assert stat_bits(got) == stat_bits(o), (s, got, o)
    bits, dec = gpu_decompress(plan, out, ws)
    assert bits == 0, hex(bits)
    for seg, d in zip(segs, dec):
        assert np.array_equal(seg, d)
    return streams, plan


def test_small_config_round_trip():
    check_segments([W.small()])


@pytest.mark.parametrize("n", [1, 7, 8, 9, 511, 2047, 2048, 2049, 4095, 65535, 65536,
                               65537, 3 * 65536 + 12345])
def test_ragged_sizes(n):
    check_segments([W.small(n, seed=n)])


@pytest.mark.parametrize("chunk", [2048, 4096, 8192, 16384, 32768])
def test_chunk_sizes(chunk):
    check_segments([W.gradient(5 * chunk + 777, seed=3)], chunk=chunk)


def test_every_pattern_every_window():
    # all 65,536 patterns, sorted and shuffled, under the window rule and
    # under every forced window L = 1..248: streams byte-identical to the
    # oracle's, round trips exact (one plan and workspace for the sweep)
    from lossless_bf16_exponent_zc_amd import Plan
    from gpu_util import pack_inputs
    allp = np.arange(65536, dtype=np.uint16)
    shuf = np.random.default_rng(6).permutation(allp)
    plan = Plan([allp.size], 8192)
    out, sizes, ws, y = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace(), plan.empty_input()
    for name, x in (("sorted", allp), ("shuffled", shuf)):
        say(f"  {name} patterns, every window")
        check_segments([x], chunk=8192)
        xd = pack_inputs(plan, [x])
        for L in range(1, 249):
            out.fill_(0xA5)
            plan.compress(xd, out, sizes, ws, window=L)
            y.fill_(0x5A5A)
            plan.decompress(out, y, ws)
            bits = plan.read_status(ws)
            n = int(sizes.cpu()[0])
            assert_same_bytes(out[:n].cpu().numpy().tobytes(), oracle.compress(x, C=8192, L=L), f"{name}, L {L}")
            assert bits == 0, (name, L, hex(bits))
            assert np.array_equal(y[:x.size].cpu().numpy().view(np.uint16), x), (name, L)


def test_hand_derived_fixtures():
    # the golden streams and statistics derived by hand (tests/golden), here
    # from the GPU: pins the kernels to the readings themselves, not only to
    # the oracle
    from conftest import check_escape_order_stream, escape_order_input, read_golden
    (g,) = read_golden("escape_order.txt")
    x = escape_order_input(g)
    streams, plan, _, ws = gpu_compress([x], int(g["chunk"]))
    check_escape_order_stream(streams[0], g)
    S1, S2, n, var, L = plan.read_sigma(ws, 0)
    assert (S1, S2, n, var, L) == (float(g["S1"]), float(g["S2"]), int(g["n"]), float(g["var"]),
                                   int(g["L"]))
    (v,) = read_golden("variance_rounding.txt")
    x = np.array([int(t, 16) for t in v["input"].split()], dtype=np.uint16)
    _, plan, _, ws = gpu_compress([x])
    h = lambda k: float(np.float64(float.fromhex(v[k])))
    want = (h("S1"), h("S2"), int(v["n"]), h("var"), int(v["L"]))
    assert stat_bits(plan.read_sigma(ws, 0)) == stat_bits(want)
    for (name, key) in (("fused multiply-add", "var_fma"), ("(S2 - S1 mean) / n", "var_alt")):
        assert stat_bits(plan.read_sigma(ws, 0))[3] != stat_bits((0, 0, 0, h(key), 0))[3], name


def test_damaged_group_table_large_span():
    # chunks of 65,536 values: a group-table entry raised to its chunk's whole
    # escape count gives the group before it a span of thousands of escapes.
    # The decoder must reject those groups before it copies any escape into
    # LDS; the other groups of the same workgroups (4 waves, 4 groups) decode
    # exactly, while the oracle rejects the stream.
    N = 65536 * 2
    x = W.gradient(N, seed=21)  # about 20% escapes: ~13,000 per chunk
    s = oracle.compress(x)
    h = oracle.parse_header(s)
    K = h["K"]
    t0 = int.from_bytes(s[64:68], "little")
    t1 = int.from_bytes(s[68:72], "little")
    assert t1 - t0 > 4096
    goff = 64 + 4 * (K + 1)
    from lossless_bf16_exponent_zc_amd import Plan
    plan = Plan([N])
    for g in (5, 17, 31):  # group g - 1 gets the large span; g itself a negative one
        b = bytearray(s)
        b[goff + 2 * g:goff + 2 * g + 2] = (t1 - t0).to_bytes(2, "little")
        obits, _ = oracle.decompress_status(bytes(b), N)
        assert obits != 0
        bits, dec = gpu_decompress(plan, streams_to_packed(plan, [bytes(b)]))
        say(f"  group table entry {g} = {t1 - t0}: oracle 0x{obits:02x} gpu 0x{bits:02x}")
        assert bits & 0x20  # count
        bad = np.zeros(N // 2048, dtype=bool)
        bad[[g - 1, g]] = True
        got = dec[0].reshape(-1, 2048)
        want = x.reshape(-1, 2048)
        assert np.array_equal(got[~bad], want[~bad]), g
        # the rejected groups wrote nothing (the output keeps its fill)
        assert (got[bad] == 0x5A5A).all(), g
        rbits, rgot = gpu_reduce([bytes(b), s], N)
        assert rbits & 0x20
        sum_ok = oracle.decompress_reduce([s, s], N).reshape(-1, 2048)
        assert np.array_equal(rgot.reshape(-1, 2048)[~bad], sum_ok[~bad]), g


def test_decode_only_workspace():
    # decoders and the fused reduce with a workspace of
    # zc_plan_decode_workspace_bytes (status words + a 2048-byte stand-in)
    from lossless_bf16_exponent_zc_amd import Plan
    for n in (1, 2049, 3 * 65536 + 5):
        x = W.gradient(n, seed=n)
        s = oracle.compress(x)
        plan = Plan([n])
        ws = plan.empty_workspace(decode_only=True)
        assert ws.numel() == plan.decode_workspace_bytes < plan.workspace_bytes
        assert plan.decode_workspace_bytes == (4 * -(-n // 2048) + 255) // 256 * 256 + 2048
        bits, dec = gpu_decompress(plan, streams_to_packed(plan, [s]), ws=ws)
        assert bits == 0 and np.array_equal(dec[0], x), n
        sh = [x, W.gradient(n, seed=n + 1)]
        streams = [oracle.compress(t) for t in sh]
        cap = (max(len(t) for t in streams) + 255) // 256 * 256
        dev = [torch.zeros(cap, dtype=torch.uint8, device="cuda") for _ in streams]
        for d, t in zip(dev, streams):
            d[:len(t)] = torch.from_numpy(np.frombuffer(t, np.uint8).copy()).cuda()
        y = plan.empty_input()
        plan.decompress_reduce(dev, y, ws, capacity=cap)
        assert plan.read_status(ws) == 0
        assert np.array_equal(y[:n].cpu().numpy().view(np.uint16), oracle.decompress_reduce(streams, n))
    # one byte short is refused before anything is enqueued
    from lossless_bf16_exponent_zc_amd import ZcError
    short = torch.empty(plan.decode_workspace_bytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ZcError):
        plan.decompress(streams_to_packed(plan, [s]), plan.empty_input(), short)


@pytest.mark.parametrize("n,S", [(1, 1), (7, 3), (8, 2), (100003, 8), (65536 * 3 + 9, 16)])
def test_reduce_native(n, S):
    # the native path of the reduce-scatter switch: the same sums as the
    # fused reduce of the shards' coded streams and of their raw streams
    import lossless_bf16_exponent_zc_amd as zc
    sh = W.shards(n=n, nshards=S)
    if n > 20:
        sh[0][:10] = [0x7F7F, 0x0001, 0x7F80, 0x7FC1, 0x8000, 0, 0x0080, 0xFF80, 0x3F80, 0x7F7F]
    want = oracle.decompress_reduce([oracle.compress(t) for t in sh], n)
    raw = oracle.decompress_reduce([oracle.compress(t, raw_fallback=True) for t in sh], n)
    assert np.array_equal(want, raw)
    dev = [torch.from_numpy(t.view(np.int16)).cuda() for t in sh]
    out = torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda")
    zc.reduce_native(dev, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


def test_special_tensors():
    n = 70000
    cases = {
        "zeros": np.zeros(n, np.uint16),
        "neg_zeros": np.full(n, 0x8000, np.uint16),
        "nan": np.full(n, 0x7FC0, np.uint16),
        "inf_mix": np.where(np.arange(n) % 3 == 0, 0x7F80, 0x3F80).astype(np.uint16),
        "subnormal": (np.arange(n) % 127 + 1).astype(np.uint16),
        "const": np.full(n, 0x4049, np.uint16),
        "huge": np.full(n, 0x7F7F, np.uint16),
    }
    for name, x in cases.items():
        say(f"  special tensor {name}")
        check_segments([x])


@pytest.mark.parametrize("n", [1, 1000, 1024, 2048, 4096, 16384, 65536, 65537, 131072])
def test_negative_zeros_statistics(n):
    # all -0.0: the sums' sign of zero depends on whether the tree over the
    # segment (padded to a power of two with +0.0) has any padding leaf
    check_segments([np.full(n, 0x8000, np.uint16)])


def test_moe_segments_scaled():
    bits, sizes = W.moe(tokens=4096, hidden=512, experts=64)
    segs, off = [], 0
    for c in sizes:
        segs.append(bits[off:off + c])
        off += c
    segs.insert(3, np.zeros(0, np.uint16))  # an empty segment in the middle
    check_segments(segs)


def test_llama_segments_scaled():
    segs = W.llama_mlp(shapes=((256, 896), (896, 256), (256, 896)))
    check_segments(segs, chunk=16384)


def test_cross_decode_oracle_streams():
    x = W.gradient(300000, seed=11)
    ref = oracle.compress(x)
    from lossless_bf16_exponent_zc_amd import Plan
    plan = Plan([x.size])
    bits, dec = gpu_decompress(plan, streams_to_packed(plan, [ref]))
    assert bits == 0 and np.array_equal(dec[0], x)


def test_determinism():
    # 20 calls, fresh and reused workspaces: the same bytes every time
    x = W.gradient(1 << 20, seed=5)
    first, plan = check_segments([x])
    ws = plan.empty_workspace()
    for i in range(20):
        again, _, _, _ = gpu_compress([x], plan=plan, ws=ws if i % 2 else None)
        assert_same_bytes(again, first, f"call {i}")


def test_decompress_reduce_scaled():
    n = 200000 + 333
    sh = W.shards(n=n, nshards=8)
    sh[2][:10] = [0x0001, 0x8001, 0x7F80, 0, 0x8000, 0x7F7F, 0x7F7F, 0x0080, 0x3F80, 0xFF80]
    sh[5][:10] = [0x0001, 0x0001, 0x3F80, 0, 0x8000, 0x7F7F, 0x7F7F, 0x8080, 0xFF80, 0x7F80]
    streams = [oracle.compress(s) for s in sh]
    ref = oracle.decompress_reduce(streams, n)
    for S in (1, 2, 8):
        say(f"  reduce over {S} shard(s)")
        bits, got = gpu_reduce(streams[:S], n)
        assert bits == 0
        assert np.array_equal(got, oracle.decompress_reduce(streams[:S], n))
    assert np.array_equal(gpu_reduce(streams, n)[1], ref)


def test_reduce_rounding_boundaries():
    # fp32 sums of two shards that land on BF16 rounding ties, just above and
    # just below them (both signs), on overflow (the largest finite value
    # plus half its ulp is a tie that rounds to Inf), on Inf - Inf and on NaNs
    # with payloads; and every pattern against a shuffled copy
    rng = np.random.default_rng(11)
    allp = np.arange(65536, dtype=np.uint16)
    a, b = [allp], [rng.permutation(allp)]
    k = 20000
    e = rng.integers(10, 255, k).astype(np.uint16)
    m = rng.integers(0, 128, k).astype(np.uint16)
    sg = (rng.integers(0, 2, k).astype(np.uint16) << 15).astype(np.uint16)
    x0 = (sg | (e << 7) | m).astype(np.uint16)
    for flip in (0, 0x8000):  # half an ulp added, then subtracted
        for de, dm in ((8, 0), (8, 1), (9, 0x7F)):  # the tie, just above, just below
            a.append(x0)
            b.append(((sg ^ flip) | ((e - de) << 7) | dm).astype(np.uint16))
    sp = [(0x7F7F, 0x7F7F), (0x7F7F, 0x7B00), (0xFF7F, 0xFB00), (0x7F7F, 0x7AFF), (0x7F80, 0xFF80),
          (0x7F80, 0x3F80), (0x7FC1, 0x3F80), (0xFF81, 0x0001), (0x7F81, 0x7F80), (0x0001, 0x8001),
          (0x8000, 0x8000), (0x0000, 0x8000), (0x0080, 0x0001), (0x007F, 0x0001)]
    a.append(np.array([p for p, _ in sp], np.uint16))
    b.append(np.array([q for _, q in sp], np.uint16))
    x0, x1 = np.concatenate(a), np.concatenate(b)
    n = x0.size
    streams = [oracle.compress(x0), oracle.compress(x1)]
    ref = oracle.decompress_reduce(streams, n)
    bits, got = gpu_reduce(streams, n)
    assert bits == 0
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(x0[i]), hex(x1[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]
    # the sums themselves, independently: fp32 adds and the rounding formula
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        acc = (f(x0) + f(x1)).view(np.uint32)
    nan = (acc & 0x7FFFFFFF) > 0x7F800000
    rne = ((acc.astype(np.uint64) + 0x7FFF + ((acc >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(got, np.where(nan, np.uint16(0x7FC0), rne))
    # the same sums through the kernel that walks 9..16 shards in turn
    # (seven all-zero shards after the two)
    zero = oracle.compress(np.zeros(n, np.uint16))
    bits, got9 = gpu_reduce(streams + [zero] * 7, n)
    assert bits == 0
    assert np.array_equal(got9, oracle.decompress_reduce(streams + [zero] * 7, n))


def _mutants(s, N):
    h = oracle.parse_header(s)
    out = []
    def flip(off, val=None, xor=None):
        b = bytearray(s)
        if xor is not None:
            b[off] ^= xor
        else:
            b[off] = val
        return bytes(b)
    out.append(flip(0, xor=1))
    out.append(flip(4, val=2))
    out.append(flip(7, val=1))
    out.append(flip(6, val=0))
    out.append(flip(6, val=249))
    out.append(flip(8, xor=1))
    out.append(flip(40, xor=1))
    out.append(s[:-1])
    out.append(flip(24, xor=1))
    out.append(flip(64 + 4, xor=1))
    out.append(flip(64, val=1))
    out.append(flip(h["code_off"] + 12, xor=1))
    out.append(flip(h["code_off"] + 256 + 12, xor=4))
    out.append(flip(h["sm_off"] + N, val=1))
    out.append(flip(h["sm_off"] - 1, xor=0x80))  # plane bit of a value past N
    return out


def test_rejection_set_matches_oracle():
    N = 3 * 2048 + 100
    x = W.small(N, seed=7)
    s = oracle.compress(x, C=2048)
    from lossless_bf16_exponent_zc_amd import Plan
    plan = Plan([N], 2048)
    for i, m in enumerate(_mutants(s, N)):
        obits, _ = oracle.decompress_status(m, N, 2048)
        packed = streams_to_packed(plan, [m])
        gbits, dec = gpu_decompress(plan, packed, capacity=len(m))
        say(f"  mutant {i}: oracle 0x{obits:02x} gpu 0x{gbits:02x}")
        assert (obits == 0) == (gbits == 0), i
        if obits == 0:
            assert np.array_equal(dec[0], oracle.decompress(m, N, 2048))


def test_reduce_rejection_set_matches_oracle():
    # the fused reduce checks headers and tables with its own (branch-free)
    # code: every mutant, as both shards, at its exact length as the capacity
    N = 3 * 2048 + 100
    x = W.small(N, seed=7)
    s = oracle.compress(x, C=2048)
    for i, m in enumerate(_mutants(s, N)):
        obits, _ = oracle.decompress_status(m, N, 2048)
        gbits, got = gpu_reduce([m, m], N, 2048, capacity=len(m))
        say(f"  reduce mutant {i}: oracle 0x{obits:02x} gpu 0x{gbits:02x}")
        assert (obits == 0) == (gbits == 0), i
        if obits == 0:
            assert np.array_equal(got, oracle.decompress_reduce([m, m], N, 2048))
    # a valid stream beside each mutant: the sum is rejected exactly when
    # the mutant is (the capacity is the valid stream's length: mutants
    # other than the truncation have the same length)
    for i, m in enumerate(_mutants(s, N)):
        if len(m) != len(s):
            continue
        obits, _ = oracle.decompress_status(m, N, 2048)
        gbits, got = gpu_reduce([s, m], N, 2048, capacity=len(s))
        assert (obits == 0) == (gbits == 0), i
        if obits == 0:
            assert np.array_equal(got, oracle.decompress_reduce([s, m], N, 2048))


def test_timed_compress_same_streams():
    # the merged tail (two kernels: us[2] is 0) and the three-kernel tail of
    # a raw-fallback plan (every time positive), same streams as the oracle's
    from lossless_bf16_exponent_zc_amd import Plan
    from gpu_util import pack_inputs
    x = W.gradient(3 * 65536 + 999, seed=12)
    for raw in (False, True):
        plan = Plan([x.size], raw_fallback=raw)
        xd = pack_inputs(plan, [x])
        out, sizes, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
        for _ in range(2):  # a fresh workspace (prediction may fail), then a settled one
            us = plan.compress_timed(xd, out, sizes, ws)
            assert len(us) == 3 and us[0] > 0 and us[1] > 0, us
            assert (us[2] > 0) if raw else (us[2] == 0), (raw, us)
            n = int(sizes.cpu()[0])
            assert_same_bytes(out[:n].cpu().numpy().tobytes(), oracle.compress(x, raw_fallback=raw))


def test_decompress_reduce_more_than_eight_shards():
    # 9..16 shards take the kernel that walks the shards in turn
    n = 70000 + 17
    sh = W.shards(n=n, nshards=16)
    streams = [oracle.compress(s) for s in sh]
    for S in (9, 16):
        say(f"  reduce over {S} shards")
        bits, got = gpu_reduce(streams[:S], n)
        assert bits == 0
        assert np.array_equal(got, oracle.decompress_reduce(streams[:S], n))
