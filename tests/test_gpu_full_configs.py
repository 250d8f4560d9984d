"""GPU parity at the full sizes of the workloads, in the launch configuration
the benchmark times (one plan per workload, 65,536-value chunks): every
stream byte-identical to the oracle's, window statistics bit-identical,
round trips bit-exact, and the fixed-order reduce bit-exact against the
oracle's.  The 1,048,576-value workload is in test_gpu_parity.

The oracle runs segment by segment in a thread pool (its C calls release the
interpreter lock).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from lossless_bf16_exponent_zc_amd import workloads as W

from conftest import assert_same_bytes
from gpu_util import gpu_compress, gpu_decompress, gpu_reduce, say, stat_bits

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CHUNK = 65536


def pool_map(fn, items):
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        return list(ex.map(fn, items))


def check_full(segs, name):
    say(f"  {name}: {len(segs)} segment(s), {sum(s.size for s in segs):,} values")
    streams, plan, out, ws = gpu_compress(segs, CHUNK)
    refs = pool_map(lambda s: oracle.compress(s, C=CHUNK), segs)
    for s, (a, b) in enumerate(zip(streams, refs)):
        if a != b:
            x, y = np.frombuffer(a, np.uint8), np.frombuffer(b, np.uint8)
            m = min(x.size, y.size)
            d = np.nonzero(x[:m] != y[:m])[0]
            raise AssertionError(f"{name} segment {s}: {x.size} vs {y.size} bytes, "
                                 f"first differences at {d[:8].tolist()}")
    say(f"  {name}: streams identical ({sum(len(r) for r in refs):,} bytes)")
    sig = pool_map(oracle.sigma, segs)
    for s, o in enumerate(sig):
        assert stat_bits(plan.read_sigma(ws, s)) == stat_bits(o), (name, s)
    bits, dec = gpu_decompress(plan, out, ws)
    assert bits == 0, hex(bits)
    for s, (seg, d) in enumerate(zip(segs, dec)):
        assert np.array_equal(seg, d), (name, s)
    say(f"  {name}: round trip exact")


def test_gradient_64M():
    check_full([W.gradient()], "gradient 67,108,864")


def times2(x):
    """BF16 bits of 2x (exact: every finite value's exponent one up; the
    gradient workload has no value near the top of the range)."""
    f = (x.astype(np.uint32) << 16).view(np.float32) * np.float32(2)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_gradient_64M_window_paths():
    # the other compress paths at full size (1024 chunks, a moment tree in
    # two parts): a failed prediction (the workspace last saw the tensor
    # times 2, whose window is one step up), the caller's fixed window equal
    # to the natural one, and a fixed window one step up
    x = W.gradient()
    ref = oracle.compress(x, C=CHUNK)
    L = ref[6]
    _, plan, _, ws = gpu_compress([times2(x)], CHUNK)
    assert plan.read_sigma(ws, 0)[4] == L + 1
    miss, _, _, _ = gpu_compress([x], CHUNK, plan=plan, ws=ws)
    assert_same_bytes(miss[0], ref, "failed prediction")
    assert plan.read_sigma(ws, 0)[4] == L
    say("  prediction miss: stream identical to the oracle's")
    fixed, _, _, _ = gpu_compress([x], CHUNK, window=L, plan=plan, ws=ws)
    assert_same_bytes(fixed[0], ref, "fixed natural window")
    up, _, _, _ = gpu_compress([x], CHUNK, window=L + 1, plan=plan, ws=ws)
    assert_same_bytes(up[0], oracle.compress(x, C=CHUNK, L=L + 1), "fixed window one step up")
    say("  fixed windows: streams identical to the oracle's")


def test_merged_tail_part_boundaries():
    # one plan, segments at the window parts' edges: 2048 moment blocks and
    # one value (two parts, the second holding one block), 8194 blocks and
    # five values (five parts: the 8-leaf join of the parts with three
    # missing leaves) and exactly 16,384 blocks (eight full parts, the
    # largest segment the merged tail takes); fresh, then after a failed
    # prediction (the workspace last saw the tensors times 2)
    segs = [W.small(2048 * 16384 + 1, seed=21), W.gradient((4 * 2048 + 2) * 16384 + 5, seed=22),
            W.gradient(16384 * 16384, seed=23)]
    refs = pool_map(lambda x: oracle.compress(x, C=CHUNK), segs)
    streams, plan, _, ws = gpu_compress(segs, CHUNK)
    for s, (st, ref) in enumerate(zip(streams, refs)):
        assert_same_bytes(st, ref, f"fresh, segment {s}")
    say("  fresh workspace: streams identical to the oracle's")
    gpu_compress([times2(x) for x in segs], CHUNK, plan=plan, ws=ws)
    streams, _, _, _ = gpu_compress(segs, CHUNK, plan=plan, ws=ws)
    for s, (st, ref) in enumerate(zip(streams, refs)):
        assert_same_bytes(st, ref, f"after a failed prediction, segment {s}")
    sig = pool_map(oracle.sigma, segs)
    for s in range(len(segs)):
        assert stat_bits(plan.read_sigma(ws, s)) == stat_bits(sig[s]), s
    say("  failed prediction: streams and statistics identical to the oracle's")


def test_llama_mlp_layer():
    check_full(W.llama_mlp(), "Llama3-8B MLP matrices")


def test_moe_all_to_all_segments():
    # drawn as the workload states it: torch's CPU generator, seed 0
    bits, sizes = W.moe()
    offs = np.concatenate([[0], np.cumsum(sizes)])
    segs = [bits[offs[i]:offs[i + 1]] for i in range(len(sizes))]
    check_full(segs, "MoE 256 experts")


def test_reduce_scatter_receive_8_shards():
    shards = W.shards()
    n = shards[0].size
    say(f"  reduce: 8 shards of {n:,} values")
    refs = pool_map(lambda s: oracle.compress(s, C=CHUNK), shards)
    for i, sh in enumerate(shards):  # the GPU's own streams are the oracle's
        got, _, _, _ = gpu_compress([sh], CHUNK)
        assert_same_bytes(got[0], refs[i], f"shard {i}")
    bits, out = gpu_reduce(refs, n, CHUNK)
    assert bits == 0, hex(bits)
    want = oracle.decompress_reduce(refs, n, C=CHUNK)
    assert np.array_equal(out, want)
    say("  reduce: bit-exact")
    # the native (uncompressed) reduce of the same shards gives the same bits
    import torch
    import lossless_bf16_exponent_zc_amd as zc
    dev = [torch.from_numpy(s.view(np.int16)).cuda() for s in shards]
    nat = torch.empty(n, dtype=torch.int16, device="cuda")
    zc.reduce_native(dev, nat)
    assert np.array_equal(nat.cpu().numpy().view(np.uint16), want)
    say("  native reduce: bit-exact")
