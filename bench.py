"""Benchmark: lossless BF16 exponent coding on one MI355X.

Workload (default): 67,108,864 gradient-like BF16 values (N(0, 1e-3^2), 1%
outliers x100, 0.5% zeros, 0.01% subnormals; seed 0), one segment, 65,536-value
chunks.  One step = compress + decompress of that tensor, inputs resident in
HBM.  Also timed: decompress-reduce of 8 shards of 33,554,432 values each.

Prints one JSON line (see the keys below).  `value` is input GB/s of the
round trip (2N bytes per step / step time); compress and decompress GB/s,
their fraction of the 8 TB/s HBM peak by algorithmic bytes, and the ratio are
extra keys.  `roofline` is the encoder pass (the step's dominant kernel,
timed by HIP events around it), `roofline_decode` the decode kernel.  Timed calls are cold: a 1 GiB read before each (outside the
timed region) evicts the caches, so inputs come from HBM; warm times (no
eviction) are reported beside them.  The oracle (plain C) is timed on a
bounded sample on the host as `cpu_baseline`.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # bytes/s, MI355X
# counter summary of the encoder pass and the decoder on this workload
# (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by a plain copy's readings);
# a kernel's figure is used while its sources hash to the value recorded there
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "zc_codec_gradient64M_hbm_traffic.txt")
KERNEL_SOURCES = {
    "zc_encode": ["zc_encode.hip", "zc_place.h", "zc_encoder.h", "zc_moments.h", "zc_internal.h",
                  "zc_kernels.h", "zc_format.h"],
    "zc_finish": ["zc_finish.hip", "zc_place.h", "zc_window.h", "zc_encoder.h", "zc_moments.h",
                  "zc_internal.h", "zc_kernels.h", "zc_format.h"],
    "zc_decode": ["zc_decode.hip", "zc_internal.h", "zc_kernels.h", "zc_format.h"],
    "zc_decode_reduce_wide": ["zc_decode.hip", "zc_internal.h", "zc_kernels.h", "zc_format.h"],
}
# VALU instructions per launch from the committed SQ counter summary (lines
# "valu <kernel> <wave64 instructions> <sources sha256>"), used while the
# kernel's sources hash to the recorded value
ISSUE_FILE = os.path.join(ROOT, "profiles", "zc_codec_instruction_issue.txt")
# VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (a wave64 VALU
# instruction holds a SIMD for 4 cycles), in 32-bit lane operations per
# second; the fp32 vector peak of 157.3 TFLOP/s is this x 2 (FMA) x 2 (packed)
VALU_PEAK = 256 * 4 * 16 * 2.4e9


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed(fn, steps, warmup, stream, flush=None):
    """Event-timed calls on `stream`; with `flush`, a read of a 1 GiB buffer
    before each call (outside the events) fills the 256 MB Infinity Cache and
    the L2s with clean lines of that buffer, so the call reads its inputs
    from HBM (cold)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        if flush is not None:
            flush.sum()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in evs]  # seconds


def code_text(src):
    """C++ source with its comments removed and every run of white space made
    one space: what the compiler sees, so that editing a comment does not
    change a kernel's hash.  (No string literal in the kernel sources holds
    // or /*.)"""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def sources_hash(kernel, root=None):
    """sha256 prefix of a kernel's sources, comments and spacing aside."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(root or ROOT, "lossless_bf16_exponent_zc_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (lines "traffic <kernel> <bytes> <sources sha256>"), or None when the
    kernel's sources have changed since it was taken."""
    try:
        for line in open(TRAFFIC_FILE):
            f = line.split()
            if len(f) == 4 and f[0] == "traffic" and f[1] == kernel:
                return int(f[2]) if f[3] == sources_hash(kernel) else None
    except (OSError, ValueError):
        pass
    return None


def measured_valu(kernel):
    """Wave64 VALU instructions per launch of `kernel` from the committed SQ
    counter summary, or None when the kernel's sources have changed since."""
    try:
        for line in open(ISSUE_FILE):
            f = line.split()
            if len(f) == 4 and f[0] == "valu" and f[1] == kernel:
                return int(f[2]) if f[3] == sources_hash(kernel) else None
    except (OSError, ValueError):
        pass
    return None


def issue_roofline(kernel, launch_s):
    """The kernel's VALU issue against the chip's peak, or None."""
    n = measured_valu(kernel)
    if n is None or launch_s <= 0:
        return None
    ops = n * 64 / launch_s  # lane operations per second
    return {"bound": "alu", "kernel": kernel, "achieved": round(ops / 1e12, 2),
            "peak": round(VALU_PEAK / 1e12, 2), "unit": "T VALU lane-op/s",
            "frac": round(ops / VALU_PEAK, 4), "valu_instructions": n,
            "launch_us": round(launch_s * 1e6, 2)}


def host_threads():
    """Threads for the oracle's all-core leg: the CPUs this process may run
    on, at most 16 (a one-GPU machine's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(x, chunk):
    """Time the oracle's compress + decompress on bounded host samples.

    Single thread: whole round trips of the workload's first 16M values until
    about 10 s have passed.  All cores: the workload's first T x 4M values as
    T segments (T threads, each segment its own stream, as a multi-segment
    plan codes them), round trips repeated for about 10 s; every thread's
    bytes are checked identical to a single-threaded run of the same segment
    first.  The oracle's C calls release the interpreter lock."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    n = min(x.size, 1 << 24)
    sample = np.ascontiguousarray(x[:n])
    reps, t0 = 0, time.perf_counter()
    while True:
        s = oracle.compress(sample, C=chunk)
        oracle.decompress(s, n, C=chunk)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 30:  # about 10 s of the oracle's work
            break
    single = 2 * n * reps / el / 1e9

    T = host_threads()
    seg = min(1 << 22, x.size // T)
    segs = [np.ascontiguousarray(x[i * seg:(i + 1) * seg]) for i in range(T)]
    ref = [oracle.compress(v, C=chunk) for v in segs]  # single-threaded, once

    def trip(i):
        st = oracle.compress(segs[i], C=chunk)
        oracle.decompress(st, seg, C=chunk)
        return st

    with ThreadPoolExecutor(max_workers=T) as ex:
        first = list(ex.map(trip, range(T)))
        assert first == ref, "threaded oracle streams differ from the single-threaded ones"
        preps, t0 = 0, time.perf_counter()
        while True:
            list(ex.map(trip, range(T)))
            preps += 1
            pel = time.perf_counter() - t0
            if pel > 10.0 or preps >= 50:
                break
    allcore = 2 * seg * T * preps / pel / 1e9
    return {"value": round(allcore, 4), "unit": "GB/s", "cores": T, "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "single_thread_value": round(single, 4),
            "sample": f"all cores: {T} threads, each a compress+decompress round trip of its "
                      f"own {seg}-value segment of the workload (one stream per segment, "
                      f"bytes identical to a single-threaded run), {preps} round(s) in "
                      f"{pel:.1f} s; single thread: the first {n} values as one stream, "
                      f"{reps} rep(s) in {el:.1f} s; plain C oracle built -O2"}


def time_config(name, segs, chunk, args, stream):
    """Cold compress and decompress of a list of segments (one plan)."""
    import lossless_bf16_exponent_zc_amd as zc
    plan = zc.Plan([x.size for x in segs], chunk)
    xd = plan.empty_input()
    for s, x in enumerate(segs):
        off = plan.input_offset(s)
        xd[off:off + x.size] = torch.from_numpy(x.view(np.int16)).cuda()
    out, sizes, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    y = plan.empty_input()
    comp = lambda: plan.compress(xd, out, sizes, ws)
    dec = lambda: plan.decompress(out, y, ws)
    comp()
    dec()
    torch.cuda.synchronize()
    assert plan.read_status(ws) == 0
    n = sum(x.size for x in segs)
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    tc = float(np.median(timed(comp, args.steps, args.warmup, stream, flush)))
    td = float(np.median(timed(dec, args.steps, args.warmup, stream, flush)))
    sb = int(sizes.sum().item())
    r = {"workload": name, "elements": n, "segments": len(segs), "chunk_elems": chunk,
         "compress_ms": round(tc * 1e3, 4), "decompress_ms": round(td * 1e3, 4),
         "compress_GBps": round(2 * n / tc / 1e9, 2), "decompress_GBps": round(2 * n / td / 1e9, 2),
         "compress_hbm_frac": round((2 * n + sb) / tc / HBM_PEAK, 4),
         "compress_hbm_frac_method_bytes": round((4 * n + sb) / tc / HBM_PEAK, 4),
         "decompress_hbm_frac": round((2 * n + sb) / td / HBM_PEAK, 4),
         "ratio": round(2 * n / sb, 4)}
    del plan, xd, out, sizes, ws, y, flush
    torch.cuda.empty_cache()
    return r


def other_configs(args, stream):
    from lossless_bf16_exponent_zc_amd import workloads as W
    log("Llama3-8B MLP matrices")
    res = [time_config("Llama3-8B MLP layer: 3 BF16 matrices (4096x14336, 14336x4096, "
                       "4096x14336), one segment each", W.llama_mlp(), 65536, args, stream)]
    log("MoE 256 experts")
    bits, counts = W.moe()
    offs = np.concatenate([[0], np.cumsum(counts)])
    segs = [bits[offs[i]:offs[i + 1]] for i in range(len(counts))]
    res.append(time_config("MoE all-to-all: 256 expert segments, 65,536 tokens x 7168", segs,
                           65536, args, stream))
    return res


def raw_fallback(zc, N, chunk, args, stream, flush, res):
    """Raw fallback (a plan flag): a tensor of zeros, which every window
    escapes, is stored as its header plus its words; the speculative coding
    pass still runs before the window kernel picks raw."""
    log("raw fallback")
    zplan = zc.Plan([N], chunk, raw_fallback=True)
    zx = zplan.empty_input().zero_()
    zout, zsz, zws, zy = zplan.empty_output(), zplan.empty_sizes(), zplan.empty_workspace(), zplan.empty_input()
    zcomp = lambda: zplan.compress(zx, zout, zsz, zws)
    zdec = lambda: zplan.decompress(zout, zy, zws)
    zcomp(); zdec(); torch.cuda.synchronize()
    assert zplan.read_status(zws) == 0 and torch.equal(zy[:N], zx[:N])
    assert int(zsz.cpu()[0]) == 64 + 2 * N
    res["raw_fallback"] = {
        "input": f"{N:,} zeros, plan with the raw fallback",
        "stream_bytes": 64 + 2 * N,
        "compress_ms": round(float(np.median(timed(zcomp, args.steps, args.warmup, stream, flush))) * 1e3, 4),
        "decompress_ms": round(float(np.median(timed(zdec, args.steps, args.warmup, stream, flush))) * 1e3, 4)}


def cold_calls(zc, W, plan, comp, dec, chunk, k):
    """K cold calls of each timed operation, nothing else: a kernel trace of
    this run gives the kernels' own cold durations, without the HIP events'
    overhead (an empty event pair reads about 4.4 us on an MI355X)."""
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    for fn in (comp, dec):
        for _ in range(k):
            flush.sum()
            fn()
            torch.cuda.synchronize()
    shards = W.shards()
    n = shards[0].size
    cplan, rplan = zc.Plan([n], chunk), zc.Plan([n], chunk)
    cap = cplan.out_bytes
    bufs = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in shards]
    csz, cws = cplan.empty_sizes(), cplan.empty_workspace()
    for s, b in zip(shards, bufs):
        xi = cplan.empty_input()
        xi[:n] = torch.from_numpy(s.view(np.int16)).cuda()
        cplan.compress(xi, b, csz, cws)
    rws, r = rplan.empty_workspace(decode_only=True), rplan.empty_input()
    for _ in range(k):
        flush.sum()
        rplan.decompress_reduce(bufs, r, rws, capacity=cap)
        torch.cuda.synchronize()
    assert rplan.read_status(rws) == 0
    log(f"{k} cold calls each of compress, decompress and the 8-shard reduce")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reduce", action="store_true")
    ap.add_argument("--no-raw", action="store_true", help="skip the raw-fallback measurement")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time compress / decompress of the Llama3-8B MLP matrices "
                         "(3 segments) and the 256-expert MoE batch (extra keys)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also time a plain 128 MiB device-to-device copy (bandwidth "
                         "reference and counter calibration)")
    ap.add_argument("--cold-calls", type=int, default=0, metavar="K",
                    help="only issue K cold compress, K cold decompress and K cold 8-shard "
                         "reduce calls (caches filled before each) and print no JSON line: "
                         "for a kernel trace of the kernels' own cold durations")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the codec is per shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import lossless_bf16_exponent_zc_amd as zc
    from lossless_bf16_exponent_zc_amd import workloads as W

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    chunk = 65536
    log("generating workload")
    x = W.gradient()
    N = x.size
    plan = zc.Plan([N], chunk)
    xd = plan.empty_input()
    xd[:N] = torch.from_numpy(x.view(np.int16)).cuda()
    out, sizes, ws = plan.empty_output(), plan.empty_sizes(), plan.empty_workspace()
    y = plan.empty_input()

    comp = lambda: plan.compress(xd, out, sizes, ws)
    dec = lambda: plan.decompress(out, y, ws)
    comp()
    dec()
    torch.cuda.synchronize()
    assert plan.read_status(ws) == 0
    assert torch.equal(y[:N], xd[:N]), "round trip not exact"
    stream_bytes = int(sizes.cpu()[0])
    E = int(np.frombuffer(out[24:32].cpu().numpy().tobytes(), "<u8")[0])

    if args.cold_calls:
        cold_calls(zc, W, plan, comp, dec, chunk, args.cold_calls)
        return

    log("timing")
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
    step = lambda: (comp(), dec())
    tc = timed(comp, args.steps, args.warmup, stream, flush)
    td = timed(dec, args.steps, args.warmup, stream, flush)
    ts = timed(step, args.steps, args.warmup, stream, flush)
    tcw = timed(comp, args.steps, args.warmup, stream)
    tdw = timed(dec, args.steps, args.warmup, stream)

    # the bytes this library must move: the input once (the moments come
    # from the coding pass), the stream out; decompress reads the stream and
    # writes the values.  The method-bytes count adds a second read of the
    # input (a separate sigma pass before coding), as the method counts it.
    comp_bytes = 2 * N + stream_bytes
    comp_bytes_method = 2 * N + 2 * N + stream_bytes
    dec_bytes = stream_bytes + 2 * N

    # the window prediction failing on every timed call: two resident tensors
    # whose windows differ compressed in turn on one workspace, so each call
    # codes with the other tensor's window first and the segment is coded
    # again in the same call.  The workload and the workload times 2 (exact
    # in BF16: every exponent one higher, sigma one binade up, the window
    # one step up) are the miss of a sigma that drifts across a binade
    # boundary; times 16 (four binades) is a far miss, where most values
    # escape in the first pass
    log("prediction miss")
    out_m = plan.empty_output()

    def miss_times(scale):
        xs = (xd.view(torch.bfloat16) * scale).view(torch.int16)
        pair = [(xd, out), (xs, out_m)]
        turn = [0]

        def comp_alt():
            a, o = pair[turn[0] % 2]
            turn[0] += 1
            plan.compress(a, o, sizes, ws)

        t = timed(comp_alt, args.steps, args.warmup, stream, flush)
        del xs
        return t

    tmiss = miss_times(2)
    tmiss_far = miss_times(16)
    comp()  # the workload's own window back in the workspace
    torch.cuda.synchronize()
    assert int(sizes.cpu()[0]) == stream_bytes

    # the caller's fixed window (the tensor's own, so the stream is the same)
    L = int(out[6].item())
    tfixed = timed(lambda: plan.compress(xd, out, sizes, ws, window=L), args.steps, args.warmup,
                   stream, flush)
    torch.cuda.synchronize()
    assert int(sizes.cpu()[0]) == stream_bytes

    # steady state: calls back to back over 4 buffer sets (1.7 GB, more than
    # the caches hold), so every call reads cold inputs and earlier calls'
    # dirty outputs are written back during later timed calls
    log("steady state")
    sets = [(xd.clone(), plan.empty_output(), plan.empty_input()) for _ in range(4)]
    for xi, oi, yi in sets:
        plan.compress(xi, oi, sizes, ws)
    rot = [0]

    def rot_call(kind):
        xi, oi, yi = sets[rot[0] % 4]
        rot[0] += 1
        if kind == "c":
            plan.compress(xi, oi, sizes, ws)
        else:
            plan.decompress(oi, yi, ws)

    tcs = timed(lambda: rot_call("c"), 4 * args.steps, 4 * args.warmup, stream)
    tds = timed(lambda: rot_call("d"), 4 * args.steps, 4 * args.warmup, stream)
    torch.cuda.synchronize()
    assert all(torch.equal(yi[:N], xd[:N]) for _, _, yi in sets)
    del sets, out_m

    # the encoder pass, timed on its own: HIP events on this stream around
    # each kernel of a compress call (cold, like the calls above)
    log("kernel times")
    ku = []
    for i in range(args.warmup + args.steps):
        flush.sum()
        us = plan.compress_timed(xd, out, sizes, ws)
        if i >= args.warmup:
            ku.append(us)
    ku = np.median(np.array(ku), axis=0)

    # the static/dynamic split: when the fixed-size regions (headers, chunk
    # tables, codes, sign+mantissa bytes) and the sizes are final, measured
    # from the call's start (cold calls, events on this stream)
    log("split event")
    sp = []
    for i in range(args.warmup + args.steps):
        flush.sum()
        e0, ef, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        ef.record(stream)
        e0.record(stream)
        plan.compress_split(xd, out, sizes, ws, ef)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            sp.append((e0.elapsed_time(ef) * 1e3, e0.elapsed_time(e1) * 1e3))
    sp = np.median(np.array(sp), axis=0)
    G = (N + 2047) // 2048
    # the encoder pass moves the input in and the codes, sign+mantissa bytes
    # and escape exponents out (the escape copy of the placement kernel is
    # overhead)
    enc_bytes = 2 * N + (768 + 2048) * G + E
    t_c, t_d, t_s, t_cw, t_dw = (float(np.median(v)) for v in (tc, td, ts, tcw, tdw))
    res = {
        "metric": "compress / decompress GB/s (BF16 input) + % of HBM peak; compression ratio",
        "value": round(2 * N / t_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": "gradient-like BF16, 67,108,864 values, 65,536-value chunks, "
                               "step = compress + decompress",
                   "elements": N, "chunk_elems": chunk},
        "compress_GBps": round(2 * N / t_c / 1e9, 2),
        "decompress_GBps": round(2 * N / t_d / 1e9, 2),
        "compress_ms": round(t_c * 1e3, 4),
        "decompress_ms": round(t_d * 1e3, 4),
        # bytes this library moves (input once + stream) / cold time / 8 TB/s
        "compress_hbm_frac": round(comp_bytes / t_c / HBM_PEAK, 4),
        # the method's count: a separate sigma pass reads the input a second time
        "compress_hbm_frac_method_bytes": round(comp_bytes_method / t_c / HBM_PEAK, 4),
        "decompress_hbm_frac": round(dec_bytes / t_d / HBM_PEAK, 4),
        "timing": "cold: caches filled by a 1 GiB read before every timed call; "
                  "medians of the timed calls",
        # every timed call a failed window prediction: windows one step apart
        # (sigma one binade away), and four apart (_far)
        "compress_ms_miss": round(float(np.median(tmiss)) * 1e3, 4),
        "compress_ms_miss_far": round(float(np.median(tmiss_far)) * 1e3, 4),
        # zc_compress_window with the tensor's own window (no moments)
        "compress_window_ms": round(float(np.median(tfixed)) * 1e3, 4),
        # back-to-back calls over 4 rotating buffer sets (no flush)
        "compress_ms_steady": round(float(np.median(tcs)) * 1e3, 4),
        "decompress_ms_steady": round(float(np.median(tds)) * 1e3, 4),
        "compress_hbm_frac_steady": round(comp_bytes / float(np.median(tcs)) / HBM_PEAK, 4),
        "decompress_hbm_frac_steady": round(dec_bytes / float(np.median(tds)) / HBM_PEAK, 4),
        "compress_ms_best": round(min(tc) * 1e3, 4),
        "decompress_ms_best": round(min(td) * 1e3, 4),
        "compress_ms_warm": round(t_cw * 1e3, 4),
        "decompress_ms_warm": round(t_dw * 1e3, 4),
        "ratio": round(2 * N / stream_bytes, 4),
        # the compressed/raw switch: links slower than this favour sending
        # the compressed stream (cold compress + decompress of this tensor)
        "break_even_link_GBps": round(zc.prefer_compressed(2 * N, stream_bytes, t_c * 1e6,
                                                           t_d * 1e6, 1.0)[1], 1),
        "escape_frac": round(E / N, 5),
        # the encoder pass, then the rest of the call (the window check and
        # the escape placement: one merged kernel on this plan)
        "compress_kernels_us": {"encode": round(float(ku[0]), 2),
                                "tail": round(float(ku[1] + ku[2]), 2)},
        # zc_compress_split: fixed-size regions and sizes final / whole call done
        "split_fixed_ready_us": round(float(sp[0]), 2),
        "split_call_us": round(float(sp[1]), 2),
        # the dominant kernel of the step: the encoder pass (moments, codes,
        # staged escapes), its time from HIP events around it (cold)
        "roofline": {"bound": "hbm", "kernel": "zc_encode",
                     "achieved": round(enc_bytes / (ku[0] * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(enc_bytes / (ku[0] * 1e-6) / HBM_PEAK, 4),
                     # HBM bytes per launch (counters); algorithmic bytes beside it
                     "traffic": measured_traffic("zc_encode"),
                     "algorithmic_bytes": enc_bytes,
                     "launch_us": round(float(ku[0]), 2)},
        # the decode kernel is the only launch of zc_decompress, so the event
        # time around the call is that kernel's launch duration
        "roofline_decode": {"bound": "hbm", "kernel": "zc_decode",
                            "achieved": round(dec_bytes / t_d / 1e9, 1),
                            "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": round(dec_bytes / t_d / HBM_PEAK, 4),
                            "traffic": measured_traffic("zc_decode"),
                            "algorithmic_bytes": dec_bytes,
                            "launch_us": round(t_d * 1e6, 2)},
    }

    # the same launches against the VALU issue peak (the encoder pass and the
    # fused reduce are close to both bounds); instruction counts from the
    # committed SQ counter summary
    res["roofline_issue"] = issue_roofline("zc_encode", float(ku[0]) * 1e-6)
    res["roofline_issue_decode"] = issue_roofline("zc_decode", t_d)
    # the whole compress call's HBM bytes from the counters (encoder pass +
    # the merged tail kernel) against the bytes it must move (input once +
    # stream): the rest is the escape staging round trip and over-reads
    te, tt = measured_traffic("zc_encode"), measured_traffic("zc_finish")
    res["compress_traffic"] = None if te is None or tt is None else {
        "encode": te, "tail": tt, "total": te + tt, "one_read_bytes": comp_bytes,
        "ratio": round((te + tt) / comp_bytes, 4)}

    if args.copy_ref:
        src = torch.empty(64 << 20, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        tcp = float(np.median(timed(lambda: dst.copy_(src), args.steps, args.warmup, stream, flush)))
        res["copy_128MiB_ms"] = round(tcp * 1e3, 4)
        res["copy_GBps"] = round(2 * src.numel() * 2 / tcp / 1e9, 1)  # read + write
        del src, dst

    if not args.no_raw:
        raw_fallback(zc, N, chunk, args, stream, flush, res)

    if not args.no_reduce:
        log("decompress-reduce workload")
        del y, flush
        shards = W.shards()
        n = shards[0].size
        rplan = zc.Plan([n], chunk)
        cplan = zc.Plan([n], chunk)
        cap = cplan.out_bytes
        bufs = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in shards]
        csz, cws = cplan.empty_sizes(), cplan.empty_workspace()
        tot = 0
        for s, b in zip(shards, bufs):
            xi = cplan.empty_input()
            xi[:n] = torch.from_numpy(s.view(np.int16)).cuda()
            cplan.compress(xi, b, csz, cws)
            tot += int(csz.cpu()[0])
        rws, r = rplan.empty_workspace(decode_only=True), rplan.empty_input()
        red = lambda: rplan.decompress_reduce(bufs, r, rws, capacity=cap)
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        tr = float(np.median(timed(red, args.steps, args.warmup, stream, flush)))
        assert rplan.read_status(rws) == 0
        res["reduce_ms"] = round(tr * 1e3, 4)
        res["reduce_hbm_frac"] = round((tot + 2 * n) / tr / HBM_PEAK, 4)
        res["reduce_out_GBps"] = round(2 * n / tr / 1e9, 2)
        # one launch per call: the event time is the kernel's launch time
        res["roofline_reduce"] = {"bound": "hbm", "kernel": "zc_decode_reduce_wide",
                                  "achieved": round((tot + 2 * n) / tr / 1e9, 1),
                                  "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                                  "frac": round((tot + 2 * n) / tr / HBM_PEAK, 4),
                                  "traffic": measured_traffic("zc_decode_reduce_wide"),
                                  "algorithmic_bytes": tot + 2 * n,
                                  "launch_us": round(tr * 1e6, 2)}
        res["roofline_issue_reduce"] = issue_roofline("zc_decode_reduce_wide", tr)

        # the native path: the same 8 shards uncompressed, summed by a plain
        # kernel in the same order with the same rounding (the same bits)
        log("native reduce")
        raw = [torch.from_numpy(s_.view(np.int16)).cuda() for s_ in shards]
        rn = torch.empty(n, dtype=torch.int16, device="cuda")
        native = lambda: zc.reduce_native(raw, rn)
        tn = float(np.median(timed(native, args.steps, args.warmup, stream, flush)))
        assert torch.equal(rn, r[:n])
        res["reduce_native_ms"] = round(tn * 1e3, 4)
        res["reduce_native_hbm_frac"] = round((8 * 2 * n + 2 * n) / tn / HBM_PEAK, 4)

        # the reduce-scatter switch for this shape (8 GPUs, one shard per
        # peer per link): the sender compresses its 7 outgoing shards (one
        # 7-segment plan), each link carries one shard, and the receiver runs
        # the fused reduce instead of the native one.  Compressed pays when
        #   t_compress7 + compressed/B + (t_fused - t_native) < raw/B
        log("reduce-scatter switch")
        splan = zc.Plan([n] * 7, chunk)
        sx = splan.empty_input()
        for i in range(7):
            o = splan.input_offset(i)
            sx[o:o + n] = raw[i + 1]
        sout, ssz, sws = splan.empty_output(), splan.empty_sizes(), splan.empty_workspace()
        c7 = lambda: splan.compress(sx, sout, ssz, sws)
        t7 = float(np.median(timed(c7, args.steps, args.warmup, stream, flush)))
        per_link = int(ssz.cpu().numpy().mean())
        extra = max(0.0, (tr - tn) * 1e6)
        xgmi = 153.0  # GB/s, one xGMI link of an MI355X
        pref, be = zc.prefer_compressed(2 * n, per_link, t7 * 1e6, extra, xgmi)
        res["reduce_scatter_switch"] = {
            "compress_7_shards_ms": round(t7 * 1e3, 4),
            "fused_minus_native_us": round((tr - tn) * 1e6, 2),
            "raw_bytes_per_link": 2 * n, "compressed_bytes_per_link": per_link,
            "break_even_link_GBps": round(be, 1),
            "xgmi_link_GBps": xgmi, "prefer_compressed_on_xgmi": pref}
        del splan, sx, sout, ssz, sws, raw, rn

    if args.all_configs:
        res["other_configs"] = other_configs(args, stream)

    if not args.no_cpu_baseline:
        log("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(x, chunk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
