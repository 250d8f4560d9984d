"""Benchmark: lossless BF16 exponent coding on one MI355X.

Workload (default): 67,108,864 gradient-like BF16 values (N(0, 1e-3^2), 1%
outliers x100, 0.5% zeros, 0.01% subnormals; seed 0), one segment, 65,536-value
chunks.  One step = compress + decompress of that tensor, inputs resident in
HBM.  Also timed: decompress-reduce of 8 shards of 33,554,432 values each.

Prints one JSON line (see the keys below).  `value` is input GB/s of the
round trip (2N bytes per step / step time); compress and decompress GB/s,
their fraction of the 8 TB/s HBM peak by algorithmic bytes, and the ratio are
extra keys.  Timed calls are cold: a 1 GiB read before each (outside the
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
# counter summary of the decode kernel on this workload (FETCH_SIZE and
# WRITE_SIZE per dispatch, scaled by a plain copy's readings), valid while the
# decoder's sources hash to the value recorded there
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "zc_decode_gradient64M_hbm_traffic.txt")
DECODER_SOURCES = ["zc_decode.hip", "zc_internal.h", "zc_kernels.h"]


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


def decoder_hash():
    import hashlib
    h = hashlib.sha256()
    for f in DECODER_SOURCES:
        with open(os.path.join(ROOT, "lossless_bf16_exponent_zc_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None
    when the decoder has changed since it was taken."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line)
        if kv.get("decoder_sources_sha256", "").strip() != decoder_hash():
            return None
        return int(kv["traffic_bytes_per_launch"].strip())
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(x, chunk):
    """Time the oracle's compress + decompress on a bounded host sample."""
    import oracle
    n = min(x.size, 1 << 24)
    sample = np.ascontiguousarray(x[:n])
    reps, t0 = 0, time.perf_counter()
    while True:
        s = oracle.compress(sample, C=chunk)
        oracle.decompress(s, n, C=chunk)
        reps += 1
        el = time.perf_counter() - t0
        if el > 8.0 or reps >= 5:
            break
    return {"value": round(2 * n * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"compress+decompress round trip of the first {n} values of the "
                      f"workload, {reps} rep(s), {el:.1f} s, single-threaded C"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reduce", action="store_true")
    ap.add_argument("--copy-ref", action="store_true",
                    help="also time a plain 128 MiB device-to-device copy (bandwidth "
                         "reference and counter calibration)")
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

    log("timing")
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
    step = lambda: (comp(), dec())
    tc = timed(comp, args.steps, args.warmup, stream, flush)
    td = timed(dec, args.steps, args.warmup, stream, flush)
    ts = timed(step, args.steps, args.warmup, stream, flush)
    tcw = timed(comp, args.steps, args.warmup, stream)
    tdw = timed(dec, args.steps, args.warmup, stream)

    # algorithmic bytes: compress reads the input twice (sigma, encode) and
    # writes the stream; decompress reads the stream and writes the values
    comp_bytes = 2 * N + 2 * N + stream_bytes
    dec_bytes = stream_bytes + 2 * N
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
        "compress_hbm_frac": round(comp_bytes / t_c / HBM_PEAK, 4),
        "decompress_hbm_frac": round(dec_bytes / t_d / HBM_PEAK, 4),
        "timing": "cold: caches filled by a 1 GiB read before every timed call; "
                  "medians of the timed calls",
        "compress_ms_best": round(min(tc) * 1e3, 4),
        "decompress_ms_best": round(min(td) * 1e3, 4),
        "compress_ms_warm": round(t_cw * 1e3, 4),
        "decompress_ms_warm": round(t_dw * 1e3, 4),
        "ratio": round(2 * N / stream_bytes, 4),
        "escape_frac": round(E / N, 5),
        # the decode kernel is the only launch of zc_decompress, so the event
        # time around the call is that kernel's launch duration
        "roofline": {"bound": "hbm", "kernel": "zc_decode",
                     "achieved": round(dec_bytes / t_d / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(dec_bytes / t_d / HBM_PEAK, 4),
                     # HBM bytes per launch (counters); algorithmic bytes beside it
                     "traffic": measured_traffic(),
                     "algorithmic_bytes": dec_bytes,
                     "launch_us": round(t_d * 1e6, 2)},
    }

    if args.copy_ref:
        src = torch.empty(64 << 20, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        tcp = float(np.median(timed(lambda: dst.copy_(src), args.steps, args.warmup, stream, flush)))
        res["copy_128MiB_ms"] = round(tcp * 1e3, 4)
        res["copy_GBps"] = round(2 * src.numel() * 2 / tcp / 1e9, 1)  # read + write
        del src, dst

    if not args.no_reduce:
        log("decompress-reduce workload")
        del xd, y, flush
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
        rws, r = rplan.empty_workspace(), rplan.empty_input()
        red = lambda: rplan.decompress_reduce(bufs, r, rws, capacity=cap)
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        tr = float(np.median(timed(red, args.steps, args.warmup, stream, flush)))
        assert rplan.read_status(rws) == 0
        res["reduce_ms"] = round(tr * 1e3, 4)
        res["reduce_hbm_frac"] = round((tot + 2 * n) / tr / HBM_PEAK, 4)
        res["reduce_out_GBps"] = round(2 * n / tr / 1e9, 2)

    if not args.no_cpu_baseline:
        log("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(x, chunk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
