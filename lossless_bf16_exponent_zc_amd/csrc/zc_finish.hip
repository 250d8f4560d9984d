// zc_finish.hip -- the tail of compress in one launch: the window check and
// the escape placement, overlapped.
//
// ZipCCL scribe notes, "Key idea and contribution": technique 1 (the window
// comes from the standard deviation) and technique 2 (the kernels pipeline
// data movement with compression work).
//
// Workgroups [0, nwin) are window workgroups, one per segment: the moments'
// top levels -> variance -> window.  As soon as the window is known the
// workgroup publishes it, with whether the encoder's pass used it, in the
// segment's flag word; then it writes the statistics and the header fields
// known before encoding.
// Workgroups [nwin, nwin + chunks) place one chunk each.  Before they look
// at the flag they load what a held prediction makes final: the chunk's
// group counts, its staged escape bytes, and its escape offset, summed from
// the encoder's per-block counts of the blocks before it.  So the window's
// latency and the placement's loads overlap, and on a hit the workgroup
// places its run at once; it also writes its chunk-table entry, and the
// segment's last chunk writes E, the total and the stream size.  Nothing
// the window workgroup writes is read in this kernel (the flag word carries
// the window), so no fence is needed.
// On a miss the workgroup codes its chunk again with the published window,
// publishes the chunk's escape count and takes its offset by a look-back
// over the chunks before it (decoupled look-back: each chunk publishes its
// count, then its inclusive prefix once known), then places as on a hit.
// Waiting never goes the other way: window workgroups wait for nothing, and
// a placement workgroup waits only for its segment's window workgroup and
// for chunks before its own, all of lower workgroup index, which the
// hardware dispatches first.  Every wait is bounded; a wait that runs out
// leaves the segment's stream size 0 (no stream is shorter than 64 bytes).
// Plans whose chunks hold fewer than 16,384 values (the look-back needs
// whole encoder items per chunk), whose segments hold more than 8192 moment
// blocks (the direct offset sums would grow), with the raw fallback, or
// with the static/dynamic split use the window and placement kernels.
#include "zc_place.h"

namespace zc {

namespace {

// the flag word: the window in bits 8-15, the verdict in bits 0-7
constexpr uint32_t kFlagHit = 1, kFlagMiss = 2;
constexpr uint64_t kAggAggregate = 1ull << 62, kAggInclusive = 2ull << 62;
// polls per wait (each a memory round trip plus a short sleep, a microsecond
// or two): a wait gives up after about a tenth of a second, far beyond what
// the window workgroup or a look-back takes
constexpr uint32_t kSpinLimit = 1u << 16;

struct WindowLdsF {
    MomentScratch mom;
};

template <int GPW>
union FinishLds {
    WindowLdsF win;
    PlaceLds<GPW> place;
    EncodeLds enc;
};

__device__ __forceinline__ uint32_t agent_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The window workgroup of segment `seg`.
template <bool SINGLE>
__device__ __forceinline__ void finish_window(const FinishArgs& f, uint32_t seg, WindowLdsF& lds) {
    const WindowArgs& a = f.win;
    const SegDesc sd_mem = SINGLE ? SegDesc{} : a.enc.segs[seg];  // read before any store
    const SegDesc& sd = SINGLE ? a.enc.seg0 : sd_mem;
    uint8_t* st = a.enc.out + sd.out_off;
    const uint32_t forced = a.enc.forced_L;
    const double* ps1 = a.enc.part.s1 + sd.sb_base;
    const double* ps2 = a.enc.part.s2 + sd.sb_base;
    const uint32_t* pn = a.enc.part.n + sd.sb_base;
    const bool moments = !forced && sd.nsb;
    const ReduceShape shape = reduce_shape(sd.nsb);
    const uint32_t pred = a.enc.pred[seg];
    double s1 = 0.0, s2 = 0.0;
    uint64_t n = 0;
    if (moments) {  // (rounds in halves: this kernel's placement shares its registers)
        uint64_t nn = 0;
        for (uint32_t k = 0; k < shape.rounds; ++k) halves_round(ps1, ps2, pn, sd.nsb, shape, k, lds.mom, nn);
        join_rounds(lds.mom, shape.rounds, nn, s1, s2, n);
    }
    if (threadIdx.x == 0) {
        // the tree above had no leaves past the data; the segment's tree pads
        // it with +0.0 to a power of two, which changes nothing but the sign
        // of a zero sum: -0.0 becomes +0.0 when any padding leaf exists
        if ((sd.n & (sd.n - 1)) != 0) {
            s1 = s1 == 0.0 ? 0.0 : s1;
            s2 = s2 == 0.0 ? 0.0 : s2;
        }
        const double var = forced ? 0.0 : variance(s1, s2, n);
        const uint32_t L = forced ? forced : window_from_variance(var);
        // the verdict first: the placement workgroups wait for it
        if (sd.k) __hip_atomic_store(a.enc.flag + seg, (L << 8) | (L == pred ? kFlagHit : kFlagMiss),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        SegStat ss{};
        ss.s1 = s1;
        ss.s2 = s2;
        ss.n = n;
        ss.var = var;
        ss.L = L;
        a.stats[seg] = ss;
        write_static_header(st, sd, a.chunk_elems, L);
        if (sd.k == 0) {  // empty: chunk table entry 0 = E = 0
            *reinterpret_cast<uint32_t*>(st + kHeaderBytes) = 0;
            *reinterpret_cast<uint64_t*>(st + 24) = 0;
            *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off;
            a.stream_bytes[seg] = sd.esc_off;
        }
    }
    for (uint64_t i = sd.gtab_off + 2ull * sd.g + threadIdx.x; i < sd.code_off; i += blockDim.x) st[i] = 0;
}

// The segment's flag word, by thread 0 (bounded wait), broadcast through
// LDS; 0 if the wait ran out.
__device__ __forceinline__ uint32_t wait_verdict(const uint32_t* flag, uint32_t* s_v) {
    if (threadIdx.x == 0) {
        uint32_t v = agent_load(flag);
        for (uint32_t it = 0; v == 0 && it < kSpinLimit; ++it) {
            __builtin_amdgcn_s_sleep(1);
            v = agent_load(flag);
        }
        *s_v = v;
    }
    __syncthreads();
    const uint32_t v = *s_v;
    __syncthreads();  // s_v is reused
    return v;
}

// Decoupled look-back by one wave (all 64 lanes): publishes `count` for
// segment-local chunk c, then sums the counts of the chunks before it back to
// the nearest one whose inclusive prefix is known; publishes c's inclusive
// prefix and returns its exclusive one.  ok = false if a wait ran out.
__device__ __forceinline__ uint32_t lookback(uint64_t* agg, uint32_t c, uint32_t count, bool& ok) {
    const uint32_t lane = lane_id();
    ok = true;
    if (c == 0) {
        if (lane == 0) __hip_atomic_store(agg, kAggInclusive | count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    if (lane == 0) __hip_atomic_store(agg + c, kAggAggregate | count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t prefix = 0;
    for (int64_t j = (int64_t)c - 1;; j -= 64) {
        if (j < 0) {  // past chunk 0 without an inclusive prefix: never with valid words
            ok = false;
            return 0;
        }
        const int64_t idx = j - (int64_t)lane;
        const bool valid = idx >= 0;
        uint64_t v = 0;
        for (uint32_t it = 0;; ++it) {
            if (valid && (v >> 62) == 0)
                v = __hip_atomic_load(agg + (valid ? idx : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (!__ballot(valid && (v >> 62) == 0)) break;
            if (it >= kSpinLimit) {
                ok = false;
                return 0;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const uint32_t val = valid ? (uint32_t)v : 0u;
        const uint64_t inc = __ballot(valid && (v >> 62) == 2);
        if (inc) {  // the nearest chunk with its inclusive prefix: stop there
            const uint32_t m = (uint32_t)__builtin_ctzll(inc);
            prefix += wave_sum(lane <= m ? val : 0u);
            break;
        }
        prefix += wave_sum(val);  // (chunk 0 is always inclusive: the walk ends)
    }
    if (lane == 0)
        __hip_atomic_store(agg + c, kAggInclusive | (uint64_t)(prefix + count), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return prefix;
}

// Escapes in the segment's first nb moment blocks (the encoder's per-block
// counts), by the whole workgroup; s_red: 4 words of LDS.
__device__ __forceinline__ uint32_t blocks_before(const uint32_t* pesc, uint32_t nb, uint32_t* s_red) {
    uint32_t t = 0;
    for (uint32_t b = threadIdx.x; b < nb; b += 16 * 256) {
        uint32_t v[16];
#pragma unroll
        for (uint32_t u = 0; u < 16; ++u) v[u] = b + 256 * u < nb ? pesc[b + 256 * u] : 0u;
#pragma unroll
        for (uint32_t u = 0; u < 16; ++u) t += v[u];
    }
    t = wave_sum(t);
    if (lane_id() == 0) s_red[wave_id()] = t;
    __syncthreads();
    t = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    __syncthreads();  // s_red is reused
    return t;
}

// The placement workgroup of plan chunk ci.
template <bool SINGLE, int GPW>
__device__ __forceinline__ void finish_place(const FinishArgs& f, uint32_t ci, FinishLds<GPW>& lds,
                                             uint32_t* s_word) {
    const PlaceArgs& a = f.place;
    PlaceChunk<GPW> pc;
    place_begin(a, ci, pc);
    place_load<GPW, true>(a, pc);  // speculative: final if the window held
    const SegDesc sd_mem = SINGLE ? SegDesc{} : f.win.enc.segs[pc.seg];
    const SegDesc& sd = SINGLE ? f.win.enc.seg0 : sd_mem;
    const uint32_t bpc = a.chunk_elems / kSigmaBlock;  // moment blocks (= encoder items) per chunk
    const uint32_t pre_hit = blocks_before(f.win.enc.part.esc + sd.sb_base, pc.local * bpc, s_word);
    const uint32_t lane = lane_id();
    uint32_t* tab = reinterpret_cast<uint32_t*>(pc.st + kHeaderBytes);
    // the run is gathered in LDS at the offset a held prediction gives; the
    // verdict decides whether it goes out
    uint32_t v = 0;
    const bool hit = place_finish<GPW>(a, pc, pre_hit, false, lds.place, [&] {
        v = wait_verdict(f.win.enc.flag + pc.seg, s_word);
        return (v & 0xFF) == kFlagHit;
    });
    if (hit) {
        if (wave_id() == 0) {
            const uint32_t cnt = wave_sum(lane < pc.ng ? pc.c_raw : 0u);
            if (lane == 0) {
                tab[pc.local] = pre_hit;
                if (pc.local + 1 == sd.k) {  // the segment's last chunk: E, total, size
                    const uint64_t E = (uint64_t)pre_hit + cnt;
                    tab[sd.k] = (uint32_t)E;
                    *reinterpret_cast<uint64_t*>(pc.st + 24) = E;
                    *reinterpret_cast<uint64_t*>(pc.st + 32) = sd.esc_off + E;
                    f.win.stream_bytes[pc.seg] = sd.esc_off + E;
                }
            }
        }
        return;
    }
    if ((v & 0xFF) != kFlagMiss) {  // the wait ran out
        if (threadIdx.x == 0) f.win.stream_bytes[pc.seg] = 0;
        return;
    }
    // the prediction failed: code the chunk's items again with the window
    // in the flag word
    const uint32_t L = (v >> 8) & 0xFF;
    for (uint32_t i = 0; i < bpc; ++i) {
        const uint32_t item = pc.local * bpc + i;
        if (item < sd.nwg) encode_wg<false>(f.win.enc, sd.wg_base + item, L, lds.enc);
    }
    __syncthreads();  // the new counts and staged bytes, for the whole workgroup
    if (wave_id() == 0) {
        const uint32_t cnt = wave_sum(lane < pc.ng ? pc.gcnt[lane] : 0u);
        bool ok;
        const uint32_t pre = lookback(f.win.enc.agg + sd.chunk_base, pc.local, cnt, ok);
        if (lane == 0) *s_word = ok ? pre : 0xFFFFFFFFu;
        if (lane == 0 && ok) {
            tab[pc.local] = pre;
            if (pc.local + 1 == sd.k) {  // the segment's last chunk: E, total, size
                const uint64_t E = (uint64_t)pre + cnt;
                tab[sd.k] = (uint32_t)E;
                *reinterpret_cast<uint64_t*>(pc.st + 24) = E;
                *reinterpret_cast<uint64_t*>(pc.st + 32) = sd.esc_off + E;
                f.win.stream_bytes[pc.seg] = sd.esc_off + E;
            }
        }
        if (lane == 0 && !ok) f.win.stream_bytes[pc.seg] = 0;
    }
    __syncthreads();
    const uint32_t pre = *s_word;
    if (pre == 0xFFFFFFFFu) return;
    PlaceChunk<GPW> pc2;  // (a fresh copy: the first loads are dead here)
    place_begin(a, ci, pc2);
    place_load<GPW, true>(a, pc2);  // the new counts and staged bytes
    place_finish<GPW>(a, pc2, pre, false, lds.place, [] { return true; });
}

}  // namespace

template <bool SINGLE, int GPW>
__global__ __launch_bounds__(256) void zc_finish(FinishArgs f) {
    __shared__ FinishLds<GPW> lds;
    __shared__ uint32_t s_word[4];
    if (blockIdx.x < f.nwin) {
        finish_window<SINGLE>(f, SINGLE ? 0u : blockIdx.x, lds.win);
        return;
    }
    finish_place<SINGLE, GPW>(f, blockIdx.x - f.nwin, lds, s_word);
}

template __global__ void zc_finish<true, 2>(FinishArgs);
template __global__ void zc_finish<true, 4>(FinishArgs);
template __global__ void zc_finish<true, 8>(FinishArgs);
template __global__ void zc_finish<false, 2>(FinishArgs);
template __global__ void zc_finish<false, 4>(FinishArgs);
template __global__ void zc_finish<false, 8>(FinishArgs);

}  // namespace zc
