// zc_finish.hip -- the tail of compress in one launch: the window check and
// the escape placement, overlapped.
//
// ZipCCL scribe notes, "Key idea and contribution": technique 1 (the window
// comes from the standard deviation) and technique 2 (the kernels pipeline
// data movement with compression work).
//
// Workgroups [0, nwin) are window workgroups: a segment's moment tree is
// split into parts of 2048 blocks (at most eight), one workgroup each; every
// part but the last publishes its sums as atomic words, and the segment's
// last part joins them (the tree's top levels) -> variance -> window.  As
// soon as the window is known that workgroup publishes it, with whether the
// encoder's pass used it, in the segment's flag word; then it writes the
// statistics and the header fields known before encoding.
// Workgroups [nwin, nwin + chunks) place one chunk each.  Before they look
// at the flag they load what a held prediction makes final: the chunk's
// group counts, its staged escape bytes, and its escape offset, summed from
// the encoder's per-block counts of the blocks before it.  So the window's
// latency and the placement's loads overlap, and on a hit the workgroup
// places its run at once; it also writes its chunk-table entry, and the
// segment's last chunk writes E, the total and the stream size.  Nothing
// the window workgroups write is read in this kernel except atomic words
// (the part sums, and the flag word, which carries the window), so no
// fence is needed.
// On a miss the workgroup codes its chunk again with the published window,
// publishes the chunk's escape count and sums the counts of the chunks
// before it as they arrive, then places as on a hit.
// Waiting never goes the other way: a segment's last window part waits only
// for its other parts, and a placement workgroup only for its segment's
// last window part and for chunks before its own, all of lower workgroup
// index, which the hardware dispatches first.  Every wait is bounded; a wait that runs out
// leaves the segment's stream size 0 (no stream is shorter than 64 bytes).
// Plans whose segments hold more than 16,384 moment blocks (the direct offset
// sums would grow), with the raw fallback, or with the static/dynamic split
// use the window and placement kernels.
#include "zc_place.h"

namespace zc {

namespace {

// the flag word: the window in bits 8-15, the verdict in bits 0-7
constexpr uint32_t kFlagHit = 1, kFlagMiss = 2;
constexpr uint64_t kAggAggregate = 1ull << 62;  // a chunk's count is in the word
// polls per wait (each a memory round trip plus a short sleep, a microsecond
// or two): a wait gives up after about a tenth of a second, far beyond what
// the window workgroups or the chunks before take
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

// Part q of a segment's moment tree: the pairwise sums over its blocks
// [2048 q, 2048 q + 2048) (an aligned subtree: a part never crosses a
// power-of-two boundary of the tree; blocks past nsb are -0.0, the
// identity).  Thread t takes blocks 2048 q + 8 t .. + 7 (one round of
// loads, from their leaf slots), then the wave butterfly and a tree over the
// 4 waves.  The result is valid in thread 0.
__device__ __forceinline__ void part_moments(const double* ps1, const double* ps2, const uint32_t* pn,
                                             uint32_t nsb, uint32_t q, MomentScratch& sh, double& s1,
                                             double& s2, uint64_t& n) {
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const LeafOrder o = leaf_order(nsb);
    double v1[8], v2[8];
    uint32_t c[8];
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {  // loads only: nothing here waits for them
        const uint32_t b = kFinishPartBlocks * q + 8 * tid + i;
        const uint32_t slot = b < nsb ? leaf_slot(b, o) : 0u;
        v1[i] = ps1[slot];
        v2[i] = ps2[slot];
        c[i] = pn[slot];
    }
    uint32_t cnt = 0;
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
        const bool ok = kFinishPartBlocks * q + 8 * tid + i < nsb;
        v1[i] = ok ? v1[i] : -0.0;
        v2[i] = ok ? v2[i] : -0.0;
        cnt += ok ? c[i] : 0u;
    }
    const double r1 = wave_tree(tree8(v1)), r2 = wave_tree(tree8(v2));
    const uint32_t rn = wave_sum(cnt);  // at most 2048 * 16,384 values
    if (lane == 0) {
        sh.v1[wave] = r1;
        sh.v2[wave] = r2;
        sh.n[wave] = rn;
    }
    __syncthreads();
    if (wave == 0) {  // lanes 0..3 hold the waves' subtrees
        const double t1 = row_tree(lane < 4 ? sh.v1[lane] : -0.0), t2 = row_tree(lane < 4 ? sh.v2[lane] : -0.0);
        if (lane == 0) {
            s1 = t1;
            s2 = t2;
            n = (sh.n[0] + sh.n[1]) + (sh.n[2] + sh.n[3]);
        }
    }
}

__device__ __forceinline__ uint64_t agent_load64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A window workgroup: part q of segment seg's moment tree.  Every part but
// the segment's last publishes its sums (three 64-bit words, each an atomic
// store; the encoder set them to ~0, a NaN pattern no sum of finite values
// has).  The last part waits for the others (lower workgroup indices), joins
// the parts pairwise (the tree's top levels), derives the window and
// publishes it, with whether the encoder's pass used it, in the segment's
// flag word; then it writes the statistics and the header fields known
// before encoding.
template <bool SINGLE>
__device__ __forceinline__ void finish_window(const FinishArgs& f, uint32_t wi, WindowLdsF& lds) {
    const WindowArgs& a = f.win;
    const ItemDesc it = SINGLE ? ItemDesc{0u, wi} : f.parts[wi];
    const uint32_t seg = it.seg, q = it.local;
    const SegDesc sd_mem = SINGLE ? SegDesc{} : a.enc.segs[seg];  // read before any store
    const SegDesc& sd = SINGLE ? a.enc.seg0 : sd_mem;
    const uint32_t forced = a.enc.forced_L;
    const uint32_t parts = sd.nsb > kFinishPartBlocks ? (sd.nsb + kFinishPartBlocks - 1) / kFinishPartBlocks : 1u;
    const bool last = q + 1 == parts;
    if (forced && !last) return;  // no moments with a fixed window
    uint64_t* fp = a.enc.fpart + 4ull * kFinishMaxParts * seg;
    double s1 = 0.0, s2 = 0.0;
    uint64_t n = 0;
    if (!forced && sd.nsb)
        part_moments(a.enc.part.s1 + sd.sb_base, a.enc.part.s2 + sd.sb_base, a.enc.part.n + sd.sb_base,
                     sd.nsb, q, lds.mom, s1, s2, n);
    if (!last) {
        if (threadIdx.x == 0) {
            __hip_atomic_store(fp + 4 * q + 0, (uint64_t)__double_as_longlong(s1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(fp + 4 * q + 1, (uint64_t)__double_as_longlong(s2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(fp + 4 * q + 2, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    uint8_t* st = a.enc.out + sd.out_off;
    const uint32_t pred = a.enc.pred[seg];
    if (threadIdx.x == 0) {
        bool failed = false;
        if (!forced && parts > 1) {  // the other parts' sums (bounded wait)
            double p1[kFinishMaxParts], p2[kFinishMaxParts];
            uint64_t pn = 0;
            bool ok = true;
            // every other part's three words requested at once, then each
            // waited for (one memory round trip when they are all out: in
            // turn, each word was one; 268,435,456 values, eight parts: the
            // tail 45.6 -> 43.7 us)
            uint64_t w[kFinishMaxParts - 1][3];
#pragma unroll
            for (uint32_t j = 0; j + 1 < kFinishMaxParts; ++j)
#pragma unroll
                for (uint32_t k = 0; k < 3; ++k) w[j][k] = j + 1 < parts ? agent_load64(fp + 4 * j + k) : 0ull;
#pragma unroll
            for (uint32_t j = 0; j < kFinishMaxParts; ++j) {
                p1[j] = -0.0;
                p2[j] = -0.0;
                if (j + 1 >= parts) continue;
#pragma unroll
                for (uint32_t k = 0; k < 3; ++k) {
                    for (uint32_t t = 0; w[j][k] == ~0ull && t < kSpinLimit; ++t) {
                        __builtin_amdgcn_s_sleep(1);
                        w[j][k] = agent_load64(fp + 4 * j + k);
                    }
                    ok = ok && w[j][k] != ~0ull;
                }
                p1[j] = __longlong_as_double((long long)w[j][0]);
                p2[j] = __longlong_as_double((long long)w[j][1]);
                pn += w[j][2];
            }
            p1[parts - 1] = s1;
            p2[parts - 1] = s2;
            // the tree's top levels: parts joined pairwise (8 leaves, the
            // missing ones -0.0)
            static_assert(kFinishMaxParts == 8, "the parts' join is an 8-leaf tree");
            s1 = tree8(p1);
            s2 = tree8(p2);
            n += pn;
            failed = !ok;  // a part never came: no window
        }
        // the tree above had no leaves past the data; the segment's tree pads
        // it with +0.0 to a power of two, which changes nothing but the sign
        // of a zero sum: -0.0 becomes +0.0 when any padding leaf exists
        if ((sd.n & (sd.n - 1)) != 0) {
            s1 = s1 == 0.0 ? 0.0 : s1;
            s2 = s2 == 0.0 ? 0.0 : s2;
        }
        const double var = forced ? 0.0 : variance(s1, s2, n);
        const uint32_t L = forced ? forced : window_from_variance(var);
        // the verdict first: the placement workgroups wait for it (0xFF, a
        // verdict that is neither, makes them report the failure)
        const uint32_t word = failed ? 0xFFu : (L << 8) | (L == pred ? kFlagHit : kFlagMiss);
        if (sd.k) __hip_atomic_store(a.enc.flag + seg, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (failed) a.stream_bytes[seg] = 0;
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

// The escape offset of segment-local chunk c after a failed prediction:
// publishes the chunk's count (an atomic word with a flag bit; the encoder
// cleared the words), then sums the counts of chunks 0 .. c-1 as they
// arrive, by the whole workgroup (each thread waits for its own words; a
// merged plan's segment has at most 16,384 chunks, so a direct sum is one
// round of loads after the last of them arrives: no chain of prefixes).
// ok = false if a wait ran out.  s_red: 4 words of LDS.
__device__ __forceinline__ uint32_t chunks_before(uint64_t* agg, uint32_t c, uint32_t count, uint32_t* s_red,
                                                 bool& ok) {
    if (threadIdx.x == 0) __hip_atomic_store(agg + c, kAggAggregate | count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t t = 0, bad = 0;
    for (uint32_t j = threadIdx.x; j < c; j += 256) {
        uint64_t v = __hip_atomic_load(agg + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (uint32_t it = 0; (v >> 62) == 0 && it < kSpinLimit; ++it) {
            __builtin_amdgcn_s_sleep(1);
            v = __hip_atomic_load(agg + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        bad |= (v >> 62) == 0 ? 1u : 0u;
        t += (uint32_t)v;
    }
    t = wave_sum(t);
    const bool wbad = __ballot(bad != 0) != 0;
    if (lane_id() == 0) s_red[wave_id()] = wbad ? 0xFFFFFFFFu : t;
    __syncthreads();
    ok = (s_red[0] != 0xFFFFFFFFu) & (s_red[1] != 0xFFFFFFFFu) & (s_red[2] != 0xFFFFFFFFu) &
         (s_red[3] != 0xFFFFFFFFu);
    t = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    __syncthreads();  // s_red is reused
    return t;
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
    const uint32_t bpc = a.chunk_elems / f.win.enc.block_elems;  // moment blocks per chunk: 1, 2 or 4
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
    recode_chunk(f.win.enc, sd, pc.gc0, pc.ng, L, lds.enc);
    __syncthreads();  // the new counts and staged bytes, for the whole workgroup
    // (every wave sums the chunk's group counts: a uniform value for all)
    const uint32_t cnt = wave_sum(lane < pc.ng ? pc.gcnt[lane] : 0u);
    bool ok;
    const uint32_t pre = chunks_before(f.win.enc.agg + sd.chunk_base, pc.local, cnt, s_word, ok);
    if (wave_id() == 0) {
        if (lane == 0) s_word[0] = ok ? pre : 0xFFFFFFFFu;
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
    if (s_word[0] == 0xFFFFFFFFu) return;
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
        finish_window<SINGLE>(f, blockIdx.x, lds.win);
        return;
    }
    finish_place<SINGLE, GPW>(f, blockIdx.x - f.nwin, lds, s_word);
}

template __global__ void zc_finish<true, 1>(FinishArgs);
template __global__ void zc_finish<true, 2>(FinishArgs);
template __global__ void zc_finish<true, 4>(FinishArgs);
template __global__ void zc_finish<true, 8>(FinishArgs);
template __global__ void zc_finish<false, 1>(FinishArgs);
template __global__ void zc_finish<false, 2>(FinishArgs);
template __global__ void zc_finish<false, 4>(FinishArgs);
template __global__ void zc_finish<false, 8>(FinishArgs);

}  // namespace zc
