// zc_place.h -- escape placement of one chunk: the group table entries and
// the chunk's escape run, gathered from the groups' staging slots to its
// final place in the stream (or, for a raw stream, the chunk's values).
// Used by the placement kernel and by the merged finish kernel, which runs
// the load phase before it knows the chunk's escape offset.
//
// ZipCCL scribe notes, "Key idea and contribution", technique 2: an aligned,
// communication-aware layout (the escapes of all chunks form one compact
// region after the fixed-size ones).
#pragma once

#include "zc_encoder.h"

namespace zc {

// One wave stores a run of n bytes (a group's escape exponents) from `src`
// (the group's 2048-byte staging slot) to `dst` in global memory (a chunk
// whose run does not fit the LDS gather buffer goes out group by group).  The
// caller has loaded, for output dwords k = lane + 64 r (r < R), lo[r] =
// source dword k and hi[r] = source dword k+1: output dword k starts at
// source byte head + 4k, where head (0..3) brings dst to a 4-byte boundary,
// so those two dwords serve whatever dst is.  The head bytes (from lane 0's
// first source dword) and the tail bytes (from the dword of the lane owning
// the partial last output dword) go out as one byte store each, by lanes
// 0..2; dwords past 64 R (runs over 256 R bytes) are loaded here.
template <int R>
__device__ __forceinline__ void store_run(uint8_t* dst, const uint32_t* src, uint32_t n,
                                          const uint32_t (&lo)[R], const uint32_t (&hi)[R]) {
    const uint32_t lane = lane_id();
    const uint32_t head = min(n, (4u - (uint32_t)(reinterpret_cast<uintptr_t>(dst) & 3u)) & 3u);
    const uint32_t nd = (n - head) >> 2, tail = (n - head) & 3u;
    uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + head);
    const uint32_t first = readlane(lo[0], 0);
    if (lane < head) dst[lane] = (uint8_t)(first >> (8 * lane));
    uint32_t last = 0;  // the partial last output dword (wave-uniform)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t k = lane + 64 * r;
        const uint32_t v = (uint32_t)((((uint64_t)hi[r] << 32) | lo[r]) >> (8 * head));
        if (k < nd) d32[k] = v;
        if ((nd >> 6) == (uint32_t)r) last = readlane(v, (int)(nd & 63));
    }
    // a run past the loaded dwords (a wave-uniform test: with a per-lane
    // loop condition, lanes past the run's end still entered the loop and
    // paid its set-up for every group, about 1.6 us of a 67,108,864-value
    // tail, where the tail runs one wave per SIMD and every wait shows)
    if (nd >= 64 * R) {
        for (uint32_t k = lane + 64 * R; k < nd + 64; k += 64) {  // also its last dword
            const uint32_t v = k <= nd ? (uint32_t)((((uint64_t)src[k + 1] << 32) | src[k]) >> (8 * head)) : 0u;
            if (k < nd) d32[k] = v;
            if (k - lane == (nd & ~63u)) last = readlane(v, (int)(nd & 63));
        }
    }
    if (lane < tail) dst[head + 4 * nd + lane] = (uint8_t)(last >> (8 * lane));
}

// One wave writes a run of n bytes (a group's escape exponents) from `src`
// (its staging slot) into the LDS gather buffer at byte `pos`, with lo / hi
// as for store_run.  Lanes with nothing to store write their own word of
// `dummy` instead of being masked off, so only a run past the loaded dwords
// (over 256 R bytes) branches: masked stores, each with its own change of
// the execution mask, made the gather cost more scalar instructions than
// vector ones (67,108,864 values: the tail 13.4 -> 13.0 us, event-timed).
// The shifts stay: unaligned LDS dword stores of the source dwords as they
// are give the same bytes but take the tail to 19.6 us.
template <int R>
__device__ __forceinline__ void gather_run(uint8_t* buf, uint32_t pos, const uint32_t* src, uint32_t n,
                                           const uint32_t (&lo)[R], const uint32_t (&hi)[R], uint32_t* dummy) {
    const uint32_t lane = lane_id();
    const uint32_t head = min(n, (4u - (pos & 3u)) & 3u);
    const uint32_t nd = (n - head) >> 2, tail = (n - head) & 3u;
    uint8_t* d = buf + pos + head;  // 4-byte aligned
    uint32_t v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t k = lane + 64 * r;
        v[r] = (uint32_t)((((uint64_t)hi[r] << 32) | lo[r]) >> (8 * head));
        *(k < nd ? reinterpret_cast<uint32_t*>(d + 4 * k) : dummy + lane) = v[r];
    }
    // the output dword after the whole ones (its first `tail` bytes); a long
    // run's comes with the rest of it (gather_rest)
    const bool longrun = nd >= 64 * R;
    uint32_t sel = v[0];
#pragma unroll
    for (int r = 1; r < R; ++r) sel = (nd >> 6) == (uint32_t)r ? v[r] : sel;
    const uint32_t last = readlane(sel, (int)(nd & 63));
    // the head bytes (lanes 0-2, from source dword 0) and the tail bytes
    // (lanes 4-6) in one byte store
    const uint32_t first = readlane(lo[0], 0);
    const bool is_head = lane < head, is_tail = !longrun && lane >= 4 && lane - 4 < tail;
    uint8_t* bp = is_head ? buf + pos + lane
                          : (is_tail ? d + 4 * nd + (lane - 4) : reinterpret_cast<uint8_t*>(dummy + 64) + lane);
    *bp = (uint8_t)(lane < 4 ? first >> (8 * lane) : last >> (8 * ((lane - 4) & 3)));
}

// The rest of a long run (over 256 R bytes) that gather_run started: its
// dwords past the loaded ones, read from the staging slot here, and its
// last bytes.
template <int R>
__device__ __forceinline__ void gather_rest(uint8_t* buf, uint32_t pos, const uint32_t* src, uint32_t n) {
    const uint32_t lane = lane_id();
    const uint32_t head = min(n, (4u - (pos & 3u)) & 3u);
    const uint32_t nd = (n - head) >> 2, tail = (n - head) & 3u;
    if (nd < 64 * R) return;  // uniform
    uint8_t* d = buf + pos + head;
    uint32_t last = 0;
    for (uint32_t k = lane + 64 * R; k < nd + 64; k += 64) {
        const uint32_t w = k <= nd ? (uint32_t)((((uint64_t)src[k + 1] << 32) | src[k]) >> (8 * head)) : 0u;
        if (k < nd) reinterpret_cast<uint32_t*>(d)[k] = w;
        if (k - lane == (nd & ~63u)) last = readlane(w, (int)(nd & 63));
    }
    if (lane < tail) d[4 * nd + lane] = (uint8_t)(last >> (8 * lane));
}

// Values [v0, min(n, v0 + C)) of a segment into its raw stream (after the
// 64-byte header), 16-byte words, four in flight per thread.  Not inlined:
// its registers stay out of the placement path's allocation.
static __device__ __noinline__ void copy_raw_chunk(const uint16_t* __restrict__ in, uint8_t* st,
                                                   uint64_t n, uint64_t v0, uint32_t C) {
    const uint32_t m = (uint32_t)min((uint64_t)C, n - v0), words = m / 8u;
    const u32x4* src = reinterpret_cast<const u32x4*>(in + v0);
    u32x4* dst = reinterpret_cast<u32x4*>(st + kHeaderBytes + 2ull * v0);
    const uint32_t step = blockDim.x;
    uint32_t i = threadIdx.x;
    for (; i + 3 * step < words; i += 4 * step) {
        u32x4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = src[i + u * step];
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[i + u * step] = w[u];
    }
    for (; i < words; i += step) dst[i] = src[i];
    const uint32_t j = 8u * words + threadIdx.x;  // the last partial word, value by value
    if (threadIdx.x < 8 && j < m)
        reinterpret_cast<uint16_t*>(st + kHeaderBytes)[v0 + j] = in[v0 + j];
}

constexpr int kPlaceR = 2;  // source dword pairs per lane and group loaded ahead

template <int GPW>
constexpr uint32_t place_buf_bytes() {  // LDS gather buffer: 8 workgroups per CU
    return 4u * GPW * kGroup + 16u < 19584u ? 4u * GPW * kGroup + 16u : 19584u;
}

template <int GPW>
struct PlaceLds {
    u32x4 buf[place_buf_bytes<GPW>() / 16];
    uint32_t dummy[80];  // where lanes with nothing to store in the gather write
};

// One chunk's geometry (the few segment fields placement needs, not the
// whole descriptor: fewer registers) and its groups' staged source dwords.
template <int GPW>
struct PlaceChunk {
    uint32_t seg, local;   // segment, chunk index in it
    uint8_t* st;           // the segment's stream
    uint64_t n, in_off, gtab_off, esc_off;
    const uint32_t* gcnt;  // the chunk's first group's count
    uint64_t gc0;          // the chunk's first group in the segment
    uint32_t ng;           // its groups
    const uint32_t* slot0; // its first group's staging slot
    uint32_t c_raw;        // lane < ng: group lane's escape count
    uint32_t lo[GPW][kPlaceR], past[GPW];
};

// The chunk's geometry.  A workgroup of up to 4 waves per chunk; wave w
// owns the chunk's groups w, w + nw, ... (GPW = groups per wave).
template <int GPW>
__device__ __forceinline__ void place_begin(const PlaceArgs& a, uint32_t ci, PlaceChunk<GPW>& pc) {
    const ItemDesc cd = a.single ? ItemDesc{0u, ci} : a.chunks[ci];
    const SegDesc sd = a.single ? a.seg0 : a.segs[cd.seg];
    pc.seg = cd.seg;
    pc.local = cd.local;
    pc.st = a.out + sd.out_off;
    pc.n = sd.n;
    pc.in_off = sd.in_off;
    pc.gtab_off = sd.gtab_off;
    pc.esc_off = sd.esc_off;
    const uint32_t gpc = a.chunk_elems / kGroup;
    pc.gc0 = (uint64_t)cd.local * gpc;
    pc.ng = (uint32_t)min((uint64_t)gpc, sd.g - pc.gc0);
    pc.gcnt = a.gcnt + sd.group_base + pc.gc0;
    pc.slot0 = reinterpret_cast<const uint32_t*>(a.staging) + (uint64_t)(sd.group_base + pc.gc0) * (kGroup / 4);
}

// The group counts and the staged source dwords of this wave's groups (the
// next dword of each comes from the next lane, lane 63's from the next round
// or, for the last round, from one scalar load).  MASKED = false: every
// load unconditional and in one round (groups past the chunk's end read its
// last group's slot and are not stored).  MASKED = true: the wave's group
// counts first, then only the dwords each group's run covers (the reads
// then track the escapes; one more round, for callers that have other
// latency to hide it behind), except each group's first dword per lane
// (256 bytes), loaded at once: a run of typical length gets most of its
// bytes without waiting for its count, and a short run's few extra bytes
// cost nothing measurable (67,108,864 values with 20% escapes: a failed
// prediction's tail 1.0 us shorter, a held one's unchanged; 2.45%: the
// same).
template <int GPW, bool MASKED>
__device__ __forceinline__ void place_load(const PlaceArgs& a, PlaceChunk<GPW>& pc) {
    const uint32_t lane = lane_id(), wave = wave_id(), nw = blockDim.x >> 6;
    const uint32_t* gcnt = pc.gcnt;
    pc.c_raw = gcnt[min(lane, pc.ng - 1)];
    uint32_t cnt[GPW];
    if (MASKED) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) cnt[q] = gcnt[min(wave + nw * q, pc.ng - 1)];  // wave-uniform
    }
    if (MASKED) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint32_t j = min(wave + nw * q, pc.ng - 1);
            pc.lo[q][0] = pc.slot0[(uint64_t)j * (kGroup / 4) + lane];
        }
    }
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const uint32_t j = min(wave + nw * q, pc.ng - 1);
        const uint32_t* s32 = pc.slot0 + (uint64_t)j * (kGroup / 4);
        if (!MASKED) {
#pragma unroll
            for (int r = 0; r < kPlaceR; ++r) pc.lo[q][r] = s32[lane + 64 * r];
            pc.past[q] = s32[64 * kPlaceR];  // wave-uniform address
        } else {
            // dwords 0 .. n/4 + 1 carry the run (an output dword needs its
            // source dword and the next); dwords past it are never stored
            const uint32_t need = min(cnt[q], kGroup) / 4 + 2;
#pragma unroll
            for (int r = 1; r < kPlaceR; ++r)
                pc.lo[q][r] = lane + 64 * r < need ? s32[lane + 64 * r] : 0u;
            pc.past[q] = 64 * kPlaceR < need ? s32[64 * kPlaceR] : 0u;
        }
    }
}

// The chunk's group table entries and its escape run at escape offset
// `prefix` (or, raw, its values).  go() is called by every thread (it may
// hold workgroup barriers) once the run is gathered in LDS (a group's run
// past 256 R bytes only up to there: its rest is gathered after go()) and
// before any global store; if it returns false nothing is stored and this
// returns false.  Contains workgroup barriers.
template <int GPW, typename Go>
__device__ __forceinline__ bool place_finish(const PlaceArgs& a, PlaceChunk<GPW>& pc, uint32_t prefix,
                                             bool raw, PlaceLds<GPW>& lds, Go&& go) {
    constexpr int R = kPlaceR;
    constexpr uint32_t kBuf = place_buf_bytes<GPW>();
    const uint32_t lane = lane_id(), wave = wave_id(), nw = blockDim.x >> 6;
    uint8_t* st = pc.st;
    const uint32_t ng = pc.ng;
    const uint64_t gc0 = pc.gc0;
    const uint32_t* slot0 = pc.slot0;
    auto& s_buf = lds.buf;
    // every wave scans the chunk's group counts itself: each group's offset
    // in the chunk's run (gb) and its count (gn) are read from registers
    const uint32_t c = lane < ng ? pc.c_raw : 0u;
    const uint32_t incl = wave_inclusive_scan(c);
    const uint32_t gb = incl - c, gn = min(c, kGroup);
    const uint32_t t = readlane(incl, 63);
    // counts that would leave the escape region mean no copy (never the case
    // when the encoder wrote them)
    const uint32_t pre = (uint64_t)prefix + t <= pc.n ? prefix : 0xFFFFFFFFu;
    uint32_t hi[GPW][R];
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t nxt = r + 1 < R ? readlane(pc.lo[q][r + 1 < R ? r + 1 : r], 0) : pc.past[q];
            const uint32_t sh = dpp<kDppWaveShl1>(pc.lo[q][r]);
            hi[q][r] = lane == 63 ? nxt : sh;
        }
    if (raw) {
        if (go())
            copy_raw_chunk(a.in + pc.in_off, st, pc.n, (uint64_t)pc.local * a.chunk_elems, a.chunk_elems);
        lds_barrier();  // the LDS is rewritten by the next chunk
        return true;
    }
    const uint32_t off = pre & 15u;  // esc_off and the stream start are multiples of 256
    const bool fits = pre != 0xFFFFFFFFu && off + t <= kBuf;
    uint8_t* buf = reinterpret_cast<uint8_t*>(s_buf);
    if (fits) {  // gathered at its final alignment modulo 16
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint32_t j = wave + nw * q;
            if (j < ng)
                gather_run<R>(buf, off + readlane(gb, (int)j), slot0 + (uint64_t)j * (kGroup / 4), readlane(gn, (int)j),
                              pc.lo[q], hi[q], lds.dummy);
        }
        lds_barrier();
    }
    if (!go()) {
        lds_barrier();  // the LDS is rewritten by the next chunk
        return false;
    }
    // long runs (over 256 R bytes) are finished only now: after a failed
    // prediction their staged bytes are never read (a uniform test: every
    // wave holds every group's count).  A first pass whose window was one
    // step too high leaves about 40% of the 67,108,864-value tensor's values
    // escaping, with runs past 512 bytes: a failed prediction's tail
    // 47.5 -> 46.9 us, a held one's unchanged
    if (fits && __ballot(gn >= 256u * R) != 0) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint32_t j = wave + nw * q;
            if (j < ng) gather_rest<R>(buf, off + readlane(gb, (int)j), slot0 + (uint64_t)j * (kGroup / 4), readlane(gn, (int)j));
        }
        lds_barrier();
    }
    if (wave == 0 && lane < ng) reinterpret_cast<uint16_t*>(st + pc.gtab_off)[gc0 + lane] = (uint16_t)gb;
    if (pre == 0xFFFFFFFFu) {
        lds_barrier();  // the LDS is rewritten by the next chunk
        return true;
    }
    uint8_t* esc = st + pc.esc_off + pre;
    if (!fits) {  // a run longer than the LDS buffer: group by group
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint32_t j = wave + nw * q;
            if (j < ng)
                store_run<R>(esc + readlane(gb, (int)j), slot0 + (uint64_t)j * (kGroup / 4), readlane(gn, (int)j), pc.lo[q], hi[q]);
        }
        lds_barrier();  // the LDS is rewritten by the next chunk
        return true;
    }
    // bytes [off, off + t) of the buffer go to esc - off (16-byte aligned):
    // whole 16-byte blocks, then the partial first and last blocks bytewise.
    // The blocks are stored non-temporally: nothing reads them before the
    // stream is sent, and the streaming hint shortens the kernel's end
    // (tail 15.2 µs against 16.5 for 67,108,864 values, event-timed).
    uint8_t* base = esc - off;
    const uint32_t end = off + t, nblk = (end + 15) >> 4;
    for (uint32_t b = threadIdx.x; b < nblk; b += blockDim.x)
        if ((b << 4) >= off && (b << 4) + 16 <= end)
            __builtin_nontemporal_store(s_buf[b], reinterpret_cast<u32x4*>(base + (b << 4)));
    if (threadIdx.x < 32 && t) {
        const uint32_t p = threadIdx.x < 16 ? threadIdx.x : 16 * (nblk - 1) + (threadIdx.x - 16);
        const bool first_partial = off > 0 || end < 16;
        const bool last_partial = nblk > 1 && (end & 15u) != 0;
        const bool mine = threadIdx.x < 16 ? first_partial && p >= off && p < end
                                           : last_partial && p < end;
        if (mine) base[p] = buf[p];
    }
    lds_barrier();  // the LDS is rewritten by the next chunk
    return true;
}

}  // namespace zc
