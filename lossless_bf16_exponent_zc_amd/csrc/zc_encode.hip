// zc_encode.hip -- the encoder's first pass and the escape placement.
//
// ZipCCL scribe notes, "Key idea and contribution", techniques 1 and 2.
//
// zc_encode: one workgroup item (zc_encoder.h) per workgroup, with the
// window predicted from the previous call (or the caller's fixed window);
// records the window it used per segment.  The window kernel checks the
// prediction and codes the segment again where it failed.
//
// zc_place_escapes, one workgroup per chunk, one wave per encoder wave: the
// group counts give the group table; the chunk's offset in the segment's
// escape stream comes from the chunk table; each wave's runs, whose source
// dwords are loaded before that offset is known, go to their place.
#include "zc_encoder.h"

namespace zc {

namespace {

// One wave stores a run of n bytes (a group's escape exponents) from `src`
// (the group's 2048-byte staging slot) to `dst` (global memory or LDS).  The
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
    for (uint32_t k = lane + 64 * R; k < nd + 64; k += 64) {  // long runs; also their last dword
        const uint32_t v = k <= nd ? (uint32_t)((((uint64_t)src[k + 1] << 32) | src[k]) >> (8 * head)) : 0u;
        if (k < nd) d32[k] = v;
        if (nd >= 64 * R && k - lane == (nd & ~63u)) last = readlane(v, (int)(nd & 63));
    }
    if (lane < tail) dst[head + 4 * nd + lane] = (uint8_t)(last >> (8 * lane));
}

}  // namespace

template <bool MOMENTS>
__global__ __launch_bounds__(256) void zc_encode(EncodeArgs a) {
    encode_wg<MOMENTS>(a, blockIdx.x, a.forced_L);  // 0: the predicted window
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.zero = 0u;
    const ItemDesc first = a.single ? ItemDesc{0u, 4 * blockIdx.x} : a.pairs[blockIdx.x * 4];
    if (first.local == 0 && threadIdx.x == 0) {  // the segment's first item
        a.pred[first.seg] = a.forced_L ? a.forced_L : predicted_L(a.stats[first.seg].L);
        a.done[first.seg] = 0;
    }
}

template __global__ void zc_encode<true>(EncodeArgs);
template __global__ void zc_encode<false>(EncodeArgs);

// Values [v0, min(n, v0 + C)) of a segment into its raw stream (after the
// 64-byte header), 16-byte words, four in flight per thread.  Not inlined:
// its registers stay out of the placement path's allocation.
__device__ __noinline__ void copy_raw_chunk(const uint16_t* __restrict__ in, uint8_t* st, uint64_t n,
                                               uint64_t v0, uint32_t C) {
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

// One workgroup of up to 4 waves per chunk; wave w owns the chunk's groups
// w, w + nw, ... (GPW = groups per wave).  The chunk's escape run is
// gathered in LDS at its final alignment modulo 16 and leaves in 16-byte
// stores (a run longer than the LDS buffer is stored group by group).
template <int GPW>
__device__ __forceinline__ void place_chunk(const PlaceArgs& a, uint32_t ci) {
    constexpr int R = 2;  // source dword pairs per lane and group loaded ahead
    constexpr uint32_t kBuf = 4u * GPW * kGroup + 16u < 19584u ? 4u * GPW * kGroup + 16u : 19584u;  // 8 workgroups per CU
    __shared__ u32x4 s_buf[kBuf / 16];
    __shared__ uint32_t s_gb[32], s_gn[32], s_prefix, s_t;  // group offsets in the chunk, counts
    const uint32_t lane = lane_id(), wave = wave_id(), nw = blockDim.x >> 6;
    const ItemDesc cd = a.single ? ItemDesc{0u, ci} : a.chunks[ci];
    const SegDesc sd = a.single ? a.seg0 : a.segs[cd.seg];
    uint8_t* st = a.out + sd.out_off;
    const uint32_t gpc = a.chunk_elems / kGroup;
    const uint64_t gc0 = (uint64_t)cd.local * gpc;  // the chunk's first group in the segment
    const uint32_t ng = (uint32_t)min((uint64_t)gpc, sd.g - gc0);
    const uint32_t* slot0 = reinterpret_cast<const uint32_t*>(a.staging) +
                            (uint64_t)(sd.group_base + gc0) * (kGroup / 4);

    // the chunk's escape offset (chunk table, written from the group counts
    // before this kernel runs) and the group counts go out first: the scan
    // waits only for them, not for the staging loads behind them
    const uint32_t l = cd.local;
    const uint32_t prefix = reinterpret_cast<const uint32_t*>(st + kHeaderBytes)[l];
    // a raw stream (flags byte 1, set by the window kernel) takes the values
    // as they are: no group table, no escapes (checked once the loads are in)
    const bool raw = (reinterpret_cast<const uint32_t*>(st)[1] >> 24) == kFlagRaw;
    const uint32_t c_raw = a.gcnt[sd.group_base + gc0 + min(lane, ng - 1)];

    // source dwords of this wave's groups, loaded once (inside the slots); the
    // next dword of each comes from the next lane, lane 63's from the next
    // round or, for the last round, from one scalar load
    // (all loads first, branch-free: groups past the chunk's end read its
    // last group's slot and are not stored)
    uint32_t lo[GPW][R], hi[GPW][R], past[GPW];
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const uint32_t j = min(wave + nw * q, ng - 1);
        const uint32_t* s32 = slot0 + (uint64_t)j * (kGroup / 4);
#pragma unroll
        for (int r = 0; r < R; ++r) lo[q][r] = s32[lane + 64 * r];
        past[q] = s32[64 * R];  // wave-uniform address
    }
    if (wave == 0) {
        const uint32_t c = lane < ng ? c_raw : 0u;
        const uint32_t incl = wave_inclusive_scan(c);
        if (lane < ng) {
            s_gb[lane] = incl - c;
            s_gn[lane] = min(c, kGroup);
        }
        if (lane == 0) {
            const uint32_t t = readlane(incl, 63);
            // counts that would leave the escape region mean no copy (never
            // the case when the encoder wrote them)
            s_prefix = (uint64_t)prefix + t <= sd.n ? prefix : 0xFFFFFFFFu;
            s_t = t;
        }
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t nxt = r + 1 < R ? readlane(lo[q][r + 1 < R ? r + 1 : r], 0) : past[q];
            const uint32_t sh = dpp<kDppWaveShl1>(lo[q][r]);
            hi[q][r] = lane == 63 ? nxt : sh;
        }
    if (raw) {
        copy_raw_chunk(a.in + sd.in_off, st, sd.n, (uint64_t)l * a.chunk_elems, a.chunk_elems);
        lds_barrier();  // s_* are rewritten by the next chunk
        return;
    }
    if (wave == 0 && lane < ng) reinterpret_cast<uint16_t*>(st + sd.gtab_off)[gc0 + lane] = (uint16_t)s_gb[lane];
    const uint32_t pre = s_prefix, t = s_t;
    if (pre == 0xFFFFFFFFu) {
        lds_barrier();  // s_* are rewritten by the next chunk
        return;
    }
    uint8_t* esc = st + sd.esc_off + pre;
    const uint32_t off = pre & 15u;  // esc_off and the stream start are multiples of 256
    if (off + t > kBuf) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint32_t j = wave + nw * q;
            if (j < ng) store_run<R>(esc + s_gb[j], slot0 + (uint64_t)j * (kGroup / 4), s_gn[j], lo[q], hi[q]);
        }
        lds_barrier();  // s_* are rewritten by the next chunk
        return;
    }
    uint8_t* buf = reinterpret_cast<uint8_t*>(s_buf);
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const uint32_t j = wave + nw * q;
        if (j < ng) store_run<R>(buf + off + s_gb[j], slot0 + (uint64_t)j * (kGroup / 4), s_gn[j], lo[q], hi[q]);
    }
    lds_barrier();
    // bytes [off, off + t) of the buffer go to esc - off (16-byte aligned):
    // whole 16-byte blocks, then the partial first and last blocks bytewise
    uint8_t* base = esc - off;
    const uint32_t end = off + t, nblk = (end + 15) >> 4;
    for (uint32_t b = threadIdx.x; b < nblk; b += blockDim.x)
        if ((b << 4) >= off && (b << 4) + 16 <= end) *reinterpret_cast<u32x4*>(base + (b << 4)) = s_buf[b];
    if (threadIdx.x < 32 && t) {
        const uint32_t p = threadIdx.x < 16 ? threadIdx.x : 16 * (nblk - 1) + (threadIdx.x - 16);
        const bool first_partial = off > 0 || end < 16;
        const bool last_partial = nblk > 1 && (end & 15u) != 0;
        const bool mine = threadIdx.x < 16 ? first_partial && p >= off && p < end
                                           : last_partial && p < end;
        if (mine) base[p] = buf[p];
    }
    lds_barrier();  // s_buf and s_* are rewritten by the next chunk
}

template <int GPW>
__global__ __launch_bounds__(256) void zc_place_escapes(PlaceArgs a) {
    for (uint32_t ci = blockIdx.x; ci < a.nchunks; ci += gridDim.x) place_chunk<GPW>(a, ci);
}

template __global__ void zc_place_escapes<1>(PlaceArgs);
template __global__ void zc_place_escapes<2>(PlaceArgs);
template __global__ void zc_place_escapes<4>(PlaceArgs);
template __global__ void zc_place_escapes<8>(PlaceArgs);

}  // namespace zc
