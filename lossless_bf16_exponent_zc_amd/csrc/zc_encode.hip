// zc_encode.hip -- exponent coding of BF16 values (compress).
//
// ZipCCL scribe notes, "Key idea and contribution": technique 1 (each value
// whose exponent lies in the window becomes a 3-bit code, sign and mantissa
// stay raw, other exponents are kept whole in a separate stream) and
// technique 2 (GPU kernel with a communication-aware, aligned layout).
//
// Two kernels, so that the streaming one never waits on another wave:
//
// zc_encode, one workgroup per chunk, each wave GPW consecutive 2048-value
// groups, both loaded at once.  Per group: one 16-byte load per lane and
// tile; packed 16-bit ops give (e - L) clamped to 7 for two values at a
// time; nibble packing and a 4-way bit interleave turn the lane's 32 codes
// into its three plane words; plane words and sign+mantissa bytes go out at
// once (static offsets).  Escapes (code 7 = all three plane bits set) are
// counted and ranked across the wave with ballots; each lane puts its 32
// exponent bytes in an LDS row (plane-bit order) and copies its escapes'
// bytes from there, in code order, into the wave's packed LDS area, which
// goes out in aligned dwords to the group's staging slot.  The chunk's count is summed
// with one LDS atomic per wave; the last wave stores it and adds it to the
// coarse counts (per 256 and per 65,536 chunks).
//
// zc_place_escapes, one workgroup per chunk, one wave per encoder wave: the
// group counts give the group table; the counts before the chunk (coarse
// counts, then chunk counts: at most 32 + 255 + 255 independent loads) give
// its offset in the segment's escape stream; each wave's runs, whose source
// dwords are loaded before that offset is known, go to their place.  The
// chunk table, the header's sizes and the stream size are written here.
#include "zc_kernels.h"
#include "zc_moments.h"

namespace zc {

namespace {

__device__ __forceinline__ void encode_group(const u32x4 (&w)[4], uint32_t L7, uint32_t (&P)[3],
                                             u32x2 (&sm)[4]) {
    uint32_t Z[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t c[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)  // (e - L) << 7 per half, wrapped values clamp to 7 << 7
            c[m] = pk_min_u16(pk_sub_u16(w[k][m] & 0x7F807F80u, L7), 0x03800380u);
        // code of value 2m -> nibble m, of value 2m+1 -> nibble m + 4
        Z[k] = (c[0] >> 7) | (c[1] >> 3) | (c[2] << 1) | (c[3] << 5);
        sm[k].x = bitsel(0x80808080u, perm(w[k][1], w[k][0], 0x07050301u),
                         perm(w[k][1], w[k][0], 0x06040200u));
        sm[k].y = bitsel(0x80808080u, perm(w[k][3], w[k][2], 0x07050301u),
                         perm(w[k][3], w[k][2], 0x06040200u));
    }
#pragma unroll
    for (int b = 0; b < 3; ++b)
        P[b] = ((Z[0] >> b) & 0x11111111u) | (((Z[1] >> b) & 0x11111111u) << 1) |
               (((Z[2] >> b) & 0x11111111u) << 2) | (((Z[3] >> b) & 0x11111111u) << 3);
}

// Exponent bytes of the lane's 32 values in plane-bit order: byte p of the
// 32-byte array belongs to bit p (p = 4n + k: tile k, nibble n).
__device__ __forceinline__ void exponent_bytes(const u32x4 (&w)[4], uint32_t (&Q)[8]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        // after << 1 the exponent of the low value is byte 1, of the high one byte 3
        const uint32_t A = w[0][m] << 1, B = w[1][m] << 1, C = w[2][m] << 1, D = w[3][m] << 1;
        const uint32_t X = perm(B, A, 0x07030501u);  // A.b1 B.b1 A.b3 B.b3
        const uint32_t Y = perm(D, C, 0x07030501u);  // C.b1 D.b1 C.b3 D.b3
        Q[m] = perm(Y, X, 0x05040100u);              // low values of tiles 0..3
        Q[m + 4] = perm(Y, X, 0x07060302u);          // high values of tiles 0..3
    }
}

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

// Four waves per workgroup, each with two consecutive groups of one segment
// (item list: one entry per wave; segment ~0 pads the grid), no barrier.
// Each wave adds its escape count to its chunk's count with a non-returning
// atomic (a chunk's count gets at most 16 such adds).
// LDS per wave: 2048 + 16 bytes of packed escapes (every value of a group may
// escape) and a 32-byte exponent row per lane.
__global__ __launch_bounds__(256) void zc_encode(EncodeArgs a) {
    __shared__ uint32_t s_e[4][(kGroup + 16) / 4];  // per wave: the group's packed escapes
    __shared__ u32x4 s_row[4][64][2];                 // per wave and lane: 32 exponent bytes
    const uint32_t lane = lane_id(), wave = wave_id();
    const ItemDesc it = a.pairs[blockIdx.x * 4 + wave];  // (segment, first group / 2)
    if (it.seg == 0xFFFFFFFFu) return;                   // grid padding
    const SegDesc sd = a.segs[it.seg];
    const uint16_t* __restrict__ x = a.in + sd.in_off;
    uint8_t* __restrict__ st = a.out + sd.out_off;
    const uint32_t gpc = a.chunk_elems / kGroup;
    const uint64_t g0 = 2ull * it.local;

    u32x4 w[2][4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (g0 + q < sd.g) {
            load_group(x, sd.n, g0 + q, lane, w[q]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) w[q][k] = u32x4{0, 0, 0, 0};
        }
    }
    const uint32_t L = a.stats[it.seg].L;
    const uint32_t L7 = (L << 7) | (L << 23);

    uint8_t* ew = reinterpret_cast<uint8_t*>(s_e[wave]);
    uint32_t ctot = 0;  // escapes of the current chunk (a wave's two groups share one unless gpc = 1)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint64_t g = g0 + q;
        if (g >= sd.g) break;  // uniform
        uint32_t P[3];
        u32x2 sm[4];
        encode_group(w[q], L7, P, sm);
        if ((uint64_t)kGroup * (g + 1) > sd.n) {  // last, partial group: padding codes are 0
            const uint32_t V = valid_bits(lane, (uint32_t)(sd.n - (uint64_t)kGroup * g));
#pragma unroll
            for (int b = 0; b < 3; ++b) P[b] &= V;
        }
        uint8_t* cw = st + sd.code_off + 768ull * g + 4u * lane;
#pragma unroll
        for (int b = 0; b < 3; ++b) *reinterpret_cast<uint32_t*>(cw + 256 * b) = P[b];
        uint8_t* sw = st + sd.sm_off + 2048ull * g + 8u * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x2*>(sw + 512 * k) = sm[k];
        const uint32_t M = P[0] & P[1] & P[2];
        uint32_t tot;
        const uint32_t excl = wave_prefix_small(__builtin_popcount(M), tot);
        const uint64_t gg = sd.group_base + g;
        if (lane == 0) a.gcnt[gg] = tot;
        uint32_t Q[8];
        exponent_bytes(w[q], Q);
        s_row[wave][lane][0] = u32x4{Q[0], Q[1], Q[2], Q[3]};
        s_row[wave][lane][1] = u32x4{Q[4], Q[5], Q[6], Q[7]};
        const uint8_t* rb = reinterpret_cast<const uint8_t*>(s_row[wave][lane]);
        for (uint32_t m = M, i = 0; m; m &= m - 1, ++i) ew[excl + i] = rb[__builtin_ctz(m)];
        __builtin_amdgcn_wave_barrier();  // the wave's packed bytes are complete
        uint32_t* slot = reinterpret_cast<uint32_t*>(a.staging + gg * kGroup);
        for (uint32_t k = lane; k < (tot + 3) / 4; k += 64) slot[k] = s_e[wave][k];
        __builtin_amdgcn_wave_barrier();  // before the next group reuses the area
        ctot += tot;
        if ((g + 1) % gpc == 0 || q == 1 || g + 1 == sd.g) {  // last group of this wave in its chunk
            if (lane == 0 && ctot)
                __hip_atomic_fetch_add(a.ctot + sd.chunk_base + (uint32_t)(g / gpc), ctot,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ctot = 0;
        }
    }
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
    __shared__ uint32_t s_part[4];                          // per wave: partial sums of earlier chunks
    const uint32_t lane = lane_id(), wave = wave_id(), nw = blockDim.x >> 6;
    const ItemDesc cd = a.chunks[ci];
    const SegDesc sd = a.segs[cd.seg];
    uint8_t* st = a.out + sd.out_off;
    const uint32_t gpc = a.chunk_elems / kGroup;
    const uint64_t gc0 = (uint64_t)cd.local * gpc;  // the chunk's first group in the segment
    const uint32_t ng = (uint32_t)min((uint64_t)gpc, sd.g - gc0);
    const uint32_t* slot0 = reinterpret_cast<const uint32_t*>(a.staging) +
                            (uint64_t)(sd.group_base + gc0) * (kGroup / 4);

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
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t nxt = r + 1 < R ? readlane(lo[q][r + 1 < R ? r + 1 : r], 0) : past[q];
            const uint32_t sh = dpp<kDppWaveShl1>(lo[q][r]);
            hi[q][r] = lane == 63 ? nxt : sh;
        }
    // escapes of the segment's earlier chunks: a strided sum by all threads,
    // eight loads in flight per thread
    const uint32_t l = cd.local;
    uint32_t v = 0;
    for (uint32_t base = 0; base < l; base += 8 * blockDim.x) {
        uint32_t c8[8];
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {
            const uint32_t j = base + threadIdx.x + u * blockDim.x;
            c8[u] = j < l ? a.ctot[sd.chunk_base + j] : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) v += c8[u];
    }
    v = wave_sum(v);
    if (lane == 0) s_part[wave] = v;
    lds_barrier();
    if (wave == 0) {
        const uint32_t c = lane < ng ? a.gcnt[sd.group_base + gc0 + lane] : 0u;
        const uint32_t incl = wave_inclusive_scan(c);
        if (lane < ng) {
            reinterpret_cast<uint16_t*>(st + sd.gtab_off)[gc0 + lane] = (uint16_t)(incl - c);
            s_gb[lane] = incl - c;
            s_gn[lane] = min(c, kGroup);
        }
        uint32_t prefix = 0;
        for (uint32_t i = 0; i < nw; ++i) prefix += s_part[i];
        if (lane == 0) {
            const uint32_t t = readlane(incl, 63);
            // counts that would leave the escape region mean no copy (never
            // the case when the encoder wrote them)
            s_prefix = (uint64_t)prefix + t <= sd.n ? prefix : 0xFFFFFFFFu;
            s_t = t;
            reinterpret_cast<uint32_t*>(st + kHeaderBytes)[l] = prefix;
            if (l + 1 == sd.k) {
                const uint64_t E = (uint64_t)prefix + t;
                reinterpret_cast<uint32_t*>(st + kHeaderBytes)[sd.k] = (uint32_t)E;
                *reinterpret_cast<uint64_t*>(st + 24) = E;
                *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off + E;
                a.stream_bytes[cd.seg] = sd.esc_off + E;
            }
        }
    }
    lds_barrier();
    const uint32_t prefix = s_prefix, t = s_t;
    if (prefix == 0xFFFFFFFFu) {
        lds_barrier();  // s_* are rewritten by the next chunk
        return;
    }
    uint8_t* esc = st + sd.esc_off + prefix;
    const uint32_t off = prefix & 15u;  // esc_off and the stream start are multiples of 256
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
