// zc_decode.hip -- decompress, and decompress fused with a fixed-order sum.
//
// Decoding inverts the exponent coding of the ZipCCL scribe notes ("Key idea
// and contribution", technique 1): e = L + code for codes 0..6, the next
// escape byte for code 7, sign and mantissa from the raw byte.  The fused
// variant is the receive side of a compressed reduce-scatter (technique 3
// names the reduce-scatter path; the UCCL-Zip page's abstract argues for
// fusing the codec into the collective to drop extra memory traffic): each
// shard's group is decoded into registers and added in shard order in fp32,
// so the only global write is the final BF16 sum.
//
// One wave per 2048-value group.  The chunk table and the group table give
// the group's first escape directly, so groups decode independently: planes
// and sign+mantissa bytes are loaded, the group's escape bytes are copied to
// LDS, values are rebuilt with packed ops and staged in LDS, and each lane
// patches its escaped values.  Every stream's header, tables, counts and
// padding are checked; a group that fails writes nothing.
#include "zc_kernels.h"

namespace zc {

namespace {

constexpr uint32_t kBadMagic = 0x01, kBadWindow = 0x02, kBadShape = 0x04, kBadSize = 0x08,
                   kBadTable = 0x10, kBadCount = 0x20, kBadPad = 0x40;

template <typename T>
__device__ __forceinline__ T ld(const uint8_t* p) {
    return *reinterpret_cast<const T*>(p);
}

__device__ __forceinline__ uint32_t check_header(const uint8_t* st, uint64_t cap, const SegDesc& sd,
                                                 uint32_t C) {
    if (cap < kHeaderBytes) return kBadSize;
    uint32_t bad = 0;
    const uint32_t w1 = ld<uint32_t>(st + 4);
    const uint32_t L = (w1 >> 16) & 0xFFu;
    if (ld<uint32_t>(st) != kMagic || (w1 & 0xFFFFu) != kVersion || (w1 >> 24) != 0) bad |= kBadMagic;
    if (L < 1 || L > 248) bad |= kBadWindow;
    if (ld<uint64_t>(st + 8) != sd.n || ld<uint32_t>(st + 16) != C || ld<uint32_t>(st + 20) != sd.k ||
        ld<uint64_t>(st + 40) != sd.code_off || ld<uint64_t>(st + 48) != sd.sm_off ||
        ld<uint64_t>(st + 56) != sd.esc_off)
        bad |= kBadShape;
    const uint64_t E = ld<uint64_t>(st + 24), total = ld<uint64_t>(st + 32);
    if (E > sd.n || total != sd.esc_off + E || total > cap) bad |= kBadSize;
    return bad;
}

__device__ __forceinline__ void decode_group(const uint32_t (&P)[3], const u32x2 (&sm)[4],
                                             uint32_t L7, u32x4 (&o)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // nibble n of Z = code of the value at plane bit 4n + k
        const uint32_t Z = ((P[0] >> k) & 0x11111111u) | (((P[1] >> k) & 0x11111111u) << 1) |
                           (((P[2] >> k) & 0x11111111u) << 2);
        // code of values 2m / 2m+1 (nibbles m / m+4) moved to bits 7 / 23
        const uint32_t c0 = (Z << 7) & 0x03800380u, c1 = (Z << 3) & 0x03800380u;
        const uint32_t c2 = (Z >> 1) & 0x03800380u, c3 = (Z >> 5) & 0x03800380u;
        // sign+mantissa bytes of values 2m, 2m, 2m+1, 2m+1 -> bits 0-6 and 15 of each half
        const uint32_t lo = sm[k].x, hi = sm[k].y;
        o[k][0] = bitsel(0x7F807F80u, c0 + L7, perm(hi, lo, 0x01010000u));
        o[k][1] = bitsel(0x7F807F80u, c1 + L7, perm(hi, lo, 0x03030202u));
        o[k][2] = bitsel(0x7F807F80u, c2 + L7, perm(hi, lo, 0x05050404u));
        o[k][3] = bitsel(0x7F807F80u, c3 + L7, perm(hi, lo, 0x07070606u));
    }
}

// BF16 round to nearest even; every NaN becomes the canonical 0x7FC0.
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Bytes of the lane's tile-k sm words that lie past the end (must be zero).
__device__ __forceinline__ uint64_t sm_pad_mask(uint32_t lane, uint32_t valid, int k) {
    const int64_t left = (int64_t)valid - (int64_t)(512u * k + 8u * lane);
    if (left >= 8) return 0;
    if (left <= 0) return ~0ull;
    return ~0ull << (8 * left);
}

__device__ __forceinline__ void store_values(uint16_t* __restrict__ out, uint64_t n, uint64_t g,
                                             uint32_t lane, const u32x4 (&o)[4]) {
    const uint64_t base = (uint64_t)kGroup * g + 8u * lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t b = base + 512u * k;
        if (b + 8 <= n) {
            *reinterpret_cast<u32x4*>(out + b) = o[k];
        } else {
            for (uint32_t j = 0; j < 8; ++j)
                if (b + j < n) out[b + j] = (uint16_t)(o[k][j >> 1] >> (16 * (j & 1)));
        }
    }
}

}  // namespace

template <bool REDUCE>
__global__ __launch_bounds__(256) void zc_decode(DecodeArgs a) {
    __shared__ u32x4 s_stage[4][256];   // decoded group per wave
    __shared__ uint8_t s_esc[4][2048];  // the group's escape bytes per wave

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
    const uint32_t gg = blockIdx.x * 4 + wave;
    if (gg >= a.ngroups) return;
    const ItemDesc gd = a.groups[gg];
    const SegDesc sd = a.segs[gd.seg];
    const uint32_t g = gd.local;
    const uint32_t gpc = a.chunk_elems / kGroup;
    const uint32_t k = g / gpc;
    const bool tail = (uint64_t)kGroup * (g + 1) > sd.n;
    const uint32_t valid = (uint32_t)(sd.n - (uint64_t)kGroup * g);  // meaningful when tail
    uint16_t* stage = reinterpret_cast<uint16_t*>(s_stage[wave]);

    float acc[REDUCE ? 32 : 1];
    uint32_t bad_all = 0;

    for (uint32_t s = 0; s < a.nstreams; ++s) {
        const uint8_t* st;
        uint64_t cap;
        if (REDUCE) {
            st = a.in[s];
            cap = a.capacity;
        } else {
            st = a.in[0] + sd.out_off;
            cap = a.capacity > sd.out_off ? a.capacity - sd.out_off : 0;
            if (cap > sd.max_bytes) cap = sd.max_bytes;
        }
        uint32_t bad = check_header(st, cap, sd, a.chunk_elems);
        uint32_t t0 = 0, rel = 0, span = 0, L = 0;
        if (!bad) {
            const uint32_t* table = reinterpret_cast<const uint32_t*>(st + kHeaderBytes);
            const uint16_t* gtab = reinterpret_cast<const uint16_t*>(st + sd.gtab_off);
            const uint64_t E = ld<uint64_t>(st + 24);
            L = st[6];
            t0 = table[k];
            const uint32_t t1 = table[k + 1];
            rel = gtab[g];
            const bool last_in_chunk = (g + 1) % gpc == 0 || g + 1 == sd.g;
            const uint32_t next = last_in_chunk ? t1 - t0 : gtab[g + 1];
            if (t0 > t1 || t1 > E || (k == 0 && t0 != 0) || (k + 1 == sd.k && t1 != E) ||
                (g % gpc == 0 && rel != 0))
                bad |= kBadTable;
            else if (rel > next || next > t1 - t0)
                bad |= kBadCount;
            span = next - rel;
        }
        if (bad) {
            bad_all |= bad;
            continue;
        }

        uint32_t P[3];
        const uint8_t* cw = st + sd.code_off + 768ull * g + 4u * lane;
#pragma unroll
        for (int b = 0; b < 3; ++b) P[b] = ld<uint32_t>(cw + 256 * b);
        u32x2 sm[4];
        const uint8_t* sw = st + sd.sm_off + 2048ull * g + 8u * lane;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sm[kk] = ld<u32x2>(sw + 512 * kk);
        bool padbad = false;
        if (tail) {
            const uint32_t V = valid_bits(lane, valid);
            padbad = ((P[0] | P[1] | P[2]) & ~V) != 0;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                padbad |= (__builtin_bit_cast(uint64_t, sm[kk]) & sm_pad_mask(lane, valid, kk)) != 0;
        }
        const uint32_t M = P[0] & P[1] & P[2];
        const uint32_t cnt = __builtin_popcount(M);
        const uint32_t incl = wave_inclusive_scan(cnt);
        const uint32_t total = __shfl(incl, 63, 64);
        if (__ballot(padbad)) bad |= kBadPad;
        if (total != span) bad |= kBadCount;
        if (bad) {
            bad_all |= bad;
            continue;
        }

        // the group's escape bytes -> LDS
        const uint8_t* esc = st + sd.esc_off + t0 + rel;
        for (uint32_t i = lane; i < total; i += 64) s_esc[wave][i] = esc[i];
        const uint32_t L7 = (L << 7) | (L << 23);
        u32x4 o[4];
        decode_group(P, sm, L7, o);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) s_stage[wave][64 * kk + lane] = o[kk];
        __builtin_amdgcn_wave_barrier();
        uint32_t m = M, i = incl - cnt;
        while (m) {
            const uint32_t p = __builtin_ctz(m);
            m &= m - 1;
            const uint32_t r = group_index(lane, p);
            stage[r] = (uint16_t)((stage[r] & 0x807Fu) | ((uint32_t)s_esc[wave][i++] << 7));
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) o[kk] = s_stage[wave][64 * kk + lane];
        __builtin_amdgcn_wave_barrier();

        if (REDUCE) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const float lo = __uint_as_float(o[kk][mm] << 16);
                    const float hi = __uint_as_float(o[kk][mm] & 0xFFFF0000u);
                    float& a0 = acc[REDUCE ? 8 * kk + 2 * mm : 0];
                    float& a1 = acc[REDUCE ? 8 * kk + 2 * mm + 1 : 0];
                    a0 = s == 0 ? lo : a0 + lo;
                    a1 = s == 0 ? hi : a1 + hi;
                }
        } else {
            store_values(a.out + sd.in_off, sd.n, g, lane, o);
        }
    }

    if (REDUCE && bad_all == 0 && a.nstreams > 0) {
        u32x4 o[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
                o[kk][mm] = to_bf16(acc[REDUCE ? 8 * kk + 2 * mm : 0]) |
                            (to_bf16(acc[REDUCE ? 8 * kk + 2 * mm + 1 : 0]) << 16);
        store_values(a.out + sd.in_off, sd.n, g, lane, o);
    }
    if (lane == 0) a.status[gg] = bad_all;
}

template __global__ void zc_decode<false>(DecodeArgs);
template __global__ void zc_decode<true>(DecodeArgs);

}  // namespace zc
