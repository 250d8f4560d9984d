// zc_decode.hip -- decompress, and decompress fused with a fixed-order sum.
//
// Decoding inverts the exponent coding of the ZipCCL scribe notes ("Key idea
// and contribution", technique 1): e = L + code for codes 0..6, the next
// escape byte for code 7, sign and mantissa from the raw byte.  The fused
// variant is the receive side of a compressed reduce-scatter (technique 3
// names the reduce-scatter path; the UCCL-Zip page's abstract argues for
// fusing the codec into the collective to drop extra memory traffic): every
// shard is decoded tile by tile into registers and added in shard order in
// fp32, so the only global write is the final BF16 sum.
//
// One workgroup per chunk; each wave owns GPW consecutive groups.  Planes are
// read first so every lane knows where its escapes start (wave scan + LDS
// scan over the chunk, plus the chunk table); the group is then rebuilt with
// packed ops, staged in LDS, and each lane patches its escaped values.
// Every stream is validated first; a chunk that fails writes nothing.
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

}  // namespace

template <int GPW, bool REDUCE>
__global__ __launch_bounds__(1024) void zc_decode(DecodeArgs a) {
    __shared__ uint32_t s_gbase[32];
    __shared__ uint32_t s_total;
    __shared__ u32x4 s_stage[16][256];

    const uint32_t chunk = blockIdx.x;
    const ChunkDesc cd = a.chunks[chunk];
    const SegDesc sd = a.segs[cd.seg];
    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const uint64_t g0 = (uint64_t)cd.local * (a.chunk_elems / kGroup) + (uint64_t)wave * GPW;
    const uint64_t tail_valid = sd.n - (uint64_t)kGroup * (sd.g ? sd.g - 1 : 0);
    uint16_t* __restrict__ out = a.out + sd.in_off;
    uint16_t* stage = reinterpret_cast<uint16_t*>(s_stage[wave]);

    float acc[REDUCE ? GPW : 1][REDUCE ? 32 : 1];
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
        uint32_t t0 = 0, t1 = 0, L = 0;
        if (!bad) {
            const uint32_t* table = reinterpret_cast<const uint32_t*>(st + kHeaderBytes);
            const uint64_t E = ld<uint64_t>(st + 24);
            L = st[6];
            t0 = table[cd.local];
            t1 = table[cd.local + 1];
            if (t0 > t1 || t1 > E || (cd.local == 0 && t0 != 0) ||
                (cd.local + 1 == sd.k && t1 != E))
                bad |= kBadTable;
        }
        if (bad) {
            bad_all |= bad;
            continue;
        }

        // planes, escape masks, per-lane escape offsets inside the chunk
        uint32_t P[GPW][3], M[GPW], base[GPW];
        uint32_t padbad = 0;
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint64_t g = g0 + q;
            if (g < sd.g) {
                const uint8_t* cw = st + sd.code_off + 768ull * g + 4u * lane;
#pragma unroll
                for (int b = 0; b < 3; ++b) P[q][b] = ld<uint32_t>(cw + 256 * b);
                if (g + 1 == sd.g && tail_valid < kGroup) {
                    const uint32_t V = valid_bits(lane, (uint32_t)tail_valid);
                    if ((P[q][0] | P[q][1] | P[q][2]) & ~V) padbad = 1;
                    const uint8_t* sw = st + sd.sm_off + 2048ull * g + 8u * lane;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (ld<uint64_t>(sw + 512 * k) & sm_pad_mask(lane, (uint32_t)tail_valid, k))
                            padbad = 1;
                }
            } else {
                P[q][0] = P[q][1] = P[q][2] = 0;
            }
            M[q] = P[q][0] & P[q][1] & P[q][2];
            const uint32_t cnt = __builtin_popcount(M[q]);
            const uint32_t incl = wave_inclusive_scan(cnt);
            base[q] = incl - cnt;
            if (lane == 63) s_gbase[wave * GPW + q] = incl;
        }
        const uint32_t anypad = __syncthreads_or(padbad) ? kBadPad : 0u;
        if (threadIdx.x < 64) {
            const uint32_t ng = nwaves * GPW;
            const uint32_t v = threadIdx.x < ng ? s_gbase[threadIdx.x] : 0u;
            const uint32_t incl = wave_inclusive_scan(v);
            if (threadIdx.x < ng) s_gbase[threadIdx.x] = incl - v;
            if (threadIdx.x == 63) s_total = incl;
        }
        __syncthreads();
        bad = anypad | (s_total != t1 - t0 ? kBadCount : 0u);
        if (bad) {
            bad_all |= bad;
            __syncthreads();  // s_gbase / s_total are rewritten by the next stream
            continue;
        }

        const uint32_t L7 = (L << 7) | (L << 23);
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint64_t g = g0 + q;
            if (g >= sd.g) continue;
            u32x2 sm[4];
            const uint8_t* sw = st + sd.sm_off + 2048ull * g + 8u * lane;
#pragma unroll
            for (int k = 0; k < 4; ++k) sm[k] = ld<u32x2>(sw + 512 * k);
            u32x4 o[4];
            decode_group(P[q], sm, L7, o);
            // stage, patch escaped exponents, read back
#pragma unroll
            for (int k = 0; k < 4; ++k) s_stage[wave][64 * k + lane] = o[k];
            __builtin_amdgcn_wave_barrier();
            const uint8_t* esc = st + sd.esc_off + t0 + s_gbase[wave * GPW + q] + base[q];
            uint32_t m = M[q], i = 0;
            while (m) {
                const uint32_t p = __builtin_ctz(m);
                m &= m - 1;
                const uint32_t r = group_index(lane, p);
                const uint32_t e = esc[i++];
                stage[r] = (uint16_t)((stage[r] & 0x807Fu) | (e << 7));
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = s_stage[wave][64 * k + lane];
            __builtin_amdgcn_wave_barrier();

            if (REDUCE) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) {
                        const float lo = __uint_as_float(o[k][mm] << 16);
                        const float hi = __uint_as_float(o[k][mm] & 0xFFFF0000u);
                        float& a0 = acc[REDUCE ? q : 0][REDUCE ? 8 * k + 2 * mm : 0];
                        float& a1 = acc[REDUCE ? q : 0][REDUCE ? 8 * k + 2 * mm + 1 : 0];
                        a0 = s == 0 ? lo : a0 + lo;
                        a1 = s == 0 ? hi : a1 + hi;
                    }
            } else {
                const uint64_t base_i = (uint64_t)kGroup * g + 8u * lane;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint64_t b = base_i + 512u * k;
                    if (b + 8 <= sd.n) {
                        *reinterpret_cast<u32x4*>(out + b) = o[k];
                    } else {
                        for (uint32_t j = 0; j < 8; ++j)
                            if (b + j < sd.n) out[b + j] = (uint16_t)(o[k][j >> 1] >> (16 * (j & 1)));
                    }
                }
            }
        }
        __syncthreads();  // s_gbase / s_total are rewritten by the next stream
    }

    if (REDUCE && bad_all == 0 && a.nstreams > 0) {
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const uint64_t g = g0 + q;
            if (g >= sd.g) continue;
            const uint64_t base_i = (uint64_t)kGroup * g + 8u * lane;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                u32x4 o;
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    o[mm] = to_bf16(acc[REDUCE ? q : 0][REDUCE ? 8 * k + 2 * mm : 0]) |
                            (to_bf16(acc[REDUCE ? q : 0][REDUCE ? 8 * k + 2 * mm + 1 : 0]) << 16);
                const uint64_t b = base_i + 512u * k;
                if (b + 8 <= sd.n) {
                    *reinterpret_cast<u32x4*>(out + b) = o;
                } else {
                    for (uint32_t j = 0; j < 8; ++j)
                        if (b + j < sd.n) out[b + j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
                }
            }
        }
    }
    if (threadIdx.x == 0) a.status[chunk] = bad_all;
}

template __global__ void zc_decode<1, false>(DecodeArgs);
template __global__ void zc_decode<2, false>(DecodeArgs);
template __global__ void zc_decode<1, true>(DecodeArgs);
template __global__ void zc_decode<2, true>(DecodeArgs);

}  // namespace zc
