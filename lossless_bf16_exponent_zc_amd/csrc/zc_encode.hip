// zc_encode.hip -- exponent coding of BF16 values (compress).
//
// ZipCCL scribe notes, "Key idea and contribution": technique 1 (each value
// whose exponent lies in the window becomes a 3-bit code, sign and mantissa
// stay raw, other exponents are kept whole in a separate stream) and
// technique 2 (GPU kernel with a communication-aware, aligned layout).
//
// One workgroup per chunk.  Each wave owns GPW consecutive 2048-value groups
// of the chunk and reads them with one 16-byte load per lane per tile.
//  1. codes: packed 16-bit ops give (e - L) clamped to 7 for two values at a
//     time; nibble-packing and a 4-way bit interleave turn a lane's 32 codes
//     into its three plane words without any per-value branch;
//  2. the sign+mantissa bytes come from two byte permutes and a bit select;
//  3. escape masks (code 7 = all three plane bits set) are counted per lane,
//     scanned across the wave (shuffles) and across the chunk (LDS);
//  4. the chunk's offset in the segment's escape stream is found by a
//     decoupled look-back over earlier chunks (an atomic work counter orders
//     the workgroups, so every chunk waited on is already running);
//  5. each lane writes its escape exponents, contiguous in code order.
#include "zc_kernels.h"

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

// Decoupled look-back: publish this chunk's escape count, add up earlier
// chunks of the segment until one with a published inclusive prefix, then
// publish our own inclusive prefix.  Returns the exclusive prefix.
__device__ uint32_t look_back(uint64_t* flags, uint32_t chunk, uint32_t local, uint32_t total) {
    if (local == 0) {
        __hip_atomic_store(&flags[chunk], kFlagPrefix | total, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        return 0;
    }
    __hip_atomic_store(&flags[chunk], kFlagAggregate | total, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    uint64_t prefix = 0;
    uint32_t j = chunk - 1;
    for (;;) {
        uint64_t f = __hip_atomic_load(&flags[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while ((f >> 62) == 0) {
            __builtin_amdgcn_s_sleep(1);
            f = __hip_atomic_load(&flags[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        prefix += f & kFlagValueMask;
        if ((f >> 62) == 2) break;
        --j;
    }
    __hip_atomic_store(&flags[chunk], kFlagPrefix | (prefix + total), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)prefix;
}

}  // namespace

template <int GPW>
__global__ __launch_bounds__(1024) void zc_encode(EncodeArgs a) {
    __shared__ uint32_t s_ticket, s_prefix;
    __shared__ uint32_t s_gbase[32];
    __shared__ u32x4 s_stage[16][256];  // one 2048-value group per wave

    const uint32_t lane = lane_id(), wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const uint32_t chunk = s_ticket;
    const ChunkDesc cd = a.chunks[chunk];
    const SegDesc sd = a.segs[cd.seg];
    const uint32_t L = a.stats[cd.seg].L;
    const uint32_t L7 = (L << 7) | (L << 23);
    const uint16_t* __restrict__ x = a.in + sd.in_off;
    uint8_t* __restrict__ st = a.out + sd.out_off;
    const uint64_t g0 = (uint64_t)cd.local * (a.chunk_elems / kGroup) + (uint64_t)wave * GPW;

    u32x4 w[GPW][4];
    uint32_t M[GPW], base[GPW];
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        if (g0 + q < sd.g) {
            load_group(x, sd.n, g0 + q, lane, w[q]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) w[q][k] = u32x4{0, 0, 0, 0};
        }
    }
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const uint64_t g = g0 + q;
        M[q] = 0;
        if (g < sd.g) {
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
            M[q] = P[0] & P[1] & P[2];
        }
        const uint32_t cnt = __builtin_popcount(M[q]);
        const uint32_t incl = wave_inclusive_scan(cnt);
        base[q] = incl - cnt;
        if (lane == 63) s_gbase[wave * GPW + q] = incl;
    }
    __syncthreads();

    if (threadIdx.x < 64) {
        const uint32_t ng = nwaves * GPW;
        const uint32_t v = threadIdx.x < ng ? s_gbase[threadIdx.x] : 0u;
        const uint32_t incl = wave_inclusive_scan(v);
        const uint32_t total = __shfl(incl, 63, 64);
        if (threadIdx.x < ng) s_gbase[threadIdx.x] = incl - v;
        if (threadIdx.x == 0) {
            const uint32_t prefix = look_back(a.flags, chunk, cd.local, total);
            s_prefix = prefix;
            reinterpret_cast<uint32_t*>(st + kHeaderBytes)[cd.local + 1] = prefix + total;
            if (cd.local + 1 == sd.k) {
                const uint64_t E = (uint64_t)prefix + total;
                *reinterpret_cast<uint64_t*>(st + 24) = E;
                *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off + E;
                a.stream_bytes[cd.seg] = sd.esc_off + E;
            }
        }
    }
    __syncthreads();

    const uint32_t prefix = s_prefix;
    const uint16_t* stage = reinterpret_cast<const uint16_t*>(s_stage[wave]);
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
#pragma unroll
        for (int k = 0; k < 4; ++k) s_stage[wave][64 * k + lane] = w[q][k];
        __builtin_amdgcn_wave_barrier();
        uint8_t* esc = st + sd.esc_off + prefix + s_gbase[wave * GPW + q] + base[q];
        uint32_t m = M[q], i = 0;
        while (m) {
            const uint32_t p = __builtin_ctz(m);
            m &= m - 1;
            esc[i++] = (uint8_t)(stage[group_index(lane, p)] >> 7);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template __global__ void zc_encode<1>(EncodeArgs);
template __global__ void zc_encode<2>(EncodeArgs);

}  // namespace zc
