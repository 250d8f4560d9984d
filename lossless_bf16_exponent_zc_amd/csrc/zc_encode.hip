// zc_encode.hip -- exponent coding of BF16 values (compress).
//
// ZipCCL scribe notes, "Key idea and contribution": technique 1 (each value
// whose exponent lies in the window becomes a 3-bit code, sign and mantissa
// stay raw, other exponents are kept whole in a separate stream) and
// technique 2 (GPU kernel with a communication-aware, aligned layout).
//
// One workgroup per chunk; each wave owns GPW consecutive 2048-value groups.
//  0. the workgroup of a segment's first chunk joins the segment's moment
//     partials (fp64, pairwise) into the variance, picks the window and
//     publishes it; the other workgroups issue their loads first and then
//     wait for the window (that chunk always holds an earlier ticket);
//  1. one 16-byte load per lane per tile; packed 16-bit ops give (e - L)
//     clamped to 7 for two values at a time; nibble packing and a 4-way bit
//     interleave turn the lane's 32 codes into its three plane words;
//  2. sign+mantissa bytes from two byte permutes and a bit select; planes and
//     sign+mantissa bytes go out at once (their offsets are static);
//  3. the lane's 32 exponent bytes go to LDS in plane-bit order, so only its
//     escape mask (code 7 = all three plane bits set) stays in registers;
//  4. escape counts are scanned across the wave (shuffles) and across the
//     chunk (LDS), which gives the group table; the chunk's offset in the
//     segment's escape stream comes from a decoupled look-back in which one
//     wave reads 64 earlier chunks per round (an atomic work counter orders
//     the workgroups, so every chunk waited on is already running);
//  5. each lane writes its escape exponents, contiguous in code order.
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

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
    return v;
}

__device__ __forceinline__ uint64_t load_flag(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_flag(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Run by one whole wave.  Publishes the chunk's count, then finds the
// exclusive escape prefix of chunk `ci` (local index `local` in its segment):
// lane i of a round looks at the chunk base + i + 1 places back; a round is
// usable once every chunk before the nearest published prefix has at least
// published its count.
__device__ uint32_t look_back(uint64_t* flags, uint32_t ci, uint32_t local, uint32_t total) {
    const uint32_t lane = lane_id();
    if (local == 0) {
        if (lane == 0) store_flag(flags + ci, kFlagPrefix | total);
        return 0;
    }
    if (lane == 0) store_flag(flags + ci, kFlagAggregate | total);
    uint32_t acc = 0;
    for (uint32_t base = 0;; base += 64) {
        const uint32_t d = base + lane + 1;
        const bool valid = d <= local;
        uint64_t f;
        uint32_t fp;
        for (;;) {
            f = valid ? load_flag(flags + ci - d) : 0;
            const uint32_t st = (uint32_t)(f >> 62);
            const uint64_t valid_m = __ballot(valid);
            const uint64_t pre_m = __ballot(valid && st == 2);
            const uint64_t rdy_m = __ballot(valid && st != 0);
            fp = pre_m ? (uint32_t)__builtin_ctzll(pre_m) : 64u;
            const uint64_t need = fp == 64 ? valid_m : ((1ull << fp) - 1);
            if ((rdy_m & need) == need && (fp < 64 || valid_m == ~0ull)) break;
            __builtin_amdgcn_s_sleep(1);
        }
        acc += wave_sum(valid && lane <= fp ? (uint32_t)f : 0u);
        if (fp < 64) break;
    }
    if (lane == 0) store_flag(flags + ci, kFlagPrefix | (acc + total));
    return acc;
}

}  // namespace

template <int GPW>
__global__ __launch_bounds__(1024) void zc_encode(EncodeArgs a) {
    __shared__ uint32_t s_ticket, s_prefix, s_L;
    __shared__ uint32_t s_gbase[32];
    __shared__ MomentScratch s_mom;
    // per wave and group: the 32 exponent bytes of each lane at a 36-byte
    // stride (9 dwords, so byte reads at lane-dependent offsets spread banks)
    __shared__ uint32_t s_q[16][GPW * 64 * 9];

    const uint32_t lane = lane_id(), wave = wave_id(), nwaves = blockDim.x >> 6;
    if (threadIdx.x == 0) s_ticket = atomicAdd(a.ticket, 1u);
    __syncthreads();
    const uint32_t ci = uniform(s_ticket);
    const ItemDesc cd = a.chunks[ci];
    const SegDesc sd = a.segs[cd.seg];
    const uint16_t* __restrict__ x = a.in + sd.in_off;
    uint8_t* __restrict__ st = a.out + sd.out_off;
    const uint32_t gpc = a.chunk_elems / kGroup;
    const uint64_t g0 = (uint64_t)cd.local * gpc + (uint64_t)wave * GPW;

    // The segment's window: its first chunk joins the moment partials (before
    // issuing its own loads, to keep registers free); the others load first,
    // then wait for the window word.
    if (cd.local == 0) {
        double s1 = 0.0, s2 = 0.0;
        uint64_t n = 0;
        if (!a.forced_L) reduce_partials(a.partials + sd.sb_base, sd.nsb, blockDim.x, s_mom, s1, s2, n);
        if (threadIdx.x == 0) {
            SegStat ss{};
            ss.s1 = s1;
            ss.s2 = s2;
            ss.n = n;
            ss.var = a.forced_L ? 0.0 : variance(s1, s2, n);
            ss.L = a.forced_L ? a.forced_L : window_from_variance(ss.var);
            a.stats[cd.seg] = ss;
            s_L = ss.L;
            __hip_atomic_store(a.lflags + cd.seg, 0x100u | ss.L, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            write_static_header(st, sd, a.chunk_elems, ss.L);
        }
        // zero the gap between the group table and the code region
        for (uint64_t i = sd.gtab_off + 2ull * sd.g + threadIdx.x; i < sd.code_off; i += blockDim.x)
            st[i] = 0;
    }

    // the first group's loads go out before the window is known; later groups
    // are loaded one at a time (fewer registers, two workgroups per CU)
    u32x4 w[GPW][4];
#pragma unroll
    for (int q = 0; q < GPW; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) w[q][k] = u32x4{0, 0, 0, 0};
    if (g0 < sd.g) load_group(x, sd.n, g0, lane, w[0]);

    if (cd.local != 0 && threadIdx.x == 0) {
        uint32_t f;
        while ((f = __hip_atomic_load(a.lflags + cd.seg, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)) == 0)
            __builtin_amdgcn_s_sleep(2);
        s_L = f & 0xFFu;
    }
    __syncthreads();
    const uint32_t L = uniform(s_L);
    const uint32_t L7 = (L << 7) | (L << 23);

    uint32_t M[GPW], excl[GPW];
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const uint64_t g = g0 + q;
        M[q] = 0;
        if (q > 0 && g < sd.g) load_group(x, sd.n, g, lane, w[q]);
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
            uint32_t Q[8];
            exponent_bytes(w[q], Q);
            uint32_t* qs = s_q[wave] + 9 * (64 * q + lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) qs[i] = Q[i];
        }
        const uint32_t cnt = __builtin_popcount(M[q]);
        const uint32_t incl = wave_inclusive_scan(cnt);
        excl[q] = incl - cnt;
        if (lane == 63) s_gbase[wave * GPW + q] = incl;
    }
    __syncthreads();

    if (wave == 0) {
        const uint32_t ng = nwaves * GPW;
        const uint32_t v = lane < ng ? s_gbase[lane] : 0u;
        const uint32_t incl = wave_inclusive_scan(v);
        const uint32_t total = __shfl(incl, 63, 64);
        const uint64_t g = (uint64_t)cd.local * gpc + lane;
        if (lane < ng) {
            s_gbase[lane] = incl - v;
            if (g < sd.g) reinterpret_cast<uint16_t*>(st + sd.gtab_off)[g] = (uint16_t)(incl - v);
        }
        const uint32_t prefix = look_back(a.flags, ci, cd.local, total);
        if (lane == 0) {
            s_prefix = prefix;
            reinterpret_cast<uint32_t*>(st + kHeaderBytes)[cd.local] = prefix;
            if (cd.local + 1 == sd.k) {
                const uint64_t E = (uint64_t)prefix + total;
                reinterpret_cast<uint32_t*>(st + kHeaderBytes)[sd.k] = (uint32_t)E;
                *reinterpret_cast<uint64_t*>(st + 24) = E;
                *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off + E;
                a.stream_bytes[cd.seg] = sd.esc_off + E;
            }
        }
    }
    __syncthreads();

    // escape exponents: each lane's are contiguous, in plane-bit order
    const uint32_t prefix = s_prefix;
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        const uint8_t* qb = reinterpret_cast<const uint8_t*>(s_q[wave] + 9 * (64 * q + lane));
        uint8_t* esc = st + sd.esc_off + prefix + s_gbase[wave * GPW + q] + excl[q];
        uint32_t m = M[q], i = 0;
        while (m) {
            const uint32_t p = __builtin_ctz(m);
            m &= m - 1;
            esc[i++] = qb[p];
        }
    }
}

template __global__ void zc_encode<1>(EncodeArgs);
template __global__ void zc_encode<2>(EncodeArgs);

}  // namespace zc
