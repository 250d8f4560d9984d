// zc_moments.h -- fp64 pairwise moments and the variance -> window rule.
//
// ZipCCL scribe notes, "Key idea and contribution", technique 1: the window
// of frequent exponents is taken from the tensor's standard deviation.  The
// moments S1 = sum v and S2 = sum v^2 are pairwise fp64 sums in index order
// (padding with +0.0 to a power of two), so every device gets the same bits.
#pragma once

#include "zc_internal.h"

namespace zc {

// Pairwise sum of 8 values in registers (index order).
__device__ __forceinline__ double tree8(double (&v)[8]) {
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i += 2 * s) v[i] = v[i] + v[i + s];
    return v[0];
}

// fp64 value of the BF16 pattern in the high / low half of a word.
__device__ __forceinline__ double bf16_hi(uint32_t w) {
    return (double)__uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ double bf16_lo(uint32_t w) {
    return (double)__uint_as_float(w << 16);
}

__device__ __forceinline__ double make_f64(uint32_t lo, uint32_t hi) {
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    return make_f64(dpp<CTRL>((uint32_t)u), dpp<CTRL>((uint32_t)(u >> 32)));
}

__device__ __forceinline__ double swizzle_x16_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    return make_f64(swizzle_x16((uint32_t)u), swizzle_x16((uint32_t)(u >> 32)));
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    return make_f64(readlane((uint32_t)u, l), readlane((uint32_t)(u >> 32), l));
}

// Pairwise tree over the lanes of a 16-lane row: afterwards every lane of
// the row holds the row's sum.  Each step adds the partner block's sum; once
// a block is uniform, the half-row and row mirrors reach the partner block
// (fp64 addition is commutative, so both blocks of a pair compute one value).
__device__ __forceinline__ double row_tree(double v) {
    v = v + dpp_f64<kDppQuadX1>(v);
    v = v + dpp_f64<kDppQuadX2>(v);
    v = v + dpp_f64<kDppHalfMirror>(v);
    v = v + dpp_f64<kDppMirror>(v);
    return v;
}

// Pairwise tree over lanes 0..31 (valid in every lane of that half).
__device__ __forceinline__ double half_tree(double v) {
    v = row_tree(v);
    return v + swizzle_x16_f64(v);
}

// Pairwise tree over the 64 lanes, as a wave-uniform value.
__device__ __forceinline__ double wave_tree(double v) {
    v = half_tree(v);
    return readlane_f64(v, 0) + readlane_f64(v, 32);
}

// L = 127 + max{k : var >= C0 * 4^k}, clamped to 1..248; var = 0 gives 1.
// C0 = 1 / (4 u^2) with u the root of Phi(256u) - Phi(128u) = Phi(2u) - Phi(u):
// the 7-binade window of largest N(0, var) mass.
__device__ __forceinline__ uint32_t window_from_variance(double var) {
    if (!(var > 0.0)) return 1u;
    const double C0 = 0x1.5b16bd46a1a0cp+9;
    // var in [2^e, 2^(e+1)) and C0 in [2^9, 2^10) bound the answer to
    // floor((e-10)/2) .. floor((e-8)/2); step down to the first k that fits.
    const int e = ilogb(var);
    int k = (e - 8) >> 1;
    while (var < ldexp(C0, 2 * k)) --k;
    const int L = 127 + k;
    return (uint32_t)(L < 1 ? 1 : (L > 248 ? 248 : L));
}

struct MomentScratch {  // LDS for one workgroup's reduction
    double v1[16], v2[16];
    unsigned long long n[16];
    double r1[512], r2[512];
};

// The reduction below runs on 256 threads; a round covers T*m leaves
// (T <= 256 threads, m <= 16 leaves each).  The encoder stores block b's
// moments at the slot where the round's loads are lane-consecutive.
constexpr uint32_t kReduceThreads = 256;

struct LeafOrder {
    uint32_t lt, lm;  // log2 T, log2 m
};

__device__ __forceinline__ LeafOrder leaf_order(uint32_t B) {
    const uint32_t lp = B <= 1 ? 0u : 32u - (uint32_t)__builtin_clz(B - 1);  // log2 P
    const uint32_t lt = lp < 8u ? lp : 8u;
    const uint32_t lm = lp - lt < 4u ? lp - lt : 4u;
    return LeafOrder{lt, lm};
}

// Leaf b = (r T + t) m + i (round r, thread t, position i) lives at slot
// r T m + i T + t.  Both lie in [0, P), P = 2^ceil(log2 B).
__device__ __forceinline__ uint32_t leaf_slot(uint32_t b, LeafOrder o) {
    const uint32_t lr = o.lt + o.lm;
    const uint32_t w = b & ((1u << lr) - 1u);
    return ((b >> lr) << lr) | ((w & ((1u << o.lm) - 1u)) << o.lt) | (w >> o.lm);
}

// Pairwise sums over B leaf partials (positions past B and past the rounds
// taken as -0.0, the identity, so the result is the tree over the leaves
// alone), by a workgroup of kReduceThreads threads.  A round covers an
// aligned run of T*m leaves: thread t sums m <= 16 of them pairwise, a wave
// butterfly and a tree over the waves join the threads.  Rounds (at most 512: a segment has fewer than 2^32 values, 2^21
// leaves of 2048, and T*m = 4096 when there are several rounds) are joined
// by a last pairwise tree.  Inputs at leaf slots (leaf_slot), so each load
// instruction reads consecutive slots.  The result is valid in thread 0.
// The round's loads (load_round) can be issued ahead of other work (the
// masks are applied by finish_round); finish_round contains __syncthreads:
// call it from uniform control flow only.
struct ReduceShape {
    LeafOrder o;
    uint32_t T, m, rounds;
};

__device__ __forceinline__ ReduceShape reduce_shape(uint32_t B) {
    ReduceShape r;
    r.o = leaf_order(B);
    r.T = 1u << r.o.lt;
    r.m = 1u << r.o.lm;
    r.rounds = (B <= 1 ? 1u : (1u << (32 - __builtin_clz(B - 1)))) >> (r.o.lt + r.o.lm);
    return r;
}

struct RoundLoads {  // raw loads; leaves past B are masked when the round is finished
    double v1[16], v2[16];
    uint32_t n[16];
};

__device__ __forceinline__ void load_round(const double* ps1, const double* ps2, const uint32_t* pn,
                                           const ReduceShape& sh, uint32_t r, RoundLoads& L) {
    const uint32_t tid = threadIdx.x, T = sh.T, m = sh.m;
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) {  // loads only: nothing here waits for them
        const uint32_t slot = (r * T * m) + (i < m ? i : 0u) * T + (tid < T ? tid : 0u);  // < P
        L.v1[i] = ps1[slot];
        L.v2[i] = ps2[slot];
        L.n[i] = pn[slot];
    }
}

__device__ __forceinline__ void finish_round(RoundLoads& L, uint32_t B, const ReduceShape& shp,
                                             uint32_t r, MomentScratch& sh, uint64_t& nn) {
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    constexpr uint32_t nw = kReduceThreads / 64;
    uint32_t rn = 0;  // at most 16 * 16384 values per thread and round
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) {
        const uint32_t leaf = (r * shp.T + tid) * shp.m + i;
        const bool ok = tid < shp.T && i < shp.m && leaf < B;
        L.v1[i] = ok ? L.v1[i] : -0.0;  // no leaf: the identity
        L.v2[i] = ok ? L.v2[i] : -0.0;
        rn += ok ? L.n[i] : 0u;
    }
#pragma unroll
    for (uint32_t h = 1; h < 16; h <<= 1)
#pragma unroll
        for (uint32_t i = 0; i < 16; i += 2 * h) {
            L.v1[i] = L.v1[i] + L.v1[i + h];
            L.v2[i] = L.v2[i] + L.v2[i + h];
        }
    const double r1 = wave_tree(L.v1[0]), r2 = wave_tree(L.v2[0]);
    rn = wave_sum(rn);
    if (lane == 0) {
        sh.v1[wave] = r1;
        sh.v2[wave] = r2;
        sh.n[wave] = rn;
    }
    __syncthreads();
    if (wave == 0) {  // lanes 0..15 join the waves' sums: a 16-leaf butterfly
        double t1 = lane < nw ? sh.v1[lane] : -0.0, t2 = lane < nw ? sh.v2[lane] : -0.0;
        t1 = row_tree(t1);
        t2 = row_tree(t2);
        if (lane == 0) {
            sh.r1[r] = t1;
            sh.r2[r] = t2;
            for (uint32_t i = 0; i < nw; ++i) nn += sh.n[i];
        }
    }
    __syncthreads();
}

// finish_round with the round's loads in two halves of 8 leaves, each half
// loaded and reduced before the next is requested: half the registers, one
// more memory round trip.  The same sums: a thread's 16-leaf tree is the add
// of the trees over its first and its last 8 leaves, and leaves past B (or
// past m) are -0.0, the identity, as in finish_round.
__device__ __forceinline__ void halves_round(const double* ps1, const double* ps2, const uint32_t* pn,
                                             uint32_t B, const ReduceShape& shp, uint32_t r,
                                             MomentScratch& sh, uint64_t& nn) {
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = wave_id(), T = shp.T, m = shp.m;
    constexpr uint32_t nw = kReduceThreads / 64;
    double h1[2], h2[2];
    uint32_t rn = 0;  // at most 16 * 16384 values per thread and round
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
        double v1[8], v2[8];
        uint32_t n[8];
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {  // loads only: nothing here waits for them
            const uint32_t i = 8 * h + u;
            const uint32_t slot = (r * T * m) + (i < m ? i : 0u) * T + (tid < T ? tid : 0u);  // < P
            v1[u] = ps1[slot];
            v2[u] = ps2[slot];
            n[u] = pn[slot];
        }
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {
            const uint32_t i = 8 * h + u;
            const uint32_t leaf = (r * T + tid) * m + i;
            const bool ok = tid < T && i < m && leaf < B;
            v1[u] = ok ? v1[u] : -0.0;  // no leaf: the identity
            v2[u] = ok ? v2[u] : -0.0;
            rn += ok ? n[u] : 0u;
        }
        h1[h] = tree8(v1);
        h2[h] = tree8(v2);
        __builtin_amdgcn_sched_barrier(0);  // the second half's loads after the first is reduced
    }
    const double r1 = wave_tree(h1[0] + h1[1]), r2 = wave_tree(h2[0] + h2[1]);
    rn = wave_sum(rn);
    if (lane == 0) {
        sh.v1[wave] = r1;
        sh.v2[wave] = r2;
        sh.n[wave] = rn;
    }
    __syncthreads();
    if (wave == 0) {  // lanes 0..15 join the waves' sums: a 16-leaf butterfly
        double t1 = lane < nw ? sh.v1[lane] : -0.0, t2 = lane < nw ? sh.v2[lane] : -0.0;
        t1 = row_tree(t1);
        t2 = row_tree(t2);
        if (lane == 0) {
            sh.r1[r] = t1;
            sh.r2[r] = t2;
            for (uint32_t i = 0; i < nw; ++i) nn += sh.n[i];
        }
    }
    __syncthreads();
}

// The wave joins the rounds: lane l the 8 rounds 8l .. 8l+7, then the lanes.
__device__ __forceinline__ void join_rounds(const MomentScratch& sh, uint32_t rounds, uint64_t nn,
                                            double& s1, double& s2, uint64_t& n) {
    const uint32_t lane = lane_id();
    if (wave_id() == 0) {
        double t1[8], t2[8];
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t j = 8 * lane + i;
            t1[i] = j < rounds ? sh.r1[j] : -0.0;
            t2[i] = j < rounds ? sh.r2[j] : -0.0;
        }
        const double u1 = wave_tree(tree8(t1)), u2 = wave_tree(tree8(t2));
        if (lane == 0) {
            s1 = u1;
            s2 = u2;
            n = nn;
        }
    }
}

// Population variance of the finite values from the moments: three
// separately rounded operations; n = 0 or var <= 0 gives 0.
__device__ __forceinline__ double variance(double s1, double s2, uint64_t n) {
    if (n == 0) return 0.0;
    const double d = (double)n;
    const double mean = s1 / d;
    const double ex2 = s2 / d;
    const double sq = mean * mean;
    const double var = ex2 - sq;
    return var > 0.0 ? var : 0.0;
}

// Header fields known before encoding (everything but E and total).
__device__ __forceinline__ void write_static_header(uint8_t* st, const SegDesc& sd, uint32_t C,
                                                    uint32_t L) {
    *reinterpret_cast<uint32_t*>(st + 0) = kMagic;
    *reinterpret_cast<uint32_t*>(st + 4) = kVersion | (L << 16);  // flags byte = 0
    *reinterpret_cast<uint64_t*>(st + 8) = sd.n;
    *reinterpret_cast<uint32_t*>(st + 16) = C;
    *reinterpret_cast<uint32_t*>(st + 20) = sd.k;
    *reinterpret_cast<uint64_t*>(st + 40) = sd.code_off;
    *reinterpret_cast<uint64_t*>(st + 48) = sd.sm_off;
    *reinterpret_cast<uint64_t*>(st + 56) = sd.esc_off;
}

// Header of a raw stream (the values follow it as they are): flags 1, L 0,
// E 0, total 64 + 2N, region offsets 0.  Written in place of the coded
// header when coding would not shrink the tensor, the ZipCCL notes' switch
// between the compressed and the native path by compression benefit
// ("Key idea and contribution", third technique), taken per stream.
__device__ __forceinline__ void write_raw_header(uint8_t* st, const SegDesc& sd, uint32_t C) {
    *reinterpret_cast<uint32_t*>(st + 0) = kMagic;
    *reinterpret_cast<uint32_t*>(st + 4) = kVersion | (kFlagRaw << 24);  // L byte = 0
    *reinterpret_cast<uint64_t*>(st + 8) = sd.n;
    *reinterpret_cast<uint32_t*>(st + 16) = C;
    *reinterpret_cast<uint32_t*>(st + 20) = sd.k;
    *reinterpret_cast<uint64_t*>(st + 24) = 0;
    *reinterpret_cast<uint64_t*>(st + 32) = kHeaderBytes + 2ull * sd.n;
    *reinterpret_cast<uint64_t*>(st + 40) = 0;
    *reinterpret_cast<uint64_t*>(st + 48) = 0;
    *reinterpret_cast<uint64_t*>(st + 56) = 0;
}

}  // namespace zc
