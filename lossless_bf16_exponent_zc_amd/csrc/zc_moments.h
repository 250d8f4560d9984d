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
    double r1[64], r2[64];
};

// Pairwise sums over B leaf partials (padded with +0.0 to P = 2^ceil(log2 B)),
// by the whole workgroup of `nthreads` (a power of two, 64..1024) threads.
// A round covers an aligned run of T*m leaves: thread t sums m <= 4 of them
// pairwise (a shorter run padded with +0.0), a wave butterfly and a tree over
// the waves join the threads.  Rounds (at most 64: 2^32 values are 2^18
// leaves, and nthreads >= 1024 here) are joined by a last pairwise tree.  The
// result is valid in thread 0.  Contains __syncthreads: call from uniform
// control flow only.
__device__ __forceinline__ void reduce_partials(const Partial* pp, uint32_t B, uint32_t nthreads,
                                                MomentScratch& sh, double& s1, double& s2,
                                                uint64_t& n) {
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const uint32_t nw = nthreads / 64;
    uint32_t P = 1;
    while (P < B) P <<= 1;
    uint32_t T, m, rounds;
    if (P <= 4 * nthreads) {
        T = P < nthreads ? P : nthreads;
        m = P / T;
        rounds = 1;
    } else {
        T = nthreads;
        m = 4;
        rounds = P / (4 * nthreads);
    }
    uint64_t nn = 0;
    for (uint32_t r = 0; r < rounds; ++r) {
        double r1 = 0.0, r2 = 0.0;
        uint32_t rn = 0;  // at most 4 * 16384 values per thread and round
        if (tid < T) {
            double v1[4], v2[4];
#pragma unroll
            for (uint32_t i = 0; i < 4; ++i) {
                const uint32_t leaf = (r * T + tid) * m + i;
                const bool ok = i < m && leaf < B;
                v1[i] = ok ? pp[leaf].s1 : 0.0;
                v2[i] = ok ? pp[leaf].s2 : 0.0;
                rn += ok ? pp[leaf].n : 0;
            }
            r1 = (v1[0] + v1[1]) + (v1[2] + v1[3]);
            r2 = (v2[0] + v2[1]) + (v2[2] + v2[3]);
        }
        r1 = wave_tree(r1);
        r2 = wave_tree(r2);
        rn = wave_sum(rn);
        if (lane == 0) {
            sh.v1[wave] = r1;
            sh.v2[wave] = r2;
            sh.n[wave] = rn;
        }
        __syncthreads();
        if (wave == 0) {  // lanes 0..15 join the waves' sums: a 16-leaf butterfly
            double t1 = lane < nw ? sh.v1[lane] : 0.0, t2 = lane < nw ? sh.v2[lane] : 0.0;
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
    if (wave == 0) {  // the wave joins the rounds: a 64-leaf tree
        double t1 = lane < rounds ? sh.r1[lane] : 0.0, t2 = lane < rounds ? sh.r2[lane] : 0.0;
        t1 = wave_tree(t1);
        t2 = wave_tree(t2);
        if (lane == 0) {
            s1 = t1;
            s2 = t2;
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

}  // namespace zc
