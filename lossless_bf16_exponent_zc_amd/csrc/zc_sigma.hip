// zc_sigma.hip -- window selection from the tensor's standard deviation.
//
// ZipCCL scribe notes, "Key idea and contribution", technique 1: the frequent
// exponent range is taken directly from the standard deviation, with no
// online histogram and no sort.  Here the statistic is the population
// variance of the finite values, from fp64 sums S1 = sum v and S2 = sum v^2
// taken by a pairwise tree over the segment (padded to a power of two with
// +0.0).  The tree's shape depends only on indices, so the result is the
// same bit pattern on any device: a lane sums 32 consecutive values, a wave
// butterfly joins lanes into 2048-value blocks, the workgroup joins blocks
// into one moment block (16,384 values, or the chunk if smaller), and the
// finalize kernel joins the moment blocks of each segment.
//
// Window: the 7 exponents [L, L+6] holding the most N(0, var) mass, i.e.
// L = 127 + max{k : var >= C0 * 4^k} clamped to 1..248, with
// C0 = 1 / (4 u^2) and u the root of Phi(256u) - Phi(128u) = Phi(2u) - Phi(u)
// (the sigma-relative position where shifting the window by one binade
// gains as much mass at the top as it loses at the bottom).
#include "zc_kernels.h"

namespace zc {

namespace {

// fp64 value of the BF16 pattern in the high / low half of a word.
__device__ __forceinline__ double bf16_hi(uint32_t w) {
    return (double)__uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ double bf16_lo(uint32_t w) {
    return (double)__uint_as_float(w << 16);
}

// Pairwise sum of 8 values in registers (index order).
__device__ __forceinline__ double tree8(double (&v)[8]) {
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int i = 0; i < 8; i += 2 * s) v[i] = v[i] + v[i + s];
    return v[0];
}

// Moments of 8 consecutive values (one 16-byte word).  Values at or past n
// are zero; an Inf or NaN among them is replaced by +0.0 and not counted.
__device__ __forceinline__ void moments8(const u32x4 w, uint64_t base, uint64_t n, double& s1,
                                         double& s2, uint32_t& cnt) {
    double v[8], q[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        v[2 * m] = bf16_lo(w[m]);
        v[2 * m + 1] = bf16_hi(w[m]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = v[i] * v[i];
    s1 = tree8(v);
    s2 = tree8(q);
    cnt = base >= n ? 0u : (n - base >= 8 ? 8u : (uint32_t)(n - base));
    if (!__builtin_isfinite(s2)) {  // rare: redo without the non-finite values
        cnt = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t d = w[i >> 1];
            const float f = __uint_as_float((i & 1) ? (d & 0xFFFF0000u) : (d << 16));
            const bool ok = __builtin_isfinite(f) && base + i < n;
            v[i] = ok ? (double)f : 0.0;
            q[i] = v[i] * v[i];
            cnt += ok ? 1u : 0u;
        }
        s1 = tree8(v);
        s2 = tree8(q);
    }
}

// The lane's 32 consecutive values (zero past n).
__device__ __forceinline__ void load32(const uint16_t* __restrict__ x, uint64_t n, uint64_t base,
                                       u32x4 (&w)[4]) {
    if (base + 32 <= n) {
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = *reinterpret_cast<const u32x4*>(x + base + 8 * t);
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t d[4] = {0, 0, 0, 0};
            for (uint32_t j = 0; j < 8; ++j) {
                const uint64_t i = base + 8 * t + j;
                if (i < n) d[j >> 1] |= (uint32_t)x[i] << (16 * (j & 1));
            }
            w[t] = u32x4{d[0], d[1], d[2], d[3]};
        }
    }
}

__device__ __forceinline__ double wave_tree(double v) {
    // after distance d every lane holds the sum of its aligned 2d-lane block
    // (fp64 addition is commutative, so both lanes compute the same value)
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v = v + __shfl_xor(v, d, 64);
    return v;
}

}  // namespace

// One workgroup per moment block: NWV waves own BPW consecutive 2048-value
// blocks each (lane l: values 32l .. 32l+31 of a block).  The block that
// opens a chunk also clears that chunk's encoder look-back word.
template <int NWV, int BPW>
__global__ __launch_bounds__(256) void zc_sigma_partials(SigmaArgs a) {
    const uint32_t blk = blockIdx.x;
    const ItemDesc bd = a.blocks[blk];
    const SegDesc sd = a.segs[bd.seg];
    const uint16_t* __restrict__ x = a.in + sd.in_off;
    const uint32_t lane = lane_id(), wave = wave_id();
    __shared__ double s_s1[NWV], s_s2[NWV];
    __shared__ uint32_t s_n[NWV];

    if (threadIdx.x == 0) {
        const uint64_t first = (uint64_t)bd.local * a.block_elems;
        if (first % a.chunk_elems == 0) a.flags[sd.chunk_base + first / a.chunk_elems] = 0;
    }
    if (wave < NWV) {
        double b1[BPW], b2[BPW];
        uint32_t cnt = 0;
        const uint64_t wbase = (uint64_t)bd.local * a.block_elems +
                               (uint64_t)wave * BPW * kGroup + 32u * lane;
        u32x4 w[BPW][4];
#pragma unroll
        for (int b = 0; b < BPW; ++b) load32(x, sd.n, wbase + (uint64_t)b * kGroup, w[b]);
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const uint64_t base = wbase + (uint64_t)b * kGroup;
            double a1[4], a2[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t c;
                moments8(w[b][t], base + 8 * t, sd.n, a1[t], a2[t], c);
                cnt += c;
            }
            b1[b] = wave_tree((a1[0] + a1[1]) + (a1[2] + a1[3]));
            b2[b] = wave_tree((a2[0] + a2[1]) + (a2[2] + a2[3]));
        }
#pragma unroll
        for (int s = 1; s < BPW; s <<= 1)
#pragma unroll
            for (int i = 0; i < BPW; i += 2 * s) {
                b1[i] = b1[i] + b1[i + s];
                b2[i] = b2[i] + b2[i + s];
            }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) cnt += __shfl_xor(cnt, d, 64);
        if (lane == 0) {
            s_s1[wave] = b1[0];
            s_s2[wave] = b2[0];
            s_n[wave] = cnt;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t1[NWV], t2[NWV];
        uint64_t n = 0;
#pragma unroll
        for (int i = 0; i < NWV; ++i) {
            t1[i] = s_s1[i];
            t2[i] = s_s2[i];
            n += s_n[i];
        }
#pragma unroll
        for (int s = 1; s < NWV; s <<= 1)
#pragma unroll
            for (int i = 0; i < NWV; i += 2 * s) {
                t1[i] = t1[i] + t1[i + s];
                t2[i] = t2[i] + t2[i + s];
            }
        Partial p;
        p.s1 = t1[0];
        p.s2 = t2[0];
        p.n = n;
        p.pad = 0;
        a.partials[sd.sb_base + bd.local] = p;
    }
}

__global__ __launch_bounds__(256) void zc_reset_flags(ResetArgs a) {
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < a.n; i += gridDim.x * 256) a.flags[i] = 0;
}

namespace {

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

constexpr int kMaxLevels = 10;  // up to 8 * 512 leaves per thread

}  // namespace

// One workgroup (1024 threads) per segment: joins the moment blocks, picks the
// window, writes the header fields known before encoding and resets the
// encoder's work counter.  With forced_L != 0 the moments are skipped.
__global__ __launch_bounds__(1024) void zc_sigma_finalize(FinalizeArgs a) {
    const uint32_t seg = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const SegDesc sd = a.segs[seg];
    __shared__ double s_v1[16], s_v2[16];
    __shared__ unsigned long long s_n[16];

    if (seg == 0 && tid == 0) *a.ticket = 0;

    double s1 = 0.0, s2 = 0.0, var = 0.0;
    uint64_t n = 0;
    uint32_t L;
    if (a.forced_L) {
        L = a.forced_L;
    } else {
        const uint32_t B = sd.nsb;
        uint32_t P = 1;
        while (P < B) P <<= 1;
        const uint32_t T = P < 1024 ? P : 1024;
        const uint32_t m = P / T;  // leaves per thread, a power of two
        const Partial* pp = a.partials + sd.sb_base;
        // thread t: pairwise sum of leaves [t*m, (t+1)*m): runs of 8 by an
        // unrolled tree (a shorter run is padded with +0.0), runs joined by a
        // binary counter whose level h holds a finished subtree of 2^h runs
        double r1 = 0.0, r2 = 0.0;
        uint64_t rn = 0;
        if (tid < T) {
            const uint32_t runs = m > 8 ? m / 8 : 1u, len = m > 8 ? 8u : m;
            double st1[kMaxLevels], st2[kMaxLevels];
            for (uint32_t r = 0; r < runs; ++r) {
                double v1[8], v2[8];
#pragma unroll
                for (uint32_t i = 0; i < 8; ++i) {
                    const uint32_t leaf = tid * m + r * len + i;
                    const bool ok = i < len && leaf < B;
                    v1[i] = ok ? pp[leaf].s1 : 0.0;
                    v2[i] = ok ? pp[leaf].s2 : 0.0;
                    rn += ok ? pp[leaf].n : 0;
                }
                double c1 = tree8(v1), c2 = tree8(v2);
                bool carry = true;
#pragma unroll
                for (int h = 0; h < kMaxLevels; ++h) {
                    if (carry) {
                        if ((r >> h) & 1u) {
                            c1 = st1[h] + c1;
                            c2 = st2[h] + c2;
                        } else {
                            st1[h] = c1;
                            st2[h] = c2;
                            carry = false;
                        }
                    }
                }
            }
            const int top = 31 - __builtin_clz(runs);
#pragma unroll
            for (int h = 0; h < kMaxLevels; ++h)
                if (h == top) {
                    r1 = st1[h];
                    r2 = st2[h];
                }
        }
        r1 = wave_tree(r1);
        r2 = wave_tree(r2);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) rn += __shfl_xor(rn, d, 64);
        if (lane == 0) {
            s_v1[wave] = r1;
            s_v2[wave] = r2;
            s_n[wave] = rn;
        }
        __syncthreads();
        if (tid == 0) {
            double t1[16], t2[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                t1[i] = s_v1[i];
                t2[i] = s_v2[i];
                n += s_n[i];
            }
#pragma unroll
            for (int s = 1; s < 16; s <<= 1)
#pragma unroll
                for (int i = 0; i < 16; i += 2 * s) {
                    t1[i] = t1[i] + t1[i + s];
                    t2[i] = t2[i] + t2[i + s];
                }
            s1 = t1[0];
            s2 = t2[0];
            if (n > 0) {
                const double d = (double)n;
                const double mean = s1 / d;
                const double ex2 = s2 / d;
                const double sq = mean * mean;
                var = ex2 - sq;
                if (!(var > 0.0)) var = 0.0;
            }
        }
        L = window_from_variance(var);
    }

    uint8_t* st = a.out + sd.out_off;
    if (tid == 0) {
        SegStat s;
        s.s1 = s1;
        s.s2 = s2;
        s.var = var;
        s.n = n;
        s.L = L;
        s.pad[0] = s.pad[1] = s.pad[2] = 0;
        a.stats[seg] = s;
        *reinterpret_cast<uint32_t*>(st + 0) = kMagic;
        *reinterpret_cast<uint32_t*>(st + 4) = kVersion | (L << 16);  // flags byte = 0
        *reinterpret_cast<uint64_t*>(st + 8) = sd.n;
        *reinterpret_cast<uint32_t*>(st + 16) = a.chunk_elems;
        *reinterpret_cast<uint32_t*>(st + 20) = sd.k;
        *reinterpret_cast<uint64_t*>(st + 40) = sd.code_off;
        *reinterpret_cast<uint64_t*>(st + 48) = sd.sm_off;
        *reinterpret_cast<uint64_t*>(st + 56) = sd.esc_off;
        if (sd.k == 0) {
            *reinterpret_cast<uint32_t*>(st + kHeaderBytes) = 0;  // chunk table entry 0 = E
            *reinterpret_cast<uint64_t*>(st + 24) = 0;
            *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off;
            a.stream_bytes[seg] = sd.esc_off;
        }
    }
    // zero the gap between the group table and the code region
    for (uint64_t i = sd.gtab_off + 2ull * sd.g + tid; i < sd.code_off; i += 1024) st[i] = 0;
}

template __global__ void zc_sigma_partials<1, 1>(SigmaArgs);
template __global__ void zc_sigma_partials<2, 1>(SigmaArgs);
template __global__ void zc_sigma_partials<4, 1>(SigmaArgs);
template __global__ void zc_sigma_partials<4, 2>(SigmaArgs);

}  // namespace zc
