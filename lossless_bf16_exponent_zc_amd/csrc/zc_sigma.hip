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
#include "zc_moments.h"

namespace zc {

namespace {

// fp64 value of the BF16 pattern in the high / low half of a word.
__device__ __forceinline__ double bf16_hi(uint32_t w) {
    return (double)__uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ double bf16_lo(uint32_t w) {
    return (double)__uint_as_float(w << 16);
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

}  // namespace

// One workgroup per moment block: NWV waves own BPW consecutive 2048-value
// blocks each (lane l: values 32l .. 32l+31 of a block).
template <int NWV, int BPW>
__global__ __launch_bounds__(256) void zc_sigma_partials(SigmaArgs a) {
    const uint32_t blk = blockIdx.x;
    const ItemDesc bd = a.blocks[blk];
    const SegDesc sd = a.segs[bd.seg];
    const uint16_t* __restrict__ x = a.in + sd.in_off;
    const uint32_t lane = lane_id(), wave = wave_id();
    __shared__ double s_s1[NWV], s_s2[NWV];
    __shared__ uint32_t s_n[NWV];

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
        cnt = wave_sum(cnt);
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

// One workgroup of 1024 threads per segment, after the moment pass: joins the
// segment's moment partials (the tree's top levels) into the variance and
// the window, and writes the statistics, the header fields known before
// encoding and the zero bytes before the code region.  It also clears the
// segment's per-chunk escape counts.  A segment without values
// gets its whole stream here (no chunk exists to write it).
__global__ __launch_bounds__(1024) void zc_window(WindowArgs a) {
    __shared__ MomentScratch s_mom;
    const uint32_t seg = blockIdx.x;
    const SegDesc sd = a.segs[seg];
    uint8_t* st = a.out + sd.out_off;
    double s1 = 0.0, s2 = 0.0;
    uint64_t n = 0;
    if (!a.forced_L && sd.nsb)
        reduce_partials(a.partials + sd.sb_base, sd.nsb, blockDim.x, s_mom, s1, s2, n);
    if (threadIdx.x == 0) {
        SegStat ss{};
        ss.s1 = s1;
        ss.s2 = s2;
        ss.n = n;
        ss.var = a.forced_L ? 0.0 : variance(s1, s2, n);
        ss.L = a.forced_L ? a.forced_L : window_from_variance(ss.var);
        a.stats[seg] = ss;
        write_static_header(st, sd, a.chunk_elems, ss.L);
        if (sd.k == 0) {  // empty: chunk table entry 0 = E = 0
            *reinterpret_cast<uint32_t*>(st + kHeaderBytes) = 0;
            *reinterpret_cast<uint64_t*>(st + 24) = 0;
            *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off;
            a.stream_bytes[seg] = sd.esc_off;
        }
    }
    for (uint64_t i = sd.gtab_off + 2ull * sd.g + threadIdx.x; i < sd.code_off; i += blockDim.x)
        st[i] = 0;
    for (uint32_t i = threadIdx.x; i < sd.k; i += blockDim.x) a.ctot[sd.chunk_base + i] = 0;
}

template __global__ void zc_sigma_partials<1, 1>(SigmaArgs);
template __global__ void zc_sigma_partials<2, 1>(SigmaArgs);
template __global__ void zc_sigma_partials<4, 1>(SigmaArgs);
template __global__ void zc_sigma_partials<4, 2>(SigmaArgs);

}  // namespace zc
