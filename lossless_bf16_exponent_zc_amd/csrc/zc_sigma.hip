// zc_sigma.hip -- window selection from the tensor's standard deviation.
//
// ZipCCL scribe notes, "Key idea and contribution", technique 1: the frequent
// exponent range is taken directly from the standard deviation, with no
// online histogram and no sort.  Here the statistic is the population
// variance of the finite values, from fp64 sums S1 = sum v and S2 = sum v^2
// taken by a pairwise tree over the segment (padded to a power of two with
// +0.0; the kernels take positions past the data as -0.0, the identity, and
// restore the padding's effect on the sign of a zero sum at the end).  The
// tree's shape depends only on indices, so the result is the same bit
// pattern on any device.  The encoder's first pass computes the tree up to
// moment blocks of 16,384 values (or the chunk, if smaller); the
// window kernel here joins the moment blocks of each segment.
//
// Window: the 7 exponents [L, L+6] holding the most N(0, var) mass, i.e.
// L = 127 + max{k : var >= C0 * 4^k} clamped to 1..248, with
// C0 = 1 / (4 u^2) and u the root of Phi(256u) - Phi(128u) = Phi(2u) - Phi(u)
// (the sigma-relative position where shifting the window by one binade
// gains as much mass at the top as it loses at the bottom).
#include "zc_window.h"

namespace zc {

// The window of each segment, the check of the first pass's prediction, and
// the segment's tables.  Workgroups of 256 threads, sd.wr per segment (item
// (segment, r)); every one of them joins the segment's moment partials (the
// tree's top levels) into the variance and the window, the same bits in
// each.  Workgroup 0 writes the statistics, the header fields known before
// encoding and the zero bytes before the code region; a segment without
// values gets its whole stream.  If the first pass used this window, its
// codes are final and workgroup 0 writes the chunk table and sizes.  If not,
// the segment's workgroups code its items again (workgroup r takes items
// r, r + wr, ...), and the last of them to finish writes the tables.
template <bool SINGLE>
__global__ __launch_bounds__(256) void zc_window(WindowArgs a) {
    __shared__ MomentScratch s_mom;
    __shared__ EncodeLds s_enc;
    __shared__ OffsetsLds s_off;
    __shared__ uint32_t s_L, s_last;
    // (SINGLE, one segment: the descriptor from the arguments; a choice made
    // at run time would read it through vector loads before anything else)
    const ItemDesc wi = SINGLE ? ItemDesc{0u, blockIdx.x} : a.items[blockIdx.x];
    const uint32_t seg = wi.seg, r = wi.local;
    const SegDesc sd_mem = SINGLE ? SegDesc{} : a.enc.segs[seg];  // read before any store
    const SegDesc& sd = SINGLE ? a.enc.seg0 : sd_mem;
    uint8_t* st = a.enc.out + sd.out_off;
    const uint32_t forced = a.enc.forced_L;
    // one round of loads: the moments' first round, and in workgroup 0 the
    // chunks' escape counts (they stand unless the prediction fails)
    const double* ps1 = a.enc.part.s1 + sd.sb_base;
    const double* ps2 = a.enc.part.s2 + sd.sb_base;
    const uint32_t* pn = a.enc.part.n + sd.sb_base;
    const bool moments = !forced && sd.nsb;
    const ReduceShape shape = reduce_shape(sd.nsb);
    RoundLoads rl;
    if (moments) load_round(ps1, ps2, pn, shape, 0, rl);
    ChunkCounts cc;
    cc.run = 0;
    cc.in_table = false;
    if (r == 0 && sd.k) chunk_counts(a, sd, st, cc);
    // the first pass's window, loaded behind the rounds above and before any
    // store, so that the check below does not wait for a load of its own
    const uint32_t pred = a.enc.pred[seg];
    double s1 = 0.0, s2 = 0.0;
    uint64_t n = 0;
    if (moments) {
        uint64_t nn = 0;
        finish_round(rl, sd.nsb, shape, 0, s_mom, nn);
        for (uint32_t k = 1; k < shape.rounds; ++k) {
            load_round(ps1, ps2, pn, shape, k, rl);
            finish_round(rl, sd.nsb, shape, k, s_mom, nn);
        }
        join_rounds(s_mom, shape.rounds, nn, s1, s2, n);
    }
    if (threadIdx.x == 0) {
        // the tree above had no leaves past the data; the segment's tree pads
        // it with +0.0 to a power of two, which changes nothing but the sign
        // of a zero sum: -0.0 becomes +0.0 when any padding leaf exists
        if ((sd.n & (sd.n - 1)) != 0) {
            s1 = s1 == 0.0 ? 0.0 : s1;
            s2 = s2 == 0.0 ? 0.0 : s2;
        }
        const double var = forced ? 0.0 : variance(s1, s2, n);
        const uint32_t L = forced ? forced : window_from_variance(var);
        s_L = L;
        if (r == 0) {
            SegStat ss{};
            ss.s1 = s1;
            ss.s2 = s2;
            ss.n = n;
            ss.var = var;
            ss.L = L;
            a.stats[seg] = ss;
            write_static_header(st, sd, a.chunk_elems, L);
            if (sd.k == 0 && a.raw_fallback) {  // empty: the header alone is shorter
                write_raw_header(st, sd, a.chunk_elems);
                a.stream_bytes[seg] = kHeaderBytes;
            } else if (sd.k == 0) {  // empty: chunk table entry 0 = E = 0
                *reinterpret_cast<uint32_t*>(st + kHeaderBytes) = 0;
                *reinterpret_cast<uint64_t*>(st + 24) = 0;
                *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off;
                a.stream_bytes[seg] = sd.esc_off;
            }
        }
    }
    if (r == 0)
        for (uint64_t i = sd.gtab_off + 2ull * sd.g + threadIdx.x; i < sd.code_off; i += blockDim.x)
            st[i] = 0;
    __syncthreads();
    const uint32_t L = s_L;
    if (sd.k == 0) return;
    if (L == pred) {  // the prediction held (always, with a fixed window)
        if (r == 0) place_offsets(a, sd, seg, st, cc, s_off);
        return;
    }
    for (uint32_t i = r; i < sd.nwg; i += sd.wr) encode_wg<false, true>(a.enc, sd.wg_base + i, L, s_enc);
    __threadfence();  // this workgroup's codes, counts and staging, before its report
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(a.enc.done + seg, 1u) == sd.wr - 1 ? 1u : 0u;
    __syncthreads();
    if (s_last) {
        __threadfence();  // the others' reports, before their counts are read
        ChunkCounts c2;
        chunk_counts(a, sd, st, c2);
        place_offsets(a, sd, seg, st, c2, s_off);
    }
}

template __global__ void zc_window<true>(WindowArgs);
template __global__ void zc_window<false>(WindowArgs);

}  // namespace zc
