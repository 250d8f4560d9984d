// zc_window.h -- the per-segment tail of compress: the chunk table, E, the
// stream size and (raw fallback) the raw header, from the moment blocks'
// escape counts.  Shared by the window kernel and the merged finish kernel.
#pragma once

#include "zc_encoder.h"

namespace zc {

// Chunk table, E, total size and stream size of segment sd from the moment
// blocks' escape counts (BPC blocks per chunk), by the whole workgroup, each
// thread a run of chunks.  chunk_counts returns the thread's run total and,
// for runs of up to 8 chunks, the chunks' counts in registers (longer runs
// leave them in the table entries); place_offsets scans the runs' totals
// across the workgroup and writes the offsets.  Loads go out in batches of
// 32, unconditionally (indexes clamped, values masked).
struct ChunkRun {
    uint32_t c0, c1;
};

__device__ __forceinline__ ChunkRun chunk_run(const SegDesc& sd) {
    const uint32_t K = sd.k, per = (K + blockDim.x - 1) / blockDim.x;
    const uint32_t c0 = min(K, threadIdx.x * per);
    return ChunkRun{c0, min(K, c0 + per)};
}

struct ChunkCounts {
    uint32_t c[8];
    uint32_t run;
    bool in_table;
};

template <uint32_t BPC>
__device__ __forceinline__ void chunk_counts_t(const WindowArgs& a, const SegDesc& sd, uint8_t* st,
                                               ChunkCounts& cc) {
    constexpr uint32_t U = 32 / BPC;  // chunks per batch
    const ChunkRun cr = chunk_run(sd);
    const uint32_t last = sd.nsb - 1;
    const uint32_t* pe = a.enc.part.esc + sd.sb_base;
    cc.run = 0;
    cc.in_table = (sd.k + blockDim.x - 1) / blockDim.x > 8;  // uniform
    if (!cc.in_table) {
        // entries outside the run read a word the encoder zeroed, so every
        // load goes out unconditionally and nothing waits between them
        uint32_t v[8][BPC];
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u)
#pragma unroll
            for (uint32_t j = 0; j < BPC; ++j) {
                const uint32_t b = (cr.c0 + u) * BPC + j;
                v[u][j] = *(cr.c0 + u < cr.c1 && b <= last ? pe + b : a.enc.zero);
            }
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u) {
            uint32_t t = 0;
#pragma unroll
            for (uint32_t j = 0; j < BPC; ++j) t += v[u][j];
            cc.c[u] = t;
            cc.run += t;
        }
        return;
    }
    uint32_t* table = reinterpret_cast<uint32_t*>(st + kHeaderBytes);
    for (uint32_t c = cr.c0; c < cr.c1; c += U) {
        uint32_t v[U][BPC];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u)
#pragma unroll
            for (uint32_t j = 0; j < BPC; ++j) {
                const uint32_t b = (c + u) * BPC + j;
                v[u][j] = *(c + u < cr.c1 && b <= last ? pe + b : a.enc.zero);
            }
#pragma unroll
        for (uint32_t u = 0; u < U; ++u) {
            uint32_t t = 0;
#pragma unroll
            for (uint32_t j = 0; j < BPC; ++j) t += v[u][j];
            if (c + u < cr.c1) table[c + u] = t;
            cc.run += t;
        }
    }
}

__device__ __forceinline__ void chunk_counts(const WindowArgs& a, const SegDesc& sd, uint8_t* st,
                                             ChunkCounts& cc) {
    switch (a.chunk_blocks) {
        case 1: chunk_counts_t<1>(a, sd, st, cc); break;
        case 2: chunk_counts_t<2>(a, sd, st, cc); break;
        default: chunk_counts_t<4>(a, sd, st, cc); break;
    }
}

struct OffsetsLds {
    uint32_t w[16], base;
};

// Contains __syncthreads.
__device__ __forceinline__ void place_offsets(const WindowArgs& a, const SegDesc& sd, uint32_t seg,
                                              uint8_t* st, const ChunkCounts& cc, OffsetsLds& lds) {
    auto& s_w = lds.w;
    auto& s_base = lds.base;
    const uint32_t lane = lane_id(), wave = wave_id(), nw = blockDim.x >> 6;
    const ChunkRun cr = chunk_run(sd);
    uint32_t* table = reinterpret_cast<uint32_t*>(st + kHeaderBytes);
    const uint32_t incl = wave_inclusive_scan(cc.run);
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const uint32_t v = lane < nw ? s_w[lane] : 0u;
        const uint32_t wi = wave_inclusive_scan(v);
        if (lane < nw) s_w[lane] = wi - v;
        if (lane == 63) s_base = wi;  // E
    }
    __syncthreads();
    uint32_t at = s_w[wave] + incl - cc.run;
    if (!cc.in_table) {
#pragma unroll
        for (uint32_t u = 0; u < 8; ++u)
            if (cr.c0 + u < cr.c1) {
                table[cr.c0 + u] = at;
                at += cc.c[u];
            }
    } else {
        for (uint32_t c = cr.c0; c < cr.c1; c += 8) {
            uint32_t t[8];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u) t[u] = table[min(c + u, cr.c1 - 1)];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u)
                if (c + u < cr.c1) {
                    table[c + u] = at;
                    at += t[u];
                }
        }
    }
    if (threadIdx.x == 0) {
        const uint64_t E = s_base;
        table[sd.k] = (uint32_t)E;
        if (a.raw_fallback && sd.esc_off + E > kHeaderBytes + 2ull * sd.n) {
            write_raw_header(st, sd, a.chunk_elems);  // the placement kernel copies the values
            a.stream_bytes[seg] = kHeaderBytes + 2ull * sd.n;
            return;
        }
        *reinterpret_cast<uint64_t*>(st + 24) = E;
        *reinterpret_cast<uint64_t*>(st + 32) = sd.esc_off + E;
        a.stream_bytes[seg] = sd.esc_off + E;
    }
}

}  // namespace zc
