// zc_kernels.h -- kernel argument blocks and kernel declarations.
#pragma once

#include "zc_internal.h"

namespace zc {

struct SigmaArgs {
    const SegDesc* segs;
    const ItemDesc* blocks;  // moment blocks
    const uint16_t* in;
    Partial* partials;
    uint32_t block_elems;
};

struct WindowArgs {
    const SegDesc* segs;
    const Partial* partials;
    SegStat* stats;
    uint8_t* out;
    uint64_t* stream_bytes;  // written here for empty segments
    uint32_t* ctot;          // per-chunk escape counts, cleared here
    uint32_t chunk_elems;
    uint32_t forced_L;       // 0: window from the moments
};

struct EncodeArgs {
    const SegDesc* segs;
    const ItemDesc* pairs;  // per wave: (segment, pair index); segment ~0 pads a segment's workgroups
    const uint16_t* in;
    uint8_t* out;
    const SegStat* stats;   // the window of each segment
    uint8_t* staging;       // 2048 bytes per group (+16): the group's escape exponents
    uint32_t* gcnt;         // per group: its escape count
    uint32_t* ctot;         // per chunk: escape count, atomic adds
    uint32_t chunk_elems;
};

struct PlaceArgs {
    const SegDesc* segs;
    const ItemDesc* chunks;
    uint8_t* out;
    uint64_t* stream_bytes;
    const uint8_t* staging;
    const uint32_t* gcnt;
    const uint32_t* ctot;
    uint32_t chunk_elems;
    uint32_t nchunks;
};

struct DecodeArgs {
    const SegDesc* segs;
    const ItemDesc* groups;
    const uint8_t* in[kMaxStreams];  // reduce: one stream per shard; else the packed buffer
    uint64_t capacity;               // readable bytes behind each in[] pointer
    uint32_t nstreams;
    uint32_t chunk_elems;
    uint32_t ngroups;
    uint16_t* out;
    uint32_t* status;                // per group
};

template <int NWV, int BPW>
__global__ void zc_sigma_partials(SigmaArgs a);
__global__ void zc_window(WindowArgs a);
__global__ void zc_encode(EncodeArgs a);
template <int GPW>
__global__ void zc_place_escapes(PlaceArgs a);
__global__ void zc_decode(DecodeArgs a);
__global__ void zc_decode_reduce(DecodeArgs a);

}  // namespace zc
