// zc_kernels.h -- kernel argument blocks and kernel declarations.
#pragma once

#include "zc_internal.h"

namespace zc {

struct EncodeArgs {
    const SegDesc* segs;
    const ItemDesc* pairs;  // per wave: (segment, pair index); segment ~0 pads a segment's workgroups
    const uint16_t* in;
    uint8_t* out;
    const SegStat* stats;   // the previous window (the first pass's prediction)
    Partials part;          // per block: escape count; with moments, the moments
    uint32_t* pred;         // per segment: the window the first pass used
    uint32_t* done;         // per segment: window workgroups done re-coding (first pass clears)
    uint32_t* zero;         // one word the first pass sets to 0 (a target for masked loads)
    uint8_t* staging;       // 2048 bytes per group (+16): the group's escape exponents
    uint32_t* gcnt;         // per group: its escape count
    uint32_t* flag;         // per segment: the finish kernel's verdict (first pass clears)
    uint64_t* agg;          // per chunk: look-back words (first pass clears)
    uint64_t* fpart;        // per segment, 8 parts x 4 words: the finish kernel's
                            // moment parts (first pass sets them to ~0, no value)
    uint32_t chunk_elems;
    uint32_t block_elems;   // moment block (16,384 values, or the chunk if smaller)
    uint32_t forced_L;      // nonzero: this window for every segment, no moments
    uint32_t single;        // one segment: seg0 is it, items are (0, index)
    SegDesc seg0;
};

struct WindowArgs {
    EncodeArgs enc;           // for segments the first pass coded with another window
    const ItemDesc* items;    // per workgroup: (segment, index among the segment's wr)
    SegStat* stats;           // written by each segment's workgroup 0
    uint64_t* stream_bytes;
    uint32_t chunk_elems;
    uint32_t chunk_blocks;    // moment blocks per chunk: 1, 2 or 4
    uint32_t raw_fallback;    // a raw stream when the coded one would be longer
};

struct PlaceArgs {
    const SegDesc* segs;
    const ItemDesc* chunks;
    uint8_t* out;
    const uint8_t* staging;
    const uint32_t* gcnt;
    const uint16_t* in;     // the values, copied into raw streams
    uint32_t chunk_elems;
    uint32_t nchunks;
    uint32_t single;        // one segment: seg0 is it, chunk i is (0, i)
    SegDesc seg0;
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
    const uint8_t* dummy;            // >= 2048 readable bytes no decoder writes: the loads'
                                     // stand-in where a buffer lacks a region
    uint32_t single;                 // one segment: seg0 is it, group i is (0, i)
    SegDesc seg0;
};

// The merged tail of compress: window workgroups (one per segment) first,
// then one placement workgroup per chunk.
struct FinishArgs {
    WindowArgs win;
    PlaceArgs place;
    const ItemDesc* parts;  // per window workgroup: (segment, part)
    uint32_t nwin;          // window workgroups
};

struct NativeReduceArgs {
    const uint16_t* in[kMaxStreams];  // uncompressed shards, 16-byte aligned
    uint16_t* out;
    uint64_t n;                       // values per shard
};

template <bool SINGLE>
__global__ void zc_window(WindowArgs a);
template <bool MOMENTS, int GW>  // GW: groups per wave (2: 256 threads, 1: 512)
__global__ void zc_encode(EncodeArgs a);
template <int GPW>
__global__ void zc_place_escapes(PlaceArgs a);
template <bool SINGLE>
__global__ void zc_decode(DecodeArgs a);
__global__ void zc_decode_reduce(DecodeArgs a);
template <int S>
__global__ void zc_decode_reduce_wide(DecodeArgs a);
template <int S>
__global__ void zc_reduce_native(NativeReduceArgs a);
template <bool SINGLE, int GPW>
__global__ void zc_finish(FinishArgs a);

}  // namespace zc
