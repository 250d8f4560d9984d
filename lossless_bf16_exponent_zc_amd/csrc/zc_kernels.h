// zc_kernels.h -- kernel argument blocks and kernel declarations.
#pragma once

#include "zc_internal.h"

namespace zc {

struct SigmaArgs {
    const SegDesc* segs;
    const ItemDesc* blocks;  // moment blocks
    const uint16_t* in;
    Partial* partials;
    uint64_t* flags;         // encoder state, cleared here: look-back words,
    uint32_t* lflags;        // window words,
    uint32_t* ticket;        // work counter
    uint32_t block_elems;
    uint32_t chunk_elems;
};

struct ResetArgs {
    uint64_t* flags;
    uint32_t* lflags;
    uint32_t* ticket;
    uint32_t nchunks;
    uint32_t nseg;
};

struct EmptyArgs {
    const SegDesc* segs;
    uint8_t* out;
    uint64_t* stream_bytes;
    SegStat* stats;
    uint32_t chunk_elems;
    uint32_t forced_L;
};

struct EncodeArgs {
    const SegDesc* segs;
    const ItemDesc* chunks;
    const uint16_t* in;
    uint8_t* out;
    uint64_t* stream_bytes;
    const Partial* partials;
    SegStat* stats;
    uint32_t* lflags;   // per segment: 0x100 | L once the window is known
    uint64_t* flags;
    uint32_t* ticket;
    uint32_t chunk_elems;
    uint32_t forced_L;  // 0: window from the moments
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
__global__ void zc_reset_flags(ResetArgs a);
__global__ void zc_empty_headers(EmptyArgs a);
template <int GPW>
__global__ void zc_encode(EncodeArgs a);
template <bool REDUCE>
__global__ void zc_decode(DecodeArgs a);

}  // namespace zc
