// zc_kernels.h -- kernel argument blocks and kernel declarations.
#pragma once

#include "zc_internal.h"

namespace zc {

struct SigmaArgs {
    const SegDesc* segs;
    const ChunkDesc* chunks;
    const uint16_t* in;
    Partial* partials;
    uint32_t chunk_elems;
};

struct FinalizeArgs {
    const SegDesc* segs;
    const Partial* partials;
    SegStat* stats;
    uint64_t* flags;
    uint32_t* ticket;
    uint8_t* out;
    uint64_t* stream_bytes;
    uint32_t chunk_elems;
    uint32_t forced_L;  // 0: window from the moments
};

struct EncodeArgs {
    const SegDesc* segs;
    const ChunkDesc* chunks;
    const uint16_t* in;
    uint8_t* out;
    uint64_t* stream_bytes;
    const SegStat* stats;
    uint64_t* flags;
    uint32_t* ticket;
    uint32_t chunk_elems;
};

struct DecodeArgs {
    const SegDesc* segs;
    const ChunkDesc* chunks;
    const uint8_t* in[kMaxStreams];  // reduce: one stream per shard; else the packed buffer
    uint64_t capacity;               // readable bytes behind each in[] pointer
    uint32_t nstreams;
    uint32_t chunk_elems;
    uint16_t* out;
    uint32_t* status;                // per chunk
};

template <int NWV, int BPW>
__global__ void zc_sigma_partials(SigmaArgs a);
__global__ void zc_sigma_finalize(FinalizeArgs a);
template <int GPW>
__global__ void zc_encode(EncodeArgs a);
template <int GPW, bool REDUCE>
__global__ void zc_decode(DecodeArgs a);

}  // namespace zc
