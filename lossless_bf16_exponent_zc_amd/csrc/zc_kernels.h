// zc_kernels.h -- kernel argument blocks and kernel declarations.
#pragma once

#include "zc_internal.h"

namespace zc {

struct SigmaArgs {
    const SegDesc* segs;
    const ItemDesc* blocks;  // moment blocks
    const uint16_t* in;
    Partial* partials;
    uint64_t* flags;         // encoder look-back words, cleared here
    uint32_t block_elems;
    uint32_t chunk_elems;
};

struct FinalizeArgs {
    const SegDesc* segs;
    const Partial* partials;
    SegStat* stats;
    uint32_t* ticket;
    uint8_t* out;
    uint64_t* stream_bytes;
    uint32_t chunk_elems;
    uint32_t forced_L;  // 0: window from the moments
};

struct ResetArgs {
    uint64_t* flags;
    uint32_t n;
};

struct EncodeArgs {
    const SegDesc* segs;
    const ItemDesc* chunks;
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
__global__ void zc_sigma_finalize(FinalizeArgs a);
__global__ void zc_reset_flags(ResetArgs a);
template <int GPW>
__global__ void zc_encode(EncodeArgs a);
template <bool REDUCE>
__global__ void zc_decode(DecodeArgs a);

}  // namespace zc
