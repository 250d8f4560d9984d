// zc_internal.h -- shared definitions of the gfx950 codec kernels.
//
// Stream format version 1 (ZipCCL scribe notes, "Key idea and contribution",
// techniques 1 and 2): header, chunk table (u32 escape offset of each chunk),
// group table (u16 escape offset of each 2048-value group inside its chunk),
// then per group three planes of 64 u32 words (bit b of each 3-bit code in
// plane b), then one sign+mantissa byte per value, then the escape exponents
// in code order.  The two-level index lets any group be decoded on its own.
//
// Lane view used by every kernel: a group is 4 tiles of 512 values; lane l of
// a wave owns values 512k + 8l + j (k = 0..3 tile, j = 0..7 slot), read with
// one 16-byte load per tile.  Inside the lane's plane word, value (k, j) sits
// at bit p = 16 (j & 1) + 4 (j >> 1) + k.  That order is what the packed
// 16-bit arithmetic below produces without any per-bit work: the code of the
// low half of dword m lands in nibble m of a tile word, the high half in
// nibble m + 4, and the four tile words interleave bit by bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zc {

constexpr uint32_t kGroup = 2048;
constexpr uint32_t kHeaderBytes = 64;
constexpr uint32_t kMagic = 0x3142435Au;  // "ZCB1"
constexpr uint32_t kVersion = 1;
constexpr uint32_t kMaxStreams = 16;
constexpr uint32_t kSigmaBlock = 16384;  // values per moment partial (or the chunk, if smaller)

// Per-segment geometry, built on the host at plan time.
struct SegDesc {
    uint64_t n;          // values
    uint64_t in_off;     // element offset in the BF16 buffers
    uint64_t out_off;    // byte offset of the stream in the compressed buffer
    uint64_t gtab_off;   // region offsets relative to the stream start
    uint64_t code_off;
    uint64_t sm_off;
    uint64_t esc_off;
    uint64_t max_bytes;  // worst-case stream size
    uint32_t k;          // chunks
    uint32_t g;          // groups
    uint32_t nsb;        // moment blocks
    uint32_t sb_base;    // first moment block of this segment in the plan's list
    uint32_t group_base; // first group of this segment in the plan's list
    uint32_t chunk_base; // first chunk of this segment in the plan's list
};

struct ItemDesc {  // a moment block, chunk or group: its segment and index inside it
    uint32_t seg;
    uint32_t local;
};

struct Partial {  // per-chunk moments
    double s1, s2;
    uint64_t n;
    uint64_t pad;
};

struct SegStat {  // per-segment window statistics
    double s1, s2, var;
    uint64_t n;
    uint32_t L;
    uint32_t pad[3];
};

// Workspace carve-up (all offsets 256-aligned), computed on the host.
struct WsLayout {
    uint64_t status;    // u32 per group: rejection bits of the last decode
    uint64_t partials;  // Partial per moment block
    uint64_t flags;     // u64 per chunk: look-back state of the encoder
    uint64_t stats;     // SegStat per segment
    uint64_t lflags;    // u32 per segment: the encoder's window word
    uint64_t ticket;    // u32: encoder work counter
    uint64_t total;
};

// Look-back flag word of a chunk: state in bits 62-63, count in bits 0-31.
//   aggregate: the chunk's escape count
//   prefix:    escapes of the segment up to and including the chunk
constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagPrefix = 2ull << 62;

// ---------------------------------------------------------------- helpers
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_sub_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, (u16x2)(x - y));
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(x, y));
}

// Byte permute: bytes 0-3 come from `lo`, 4-7 from `hi`.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) {
    return (mask & a) | (~mask & b);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Index of the calling wave in its workgroup, as a wave-uniform value (so
// that values derived from it live in scalar registers).
__device__ __forceinline__ uint32_t wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t t = __shfl_up(x, d, 64);
        if (lane >= (uint32_t)d) x += t;
    }
    return x;
}

// Value index inside a group of the value at (lane, plane bit p).
__device__ __forceinline__ uint32_t group_index(uint32_t lane, uint32_t p) {
    return 512u * (p & 3u) + 8u * lane + 2u * ((p >> 2) & 3u) + (p >> 4);
}

// Plane-bit mask of the lane's values with group index < valid.
__device__ __forceinline__ uint32_t valid_bits(uint32_t lane, uint32_t valid) {
    uint32_t v = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        int64_t left = (int64_t)valid - (int64_t)(512u * k + 8u * lane);
        uint32_t nv = left <= 0 ? 0u : (left >= 8 ? 8u : (uint32_t)left);
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j)
            if (j < nv) v |= 1u << (16u * (j & 1u) + 4u * (j >> 1) + k);
    }
    return v;
}

// Load the lane's 8 values of each tile of group g (zero past n).
__device__ __forceinline__ void load_group(const uint16_t* __restrict__ x, uint64_t n,
                                           uint64_t g, uint32_t lane, u32x4 (&w)[4]) {
    const uint64_t base = (uint64_t)kGroup * g + 8u * lane;
    if ((uint64_t)kGroup * (g + 1) <= n) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = *reinterpret_cast<const u32x4*>(x + base + 512u * k);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t b = base + 512u * k;
            if (b + 8 <= n) {
                w[k] = *reinterpret_cast<const u32x4*>(x + b);
            } else {
                uint32_t d[4] = {0, 0, 0, 0};
                for (uint32_t j = 0; j < 8; ++j)
                    if (b + j < n) d[j >> 1] |= (uint32_t)x[b + j] << (16 * (j & 1));
                w[k] = u32x4{d[0], d[1], d[2], d[3]};
            }
        }
    }
}

}  // namespace zc
