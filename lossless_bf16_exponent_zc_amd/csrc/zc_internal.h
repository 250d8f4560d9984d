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

#include "zc_format.h"

namespace zc {

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

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
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

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for the waves' outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane exchange without LDS addresses: DPP moves within 16-lane rows
// (plus the row broadcasts of the GFX9 family) and a 32-lane swizzle.  Every
// lane of the wave must be active.
enum : int {
    kDppQuadX1 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
    kDppQuadX2 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
    kDppMirror = 0x140,      // row_mirror: lane 15 - i of the row
    kDppHalfMirror = 0x141,  // row_half_mirror: lane 7 - i of the half row
    kDppBcast15 = 0x142,     // row_bcast:15: lane 15 of the previous row
    kDppBcast31 = 0x143,     // row_bcast:31: lane 31
    kDppWaveShl1 = 0x130,    // wave_shl:1: lane i + 1 of the wave (lane 63 reads 0)
};
__device__ __forceinline__ constexpr int dpp_row_shr(int n) { return 0x110 + n; }

// DPP move; lanes whose source is out of range, or whose row is not in
// `rows`, read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}

// Lane ^ 16 inside each 32-lane half (swizzle bit mode: and 0x1F, xor 0x10).
__device__ __forceinline__ uint32_t swizzle_x16(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Inclusive prefix sum over the 64 lanes of a wave (row shifts, then the
// row totals carried across rows by the two broadcasts).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += dpp<dpp_row_shr(1)>(x);
    x += dpp<dpp_row_shr(2)>(x);
    x += dpp<dpp_row_shr(4)>(x);
    x += dpp<dpp_row_shr(8)>(x);
    x += dpp<kDppBcast15, 0xA>(x);
    x += dpp<kDppBcast31, 0xC>(x);
    return x;
}

// Sum over the wave, as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    v += dpp<kDppQuadX1>(v);
    v += dpp<kDppQuadX2>(v);
    v += dpp<kDppHalfMirror>(v);  // each quad holds one value: the mirror pairs quads
    v += dpp<kDppMirror>(v);      // each half row holds one value
    return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// Exclusive prefix over the wave of per-lane counts; `total` is the wave's
// sum (wave-uniform).  The DPP scan, not one ballot per bit of the count:
// the same time on a held prediction, and a failed one's recode, which
// ranks every group's escapes with it at a few waves per SIMD, 0.7 us
// shorter.
__device__ __forceinline__ uint32_t wave_prefix_small(uint32_t c, uint32_t& total) {
    const uint32_t incl = wave_inclusive_scan(c);
    total = readlane(incl, 63);
    return incl - c;
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
