// zc_encoder.h -- one encoder workgroup item: exponent codes, sign+mantissa
// bytes, staged escape exponents and escape counts of 16,384 values, and
// optionally the moment partials of the window's pairwise tree.
//
// ZipCCL scribe notes, "Key idea and contribution": technique 1 (each value
// whose exponent lies in the 7-exponent window [L, L+6] becomes a 3-bit
// code, sign and mantissa stay raw, other exponents are kept whole in a
// separate stream; the window comes from the standard deviation) and
// technique 2 (GPU kernel with an aligned, communication-aware layout).
//
// Per group (2048 values, one wave): one 16-byte load per lane and tile;
// packed 16-bit ops give (e - L) clamped to 7 for two values at a time;
// nibble packing and a 4-way bit interleave turn the lane's 32 codes into
// its three plane words; plane words and sign+mantissa bytes go out at once
// (static offsets).  The same masked exponent fields give, by a packed max,
// whether the group holds an Inf or NaN (the moments then take their careful
// path).  Escapes (code 7 = all three plane bits set) are counted
// and ranked across the wave with ballots; each lane puts its 32 exponent
// bytes in an LDS row (plane-bit order) and copies its escapes' bytes from
// there, in code order, into the wave's packed LDS area, which goes out in
// aligned dwords to the group's staging slot.
#pragma once

#include "zc_kernels.h"
#include "zc_moments.h"

namespace zc {

// mx: the largest masked exponent field (bits 7-14 of each half) of the
// lane's 32 values, per half: 0x7F80 in a half only for an Inf or NaN.
__device__ __forceinline__ void encode_group(const u32x4 (&w)[4], uint32_t L7, uint32_t (&P)[3],
                                             u32x2 (&sm)[4], uint32_t& mx) {
    uint32_t Z[4];
    mx = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t c[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {  // (e - L) << 7 per half, wrapped values clamp to 7 << 7
            const uint32_t e = w[k][m] & 0x7F807F80u;
            mx = pk_max_u16(mx, e);
            c[m] = pk_min_u16(pk_sub_u16(e, L7), 0x03800380u);
        }
        // code of value 2m -> nibble m, of value 2m+1 -> nibble m + 4
        Z[k] = (c[0] >> 7) | (c[1] >> 3) | (c[2] << 1) | (c[3] << 5);
        sm[k].x = bitsel(0x80808080u, perm(w[k][1], w[k][0], 0x07050301u),
                         perm(w[k][1], w[k][0], 0x06040200u));
        sm[k].y = bitsel(0x80808080u, perm(w[k][3], w[k][2], 0x07050301u),
                         perm(w[k][3], w[k][2], 0x06040200u));
    }
#pragma unroll
    for (int b = 0; b < 3; ++b)
        P[b] = ((Z[0] >> b) & 0x11111111u) | (((Z[1] >> b) & 0x11111111u) << 1) |
               (((Z[2] >> b) & 0x11111111u) << 2) | (((Z[3] >> b) & 0x11111111u) << 3);
}

// Exponent bytes of the lane's 32 values in plane-bit order: byte p of the
// 32-byte array belongs to bit p (p = 4n + k: tile k, nibble n).
__device__ __forceinline__ void exponent_bytes(const u32x4 (&w)[4], uint32_t (&Q)[8]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        // after << 1 the exponent of the low value is byte 1, of the high one byte 3
        const uint32_t A = w[0][m] << 1, B = w[1][m] << 1, C = w[2][m] << 1, D = w[3][m] << 1;
        const uint32_t X = perm(B, A, 0x07030501u);  // A.b1 B.b1 A.b3 B.b3
        const uint32_t Y = perm(D, C, 0x07030501u);  // C.b1 D.b1 C.b3 D.b3
        Q[m] = perm(Y, X, 0x05040100u);              // low values of tiles 0..3
        Q[m + 4] = perm(Y, X, 0x07060302u);          // high values of tiles 0..3
    }
}

// Slot of 16-byte unit u of a wave's transpose area: an XOR swizzle that
// keeps both the tile-order writes (lane j: units 64k + j) and the run-order
// reads (lane l: units 4l + t) free of LDS bank conflicts.
__device__ __forceinline__ uint32_t tslot(uint32_t u) { return u ^ ((u >> 2) & 15u); }

// Moments of 8 consecutive values, all of them real (index < n) and finite:
// the 8-leaf pairwise trees of v and v^2, with the first level of the
// squares as one fused multiply-add (v^2 of a BF16 value is exact in fp64,
// so fma(b, b, a*a) rounds a^2 + b^2 once, as the add of the two squares
// does).
__device__ __forceinline__ void moments4_half(uint32_t w0, uint32_t w1, double& a01, double& q01) {
    const double v0 = bf16_lo(w0), v1 = bf16_hi(w0), v2 = bf16_lo(w1), v3 = bf16_hi(w1);
    a01 = (v0 + v1) + (v2 + v3);
    q01 = __builtin_fma(v1, v1, v0 * v0) + __builtin_fma(v3, v3, v2 * v2);
}

__device__ __forceinline__ void moments8_full(const u32x4 w, double& s1, double& s2) {
    // two halves one after the other: only four values' fp64 temporaries live
    double a0, q0, a1, q1;
    moments4_half(w[0], w[1], a0, q0);
    __builtin_amdgcn_sched_barrier(0);
    moments4_half(w[2], w[3], a1, q1);
    s1 = a0 + a1;
    s2 = q0 + q1;
}

// The same sums with Inf/NaN values taken as +0.0 and positions at or past
// the data's end as -0.0 (the sum's identity: beyond the data the tree has
// no leaves; the window kernel restores the +0.0 padding's one effect, the
// sign of a zero sum), and the count of the finite values.  rem: how many of
// the four values lie before the end (0..4 or more).
__device__ __forceinline__ uint32_t moments4_careful(uint32_t w0, uint32_t w1, uint32_t rem,
                                                     double& a01, double& q01) {
    const uint32_t wd[2] = {w0, w1};
    double v[4];
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t d = wd[i >> 1];
        const float f = __uint_as_float((i & 1) ? (d & 0xFFFF0000u) : (d << 16));
        const bool in = (uint32_t)i < rem, ok = in && __builtin_isfinite(f);
        v[i] = ok ? (double)f : (in ? 0.0 : -0.0);
        cnt += ok ? 1u : 0u;
    }
    a01 = (v[0] + v[1]) + (v[2] + v[3]);
    q01 = __builtin_fma(v[1], v[1], v[0] * v[0]) + __builtin_fma(v[3], v[3], v[2] * v[2]);
    return cnt;
}

// rem: values of the 8 before the data's end (32-bit group-local arithmetic).
__device__ __forceinline__ uint32_t moments8_careful(const u32x4 w, uint32_t rem, double& s1,
                                                     double& s2) {
    double a0, q0, a1, q1;
    uint32_t c = moments4_careful(w[0], w[1], rem, a0, q0);
    __builtin_amdgcn_sched_barrier(0);
    c += moments4_careful(w[2], w[3], rem > 4 ? rem - 4 : 0u, a1, q1);
    s1 = a0 + a1;
    s2 = q0 + q1;
    return c;
}

// Moments of one group (the wave's LDS area holds its 2048 values in index
// order at tslot units; lane l takes values 32l .. 32l + 31): per lane the
// 8-value trees of its four runs joined as (r0 + r1) + (r2 + r3), then the
// lane butterfly.  The runs are taken one after the other, each in two
// halves (scheduling barriers between them keep only four values' fp64
// temporaries live).  A full group without Inf or NaN values (careful =
// false, decided once per group) needs no count; otherwise the careful sums
// leave values past n and non-finite ones out (as +0.0) and count the
// others (for finite values within the data both give the same sums).
__device__ __forceinline__ void run_moments(const u32x4* area, uint32_t lane, uint32_t t,
                                            uint32_t valid, bool careful, double& r1, double& r2,
                                            uint32_t& cnt) {
    const u32x4 w = area[tslot(4 * lane + t)];
    uint32_t c = 8;
    if (!careful) {  // uniform
        moments8_full(w, r1, r2);
    } else {
        const uint32_t start = 32u * lane + 8u * t;  // the run's first value in the group
        c = moments8_careful(w, valid > start ? valid - start : 0u, r1, r2);
    }
    cnt += c;
    __builtin_amdgcn_sched_barrier(0);
}

// valid: the group's values before the data's end (2048 for a full group);
// special: the group holds an Inf or NaN.
__device__ __forceinline__ void group_moments(const u32x4* area, uint32_t lane, uint32_t valid,
                                              bool special, double& g1, double& g2, uint32_t& gn) {
    const bool careful = special || valid < kGroup;
    uint32_t cnt = 0;
    double a1, a2, b1, b2;
    run_moments(area, lane, 0, valid, careful, a1, a2, cnt);
    run_moments(area, lane, 1, valid, careful, b1, b2, cnt);
    const double h1 = a1 + b1, h2 = a2 + b2;
    run_moments(area, lane, 2, valid, careful, a1, a2, cnt);
    run_moments(area, lane, 3, valid, careful, b1, b2, cnt);
    g1 = wave_tree(h1 + (a1 + b1));
    g2 = wave_tree(h2 + (a2 + b2));
    gn = wave_sum(cnt);
}

// The window the first pass uses: the previous call's window recorded in the
// workspace, clamped to 1..248 (whatever the workspace held: it is only a
// prediction, checked by the window kernel).
__device__ __forceinline__ uint32_t predicted_L(uint32_t raw) {
    return raw < 1u ? 1u : (raw > 248u ? 248u : raw);
}

// One workgroup item: four waves, each with two consecutive groups of one
// segment (item list: one entry per wave pair of groups; each segment's list
// is padded to whole workgroups with entries of segment ~0, whose waves do
// no work), or eight waves with one group each (GW = 1, below), so the item
// covers 16,384 aligned values of one segment: one moment block, or
// several whole ones when the chunk is smaller.  Codes with window L; each
// group's escape count and each block's total; with MOMENTS, the blocks'
// moment partials: the tree needs each lane to hold 32 consecutive values,
// so once a group is coded its words are transposed through the wave's LDS
// area, and groups join pairwise into blocks.  A wave loads its second
// group once the first group's words are in LDS (with MOMENTS) or coded
// (without), so the two groups' words are never live together (80 VGPRs
// and 6 waves per SIMD with MOMENTS, 44 VGPRs without).
// LDS per wave: 4112 bytes, first a 32-byte exponent row per lane and the
// packed escapes (every value may escape), then the group's values for the
// transpose.  Every thread of the workgroup (256 or 512 threads) calls
// this (barriers).  L = 0: the predicted window, read once the item's loads are
// out (the first pass: its waves do not wait for the statistics before
// loading).
// LDS of one encoder workgroup item (the caller declares it, so kernels with
// several roles can overlay their roles' areas).
struct EncodeLds {
    u32x4 area[4][257];  // per wave, 4112 bytes
    double g1[8], g2[8];
    uint32_t gn[8], gc[8];
};

// The same for a workgroup of eight waves with one group each.
struct EncodeLds8 {
    u32x4 area[8][257];  // per wave, 4112 bytes
    double g1[8], g2[8];
    uint32_t gn[8], gc[8];
};

// AGAIN: a second coding of the item with another window (a failed
// prediction): the sign+mantissa bytes do not depend on the window and are
// already in place, so they are not written again.  GW: groups per wave,
// 2 (four waves, EncodeLds) or 1 (eight waves, EncodeLds8: the same item,
// each wave's chain one group long, for grids that fill less than one
// round of the chip).
template <bool MOMENTS, bool AGAIN = false, int GW = 2, typename Lds = EncodeLds>
__device__ __forceinline__ void encode_wg(const EncodeArgs& a, uint32_t wg, uint32_t L, Lds& lds) {
    auto& s_area = lds.area;
    auto& s_g1 = lds.g1;
    auto& s_g2 = lds.g2;
    auto& s_gn = lds.gn;
    auto& s_gc = lds.gc;
    const uint32_t lane = lane_id(), wave = wave_id();
    uint8_t* area = reinterpret_cast<uint8_t*>(s_area[wave]);
    u32x4* rowp = s_area[wave] + 2 * lane;  // the lane's exponent row
    uint8_t* ew = area + 2048;              // the wave's packed escapes
    const uint32_t* ew32 = reinterpret_cast<const uint32_t*>(ew);
    // the workgroup's first entry is live: its segment is the workgroup's
    const ItemDesc first = a.single ? ItemDesc{0u, 4 * wg} : a.pairs[wg * 4];
    const SegDesc sd = a.single ? a.seg0 : a.segs[first.seg];
    const uint32_t pw = GW == 2 ? wave : wave >> 1;  // the wave's entry in the item list
    const ItemDesc it = a.single ? ItemDesc{4 * wg + pw < (sd.g + 1) / 2 ? 0u : 0xFFFFFFFFu, 4 * wg + pw}
                                 : a.pairs[wg * 4 + pw];
    const uint64_t g0 = 2ull * it.local + (GW == 2 ? 0u : (wave & 1u));
    const bool live = it.seg != 0xFFFFFFFFu && g0 < sd.g;
    const uint32_t gi0 = GW == 2 ? 2 * wave : wave;  // the wave's first group in the item
    // group 0's words; group 1's are loaded once group 0's are in LDS (or
    // coded), so the two groups' words are never live together
    u32x4 w[2][4];
    if (live) load_group(a.in + sd.in_off, sd.n, g0, lane, w[0]);
    if (!L) L = predicted_L(a.stats[first.seg].L);
    // each group's moments and escape count go to LDS as soon as they are
    // known (lane 0); groups past the data keep -0.0 (the identity) and 0
    if (lane == 0) {
#pragma unroll
        for (int q = 0; q < GW; ++q) {
            s_gc[gi0 + q] = 0;
            if (MOMENTS) {
                s_g1[gi0 + q] = -0.0;
                s_g2[gi0 + q] = -0.0;
                s_gn[gi0 + q] = 0;
            }
        }
    }
    if (live) {
        uint8_t* __restrict__ st = a.out + sd.out_off;
        const uint32_t L7 = (L << 7) | (L << 23);
#pragma unroll
        for (int q = 0; q < GW; ++q) {
            const uint64_t g = g0 + q;
            if (g >= sd.g) break;  // uniform
            // coding first, with the words in registers; then (MOMENTS) the
            // words go to LDS for the moments' transpose
            uint32_t P[3], mx;
            u32x2 sm[4];
            encode_group(w[q], L7, P, sm, mx);
            // an Inf or NaN anywhere in the group (a half of mx at 0x7F80)
            const bool special = MOMENTS && __ballot(((mx + 0x00800080u) & 0x80008000u) != 0) != 0;
            if ((uint64_t)kGroup * (g + 1) > sd.n) {  // last, partial group: padding codes are 0
                const uint32_t V = valid_bits(lane, (uint32_t)(sd.n - (uint64_t)kGroup * g));
#pragma unroll
                for (int b = 0; b < 3; ++b) P[b] &= V;
            }
            uint8_t* cw = st + sd.code_off + 768ull * g + 4u * lane;
#pragma unroll
            for (int b = 0; b < 3; ++b) *reinterpret_cast<uint32_t*>(cw + 256 * b) = P[b];
            uint8_t* sw = st + sd.sm_off + 2048ull * g + 8u * lane;
            if (!AGAIN) {
#pragma unroll
                for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x2*>(sw + 512 * k) = sm[k];
            }
            const uint32_t M = P[0] & P[1] & P[2];
            uint32_t tot;
            const uint32_t excl = wave_prefix_small(__builtin_popcount(M), tot);
            const uint64_t gg = sd.group_base + g;
            if (lane == 0) {
                a.gcnt[gg] = tot;
                s_gc[gi0 + q] = tot;
            }
            uint32_t Q[8];
            exponent_bytes(w[q], Q);
            rowp[0] = u32x4{Q[0], Q[1], Q[2], Q[3]};
            rowp[1] = u32x4{Q[4], Q[5], Q[6], Q[7]};
            if (!MOMENTS && GW == 2 && q == 0 && g + 1 < sd.g) load_group(a.in + sd.in_off, sd.n, g + 1, lane, w[1]);
            const uint8_t* rb = reinterpret_cast<const uint8_t*>(rowp);
            for (uint32_t m = M, i = 0; m; m &= m - 1, ++i) ew[excl + i] = rb[__builtin_ctz(m)];
            __builtin_amdgcn_wave_barrier();  // the wave's packed bytes are complete
            uint32_t* slot = reinterpret_cast<uint32_t*>(a.staging + gg * kGroup);
            for (uint32_t k = lane; k < (tot + 3) / 4; k += 64) slot[k] = ew32[k];
            __builtin_amdgcn_wave_barrier();  // before the area is reused
            if (MOMENTS) {
#pragma unroll
                for (int k = 0; k < 4; ++k) s_area[wave][tslot(64 * k + lane)] = w[q][k];
                __builtin_amdgcn_wave_barrier();
                // group q + 1's loads now: the moments read the LDS copy, so
                // its words take the registers group q's words leave, and
                // the loads overlap the moments (80 VGPRs, 6 waves per SIMD:
                // 46.8 us against 47.6 for the pass at 64 VGPRs and 8 waves
                // with the loads after the moments)
                if (GW == 2 && q == 0 && g + 1 < sd.g) load_group(a.in + sd.in_off, sd.n, g + 1, lane, w[1]);
                const uint64_t left = sd.n - (uint64_t)kGroup * g;
                double m1, m2;
                uint32_t mn;
                group_moments(s_area[wave], lane, left < kGroup ? (uint32_t)left : kGroup, special,
                              m1, m2, mn);
                if (lane == 0) {
                    s_g1[gi0 + q] = m1;
                    s_g2[gi0 + q] = m2;
                    s_gn[gi0 + q] = mn;
                }
                __builtin_amdgcn_wave_barrier();  // before the next group reuses the area
            }
        }
    }
    // the workgroup's blocks (all four waves reach this)
    lds_barrier();
    const uint32_t per = a.block_elems / kGroup;  // groups per block: 1, 2, 4 or 8
    const uint32_t b = threadIdx.x;
    const uint32_t blk = (uint32_t)(2ull * first.local / per) + b;
    if (per == 8) {
        // one block per item (chunks of 16,384 values or more), the common
        // case: every LDS value read at once and the trees unrolled.  With
        // the loops below (trip count known only at run time) the reads
        // went one after another, and the workgroup's other waves waited
        // at the barrier meanwhile: 2 us of a workgroup's 11 us (pass
        // 47.0 -> 45.0 us for 67,108,864 values)
        if (b == 0 && blk < sd.nsb) {
            uint32_t c[8], nn[8];
            double t1[8], t2[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                c[i] = s_gc[i];
                if (MOMENTS) {
                    t1[i] = s_g1[i];
                    t2[i] = s_g2[i];
                    nn[i] = s_gn[i];
                }
            }
            a.part.esc[sd.sb_base + blk] = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
            if (MOMENTS) {
                const uint32_t slot = sd.sb_base + leaf_slot(blk, leaf_order(sd.nsb));
                a.part.s1[slot] = tree8(t1);
                a.part.s2[slot] = tree8(t2);
                a.part.n[slot] = ((nn[0] + nn[1]) + (nn[2] + nn[3])) + ((nn[4] + nn[5]) + (nn[6] + nn[7]));
            }
        }
    } else if (b < 8 / per && blk < sd.nsb) {
        uint32_t e = 0;
        for (uint32_t i = 0; i < per; ++i) e += s_gc[b * per + i];
        a.part.esc[sd.sb_base + blk] = e;
        if (MOMENTS) {
            double t1[8], t2[8];
            uint32_t n = 0;
            for (uint32_t i = 0; i < per; ++i) {
                t1[i] = s_g1[b * per + i];
                t2[i] = s_g2[b * per + i];
                n += s_gn[b * per + i];
            }
            for (uint32_t h = 1; h < per; h <<= 1)
                for (uint32_t i = 0; i < per; i += 2 * h) {
                    t1[i] = t1[i] + t1[i + h];
                    t2[i] = t2[i] + t2[i + h];
                }
            const uint32_t slot = sd.sb_base + leaf_slot(blk, leaf_order(sd.nsb));
            a.part.s1[slot] = t1[0];
            a.part.s2[slot] = t2[0];
            a.part.n[slot] = n;
        }
    }
    lds_barrier();  // s_g* are rewritten by the next workgroup item
}

// One group coded again with window L7 (packed as the encoder packs it):
// its code planes, escape count and staged escape exponents, as encode_wg
// writes them (the sign+mantissa bytes are the first pass's: they do not
// depend on the window).  rowp: the lane's 32-byte LDS row; ew: the wave's
// packed escape area (2048 + 16 bytes).
__device__ __forceinline__ void recode_group(const EncodeArgs& a, const SegDesc& sd, uint8_t* st, uint64_t g,
                                             const u32x4 (&w)[4], uint32_t L7, u32x4* rowp, uint8_t* ew,
                                             uint32_t lane) {
    uint32_t P[3], mx;
    u32x2 sm[4];
    encode_group(w, L7, P, sm, mx);
    if ((uint64_t)kGroup * (g + 1) > sd.n) {  // last, partial group: padding codes are 0
        const uint32_t V = valid_bits(lane, (uint32_t)(sd.n - (uint64_t)kGroup * g));
#pragma unroll
        for (int b = 0; b < 3; ++b) P[b] &= V;
    }
    uint8_t* cw = st + sd.code_off + 768ull * g + 4u * lane;
#pragma unroll
    for (int b = 0; b < 3; ++b) *reinterpret_cast<uint32_t*>(cw + 256 * b) = P[b];
    const uint32_t M = P[0] & P[1] & P[2];
    uint32_t tot;
    const uint32_t excl = wave_prefix_small(__builtin_popcount(M), tot);
    const uint64_t gg = sd.group_base + g;
    if (lane == 0) a.gcnt[gg] = tot;
    uint32_t Q[8];
    exponent_bytes(w, Q);
    rowp[0] = u32x4{Q[0], Q[1], Q[2], Q[3]};
    rowp[1] = u32x4{Q[4], Q[5], Q[6], Q[7]};
    const uint8_t* rb = reinterpret_cast<const uint8_t*>(rowp);
    for (uint32_t m = M, i = 0; m; m &= m - 1, ++i) ew[excl + i] = rb[__builtin_ctz(m)];
    __builtin_amdgcn_wave_barrier();  // the wave's packed bytes are complete
    const uint32_t* ew32 = reinterpret_cast<const uint32_t*>(ew);
    uint32_t* slot = reinterpret_cast<uint32_t*>(a.staging + gg * kGroup);
    for (uint32_t k = lane; k < (tot + 3) / 4; k += 64) slot[k] = ew32[k];
    __builtin_amdgcn_wave_barrier();  // before the area is reused
}

// A chunk's ng groups (from segment group gc0) coded again with window L
// after a failed prediction: code planes, escape counts and staged escape
// exponents (no moments: the window is known; no per-block counts: nothing
// reads them after a miss).  Wave w codes groups w, w + 4, ...; the next
// group's words are requested before the current one is coded.  Every
// thread of the 256-thread workgroup calls this.
__device__ __forceinline__ void recode_chunk(const EncodeArgs& a, const SegDesc& sd, uint64_t gc0, uint32_t ng,
                                             uint32_t L, EncodeLds& lds) {
    const uint32_t lane = lane_id(), wave = wave_id();
    u32x4* rowp = lds.area[wave] + 2 * lane;
    uint8_t* ew = reinterpret_cast<uint8_t*>(lds.area[wave]) + 2048;
    const uint16_t* in = a.in + sd.in_off;
    uint8_t* st = a.out + sd.out_off;
    const uint32_t L7 = (L << 7) | (L << 23);
    u32x4 wa[4], wb[4];
    if (wave < ng) load_group(in, sd.n, gc0 + wave, lane, wa);
    for (uint32_t j = wave; j < ng; j += 8) {  // (uniform)
        if (j + 4 < ng) load_group(in, sd.n, gc0 + j + 4, lane, wb);
        recode_group(a, sd, st, gc0 + j, wa, L7, rowp, ew, lane);
        if (j + 8 < ng) load_group(in, sd.n, gc0 + j + 8, lane, wa);
        if (j + 4 < ng) recode_group(a, sd, st, gc0 + j + 4, wb, L7, rowp, ew, lane);
    }
}

}  // namespace zc
