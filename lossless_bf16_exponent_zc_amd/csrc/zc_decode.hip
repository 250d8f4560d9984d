// zc_decode.hip -- decompress, and decompress fused with a fixed-order sum.
//
// Decoding inverts the exponent coding of the ZipCCL scribe notes ("Key idea
// and contribution", technique 1): e = L + code for codes 0..6, the next
// escape byte for code 7, sign and mantissa from the raw byte.  The fused
// variant is the receive side of a compressed reduce-scatter (technique 3
// names the reduce-scatter path; the UCCL-Zip page's abstract argues for
// fusing the codec into the collective to drop extra memory traffic): each
// shard's group is decoded into registers and added in shard order in fp32,
// so the only global write is the final BF16 sum.
//
// One wave per 2048-value group.  The chunk table and the group table give
// the group's first escape directly, so groups decode independently.  The
// plane words and sign+mantissa bytes are requested before the header is
// checked (their offsets follow from the plan alone), the escape bytes as
// soon as the tables arrive, so a group costs two memory round trips.
// Values are rebuilt with packed ops, staged in LDS, and each lane patches
// its escaped values.  Every stream's header, tables, counts and padding are
// checked; a group that fails writes nothing.
#include "zc_kernels.h"

namespace zc {

namespace {

constexpr uint32_t kBadMagic = 0x01, kBadWindow = 0x02, kBadShape = 0x04, kBadSize = 0x08,
                   kBadTable = 0x10, kBadCount = 0x20, kBadPad = 0x40;
// check_header's answer for a valid raw stream (no rejection bit: never stored)
constexpr uint32_t kRawStream = 0x100;

template <typename T>
__device__ __forceinline__ T ld(const uint8_t* p) {
    return *reinterpret_cast<const T*>(p);
}

// The 64-byte header, read as one block (one scalar load: every field
// arrives in one round trip) and checked with bitwise ORs, so no check waits
// for another.
struct HeaderWords {
    uint32_t w[16];
};

__device__ __forceinline__ uint64_t hword64(const HeaderWords& h, int i) {
    return (uint64_t)h.w[i] | ((uint64_t)h.w[i + 1] << 32);
}

// 0 for a valid coded header, kRawStream for a valid raw one (flags 1: L 0,
// E 0, total 64 + 2N, offsets 0), else the rejection bits.  h: the header's
// words, read whether or not the buffer holds them (hdr_ok: it does).
// E and L receive the header's escape count and window (0 without a header).
// FLAT: both verdicts without branches, so every header word is needed at
// once (the fused reduce); otherwise the raw verdict is a branch (fewer
// registers: the plain decoder runs at 64).
template <bool FLAT>
__device__ __forceinline__ uint32_t check_header(const HeaderWords& h, bool hdr_ok, uint64_t cap,
                                                 const SegDesc& sd, uint32_t C, uint64_t& E,
                                                 uint32_t& L) {
    const uint32_t w1 = h.w[1], flags = w1 >> 24;
    L = hdr_ok ? (w1 >> 16) & 0xFFu : 0u;
    E = hdr_ok ? hword64(h, 6) : 0u;
    if (!hdr_ok) return kBadSize;
    const uint64_t N = hword64(h, 2), total = hword64(h, 8);
    const uint64_t o40 = hword64(h, 10), o48 = hword64(h, 12), o56 = hword64(h, 14);
    const bool id_ok = (h.w[0] == kMagic) & ((w1 & 0xFFFFu) == kVersion);
    const bool dims_ok = (N == sd.n) & (h.w[4] == C) & (h.w[5] == sd.k);
    const uint64_t raw_total = kHeaderBytes + 2ull * sd.n;
    if (!FLAT && flags == kFlagRaw) {
        uint32_t bad = id_ok ? 0u : kBadMagic;
        bad |= L != 0 ? kBadWindow : 0u;
        bad |= (dims_ok & ((o40 | o48 | o56) == 0)) ? 0u : kBadShape;
        bad |= ((E == 0) & (total == raw_total) & (raw_total <= cap)) ? 0u : kBadSize;
        return bad ? bad : kRawStream;
    }
    uint32_t raw_bad = id_ok ? 0u : kBadMagic;
    raw_bad |= L != 0 ? kBadWindow : 0u;
    raw_bad |= (dims_ok & ((o40 | o48 | o56) == 0)) ? 0u : kBadShape;
    raw_bad |= ((E == 0) & (total == raw_total) & (raw_total <= cap)) ? 0u : kBadSize;
    uint32_t bad = (id_ok & (flags == 0)) ? 0u : kBadMagic;
    bad |= ((L >= 1) & (L <= 248)) ? 0u : kBadWindow;
    bad |= (dims_ok & (o40 == sd.code_off) & (o48 == sd.sm_off) & (o56 == sd.esc_off)) ? 0u : kBadShape;
    bad |= ((E <= sd.n) & (total == sd.esc_off + E) & (total <= cap)) ? 0u : kBadSize;
    return flags == kFlagRaw ? (raw_bad ? raw_bad : kRawStream) : bad;
}

// Nibble words of tile k: nibble n of Z[k] = code of the value at plane bit
// 4n + k.
__device__ __forceinline__ void code_nibbles(const uint32_t (&P)[3], uint32_t (&Z)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
        Z[k] = ((P[0] >> k) & 0x11111111u) | (((P[1] >> k) & 0x11111111u) << 1) |
               (((P[2] >> k) & 0x11111111u) << 2);
}

// Exponent bytes in plane-bit order: byte k of Q[n] = L + code of the value
// at plane bit 4n + k (byte j of Z[k] holds nibbles 2j and 2j+1; codes <= 7
// and L <= 248, so the bytewise add never carries).
__device__ __forceinline__ void exponent_rows(const uint32_t (&Z)[4], uint32_t L, uint32_t (&Q)[8]) {
    const uint32_t LL = L * 0x01010101u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t T = perm(Z[1], Z[0], 0x0C0C0400u | (j << 8) | j) |
                           perm(Z[3], Z[2], 0x04000C0Cu | (j << 24) | (j << 16));
        Q[2 * j] = (T & 0x0F0F0F0Fu) + LL;
        Q[2 * j + 1] = ((T >> 4) & 0x0F0F0F0Fu) + LL;
    }
}

// BF16 words from exponent bytes (plane-bit order) and sign+mantissa bytes.
// Word m of tile k holds the values at plane bits 4m + k (low half) and
// 4(m+4) + k (high half).
__device__ __forceinline__ void assemble(const uint32_t (&Q)[8], const u32x2 (&sm)[4], u32x4 (&o)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = sm[k].x, hi = sm[k].y;
        // exponent of the low value to bits 7-14, of the high one to bits 23-30
        const uint32_t sel = 0x0C000C00u | ((4u + k) << 16) | (uint32_t)k;
        const uint32_t e0 = perm(Q[4], Q[0], sel) << 7, e1 = perm(Q[5], Q[1], sel) << 7;
        const uint32_t e2 = perm(Q[6], Q[2], sel) << 7, e3 = perm(Q[7], Q[3], sel) << 7;
        // sign+mantissa bytes of values 2m, 2m, 2m+1, 2m+1 -> bits 0-6 and 15 of each half
        o[k][0] = bitsel(0x7F807F80u, e0, perm(hi, lo, 0x01010000u));
        o[k][1] = bitsel(0x7F807F80u, e1, perm(hi, lo, 0x03030202u));
        o[k][2] = bitsel(0x7F807F80u, e2, perm(hi, lo, 0x05050404u));
        o[k][3] = bitsel(0x7F807F80u, e3, perm(hi, lo, 0x07070606u));
    }
}

// BF16 round to nearest even, two values at once (low half: lo), by the
// hardware's packed conversion (denormals kept, as this library is built);
// every NaN becomes the canonical 0x7FC0: it is made the quiet NaN with no
// payload first, which converts to 0x7FC0.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t to_bf16x2(float lo, float hi) {
    const float qnan = __uint_as_float(0x7FC00000u);
    const f32x2 v = {lo != lo ? qnan : lo, hi != hi ? qnan : hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Bytes of the lane's tile-k sm words that lie past the end (must be zero).
__device__ __forceinline__ uint64_t sm_pad_mask(uint32_t lane, uint32_t valid, int k) {
    const int64_t left = (int64_t)valid - (int64_t)(512u * k + 8u * lane);
    if (left >= 8) return 0;
    if (left <= 0) return ~0ull;
    return ~0ull << (8 * left);
}

template <bool TAIL>
__device__ __forceinline__ void store_values(uint16_t* __restrict__ out, uint64_t n, uint64_t g,
                                             uint32_t lane, const u32x4 (&o)[4]) {
    const uint64_t base = (uint64_t)kGroup * g + 8u * lane;
    if (!TAIL) {
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(out + base + 512u * k) = o[k];
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t b = base + 512u * k;
        if (b + 8 <= n) {
            *reinterpret_cast<u32x4*>(out + b) = o[k];
        } else {
            for (uint32_t j = 0; j < 8; ++j)
                if (b + j < n) out[b + j] = (uint16_t)(o[k][j >> 1] >> (16 * (j & 1)));
        }
    }
}

// The lane's four 8-value words of group g of a raw stream (the values
// after the header, 64 + 2N bytes checked to be in the buffer); word k holds
// values 2048 g + 512 k + 8 lane .. + 7, zeros past N.
template <bool TAIL>
__device__ __forceinline__ void raw_words(const uint8_t* st, uint64_t n, uint64_t g, uint32_t lane,
                                          u32x4 (&o)[4]) {
    const uint8_t* src = st + kHeaderBytes + 2ull * ((uint64_t)kGroup * g + 8u * lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t b = (uint64_t)kGroup * g + 512u * k + 8u * lane;
        if (!TAIL || b + 8 <= n) {
            o[k] = ld<u32x4>(src + 1024 * k);
        } else {
            o[k] = u32x4{0, 0, 0, 0};
#pragma unroll
            for (uint32_t j = 0; j < 8; ++j)
                if (b + j < n) o[k][j >> 1] |= (uint32_t)ld<uint16_t>(src + 1024 * k + 2 * j) << (16 * (j & 1));
        }
    }
}

// Everything one wave reads of one stream for one group.
struct GroupData {
    uint32_t P[3];
    u32x2 sm[4];
    uint32_t bad, L, t0, rel, span;
};

// Issue the loads of group g of stream st (cap readable bytes): the header
// and (EARLY) the table words first, then the plane words and sm bytes, all
// in one round with no branch between them, so the checks wait only for
// the header and tables.  Every load is unconditional: where the buffer
// does not hold a region, the load reads `dummy` (at least 2048 readable
// bytes) instead and the value is never used (a buffer without its fixed
// regions fails the size check; a raw stream reads its words elsewhere).
// EARLY = false (the reduce that walks the shards in turn, which holds a
// second stream's loads meanwhile): the table words are read after the
// header check, to stay within its registers.  FLAT (the fused reduce,
// which reads S streams for every value it writes): the plane and sign+
// mantissa words are non-temporal loads (8 x 32M shards: 95.7 -> 94.0 us;
// the plain decoder, one stream in and one out, is faster without).
template <bool EARLY, bool FLAT>
__device__ __forceinline__ void fetch(const uint8_t* st, uint64_t cap, const SegDesc& sd,
                                      uint32_t C, uint32_t g, uint32_t lane, const uint8_t* dummy,
                                      GroupData& d) {
    const bool hdr_ok = cap >= kHeaderBytes;
    const bool fixed_ok = cap >= sd.esc_off;  // (implies hdr_ok)
    const HeaderWords h = *reinterpret_cast<const HeaderWords*>(hdr_ok ? st : dummy);
    // C is a power of two >= 2048: chunk k = g >> (log2 C - 11)
    const uint32_t gpc = C / kGroup, k = g >> (__builtin_ctz(C) - 11);
    const bool last_in_chunk = ((g + 1) & (gpc - 1)) == 0 || g + 1 == sd.g;
    const uint8_t* fb = fixed_ok ? st : dummy;  // the fixed regions, or the stand-in
    uint32_t t0 = 0, t1 = 0, rel = 0, rel1 = 0, gw0 = 0, gw1 = 0;
    if (EARLY) {
        // table entries k, k + 1 (scalar loads) and group-table entries g,
        // g + 1; everything read here lies before esc_off (past the last
        // entry: padding or the code region).  FLAT (the fused reduce, whose
        // workgroup reads one group of each shard): the two aligned dwords
        // that hold the entries (gtab_off is a multiple of 4), by scalar
        // loads.  Otherwise 16-bit vector loads issued before the data
        // words': with many segments, scalar loads of every segment's group
        // table crowd the scalar cache.
        const uint32_t* tw = reinterpret_cast<const uint32_t*>(fb + (fixed_ok ? kHeaderBytes + 4ull * k : 0));
        t0 = tw[0];
        t1 = tw[1];
        if (FLAT) {
            const uint32_t* gw = reinterpret_cast<const uint32_t*>(fb + (fixed_ok ? (sd.gtab_off + 2ull * g) & ~3ull : 0));
            gw0 = gw[0];
            gw1 = gw[1];
        } else {
            const uint16_t* gh = reinterpret_cast<const uint16_t*>(fb + (fixed_ok ? sd.gtab_off + 2ull * g : 0));
            gw0 = gh[0];
            gw1 = gh[1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // the data words' loads after the header's and tables'
    const uint8_t* cw = fb + (fixed_ok ? sd.code_off + 768ull * g : 0) + 4u * lane;
    const uint8_t* sw = fb + (fixed_ok ? sd.sm_off + 2048ull * g : 0) + 8u * lane;
#pragma unroll
    for (int b = 0; b < 3; ++b)
        d.P[b] = FLAT ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(cw + 256 * b))
                      : ld<uint32_t>(cw + 256 * b);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        d.sm[q] = FLAT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sw + 512 * q))
                       : ld<u32x2>(sw + 512 * q);
    // every header and table word is needed here, after all the loads are
    // issued: the compiler may not sink any of them behind a check (the
    // scalar loads then all go out in the first round)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"s"(h.w[0]), "s"(h.w[1]), "s"(h.w[2]), "s"(h.w[3]), "s"(h.w[4]), "s"(h.w[5]),
                 "s"(h.w[6]), "s"(h.w[7]), "s"(h.w[8]), "s"(h.w[9]), "s"(h.w[10]), "s"(h.w[11]),
                 "s"(h.w[12]), "s"(h.w[13]), "s"(h.w[14]), "s"(h.w[15]), "s"(t0), "s"(t1));
    if (EARLY && FLAT) {
        asm volatile("" ::"s"(gw0), "s"(gw1));
        const uint64_t gq = (uint64_t)gw0 | ((uint64_t)gw1 << 32);
        const uint32_t sh = fixed_ok ? 16u * (g & 1u) : 0u;
        rel = (uint32_t)(gq >> sh) & 0xFFFFu;
        rel1 = last_in_chunk ? rel : (uint32_t)(gq >> (sh + 16)) & 0xFFFFu;
    } else if (EARLY) {
        rel = gw0;
        rel1 = last_in_chunk ? rel : gw1;
    }

    uint64_t E;
    uint32_t L;
    uint32_t bad = check_header<FLAT>(h, hdr_ok, cap, sd, C, E, L);
    if (!EARLY && !bad) {
        const uint32_t* table = reinterpret_cast<const uint32_t*>(st + kHeaderBytes);
        const uint16_t* gtab = reinterpret_cast<const uint16_t*>(st + sd.gtab_off);
        t0 = table[k];
        t1 = table[k + 1];
        rel = gtab[g];
        rel1 = gtab[last_in_chunk ? g : g + 1];
    }
    // table and count checks, computed whatever the header said (no branch:
    // the table loads stay with the others), applied to a valid header only
    const uint32_t next = last_in_chunk ? t1 - t0 : rel1;
    const bool tbad = (t0 > t1) | (t1 > E) | ((k == 0) & (t0 != 0)) | ((k + 1 == sd.k) & (t1 != E)) |
                      (((g & (gpc - 1)) == 0) & (rel != 0));
    // a group holds at most kGroup escapes: a larger span (a damaged group
    // table) is rejected here, before fetch_escapes writes the span into the
    // wave's fixed LDS area (520 dwords)
    const bool cbad = (rel > next) | (next > t1 - t0) | (next - rel > kGroup);
    if (!bad) bad = tbad ? kBadTable : (cbad ? kBadCount : 0u);
    d.bad = bad;
    const bool use = bad == 0;
    d.L = use ? L : 0u;
    d.t0 = use ? t0 : 0u;
    d.rel = use ? rel : 0u;
    d.span = use ? next - rel : 0u;
}

// Copy the group's `span` escape bytes (starting at stream byte `at`) into
// LDS as whole dwords; returns the offset of the first byte in `dst`.
__device__ __forceinline__ uint32_t fetch_escapes(const uint8_t* st, uint64_t cap, uint64_t at,
                                                  uint32_t span, uint32_t lane, uint32_t* dst) {
    const uint64_t a0 = at & ~3ull;
    const uint32_t ndw = (uint32_t)((at + span + 3 - a0) >> 2);
    for (uint32_t i = lane; i < ndw; i += 64) {
        const uint64_t o = a0 + 4ull * i;
        uint32_t v;
        if (o + 4 <= cap) {
            v = ld<uint32_t>(st + o);
        } else {
            v = 0;
            for (uint32_t b = 0; b < 4; ++b)
                if (o + b < cap) v |= (uint32_t)st[o + b] << (8 * b);
        }
        dst[i] = v;
    }
    return (uint32_t)(at - a0);
}

// Rebuild the group's values into o.  The lane's exponent bytes go to its
// 32-byte LDS row in plane-bit order; each escape overwrites its byte there
// with the next escape byte (the lane's escapes are contiguous from `first`
// in `esc`, a 4-byte aligned LDS area with at least 20 readable bytes past
// the group's last escape).  REG, for a group with more than two escapes
// per lane on average: the first 16 escape bytes come from five dwords read
// at once and funnel-shifted to the run, so the patch loop does not wait on
// LDS per byte (a lane with more takes the rest byte by byte).  With fewer
// escapes the unrolled steps cost more than the waits they save, and the
// fused reduce, bound by instruction issue, always reads byte by byte.
template <bool REG>
__device__ __forceinline__ void rebuild(const GroupData& d, uint32_t M, uint32_t first,
                                        const uint8_t* esc, u32x4* row, u32x4 (&o)[4]) {
    __builtin_amdgcn_wave_barrier();  // the escape bytes are in LDS
    uint32_t Z[4], Q[8];
    code_nibbles(d.P, Z);
    exponent_rows(Z, d.L, Q);
    row[0] = u32x4{Q[0], Q[1], Q[2], Q[3]};
    row[1] = u32x4{Q[4], Q[5], Q[6], Q[7]};
    uint8_t* rb = reinterpret_cast<uint8_t*>(row);
    if (REG && d.span > 128) {  // uniform
      if (M) {
        const uint32_t* e32 = reinterpret_cast<const uint32_t*>(esc) + (first >> 2);
        const uint32_t sh = first & 3u;
        uint32_t e[5], f[4];
#pragma unroll
        for (int j = 0; j < 5; ++j) e[j] = e32[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __builtin_amdgcn_alignbyte(e[j + 1], e[j], sh);
        uint32_t m = M;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (m) {
                rb[__builtin_ctz(m)] = (uint8_t)(f[k >> 2] >> (8 * (k & 3)));
                m &= m - 1;
            }
        }
        for (uint32_t i = first + 16; m; m &= m - 1, ++i) rb[__builtin_ctz(m)] = esc[i];
      }
    } else {
        for (uint32_t m = M, i = first; m; m &= m - 1, ++i) rb[__builtin_ctz(m)] = esc[i];
    }
    const u32x4 r0 = row[0], r1 = row[1];
    const uint32_t Qe[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    assemble(Qe, d.sm, o);
    __builtin_amdgcn_wave_barrier();
}

}  // namespace

// One group of every stream: decode (REDUCE: and sum in shard order).  TAIL
// is the segment's last, partial group: padding checks and partial stores.
template <bool REDUCE, bool TAIL>
__device__ __forceinline__ uint32_t decode_group_all(const DecodeArgs& a, const SegDesc& sd, uint32_t g,
                                                     uint32_t lane, uint32_t* esc_lds, u32x4* row) {
    const uint32_t valid = TAIL ? (uint32_t)(sd.n - (uint64_t)kGroup * g) : kGroup;
    const uint8_t* escb = reinterpret_cast<const uint8_t*>(esc_lds);
    float acc[REDUCE ? 32 : 1];
    uint32_t bad_all = 0;

    auto stream_of = [&](uint32_t s, uint64_t& cap) -> const uint8_t* {
        if (REDUCE) {
            cap = a.capacity;
            return a.in[s];
        }
        cap = a.capacity > sd.out_off ? a.capacity - sd.out_off : 0;
        if (cap > sd.max_bytes) cap = sd.max_bytes;
        return a.in[0] + sd.out_off;
    };

    uint64_t cap;
    const uint8_t* st = stream_of(0, cap);
    GroupData cur;
    fetch<!REDUCE, false>(st, cap, sd, a.chunk_elems, g, lane, a.dummy, cur);
    if (!REDUCE && cur.bad == kRawStream) {  // uniform: a raw stream, its words as they are
        u32x4 o[4];
        raw_words<TAIL>(st, sd.n, g, lane, o);
        store_values<TAIL>(a.out + sd.in_off, sd.n, g, lane, o);
        return 0;
    }
    for (uint32_t s = 0; s < a.nstreams; ++s) {
        // escape bytes of this stream, then the next stream's loads
        uint32_t first = 0;
        if (!cur.bad) first = fetch_escapes(st, cap, sd.esc_off + cur.t0 + cur.rel, cur.span, lane, esc_lds);
        GroupData nxt;
        uint64_t ncap = 0;
        const uint8_t* nst = nullptr;
        if (REDUCE && s + 1 < a.nstreams) {
            nst = stream_of(s + 1, ncap);
            fetch<!REDUCE, false>(nst, ncap, sd, a.chunk_elems, g, lane, a.dummy, nxt);
        }

        // (raw shards of the sum join the decoded ones before the adds)
        uint32_t bad = cur.bad;
        u32x4 o[4];
        bool have = false;
        if (REDUCE && bad == kRawStream) {  // uniform
            bad = 0;
            raw_words<TAIL>(st, sd.n, g, lane, o);
            have = true;
        } else if (!bad) {
            if (TAIL) {
                const uint32_t V = valid_bits(lane, valid);
                bool padbad = ((cur.P[0] | cur.P[1] | cur.P[2]) & ~V) != 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    padbad |= (__builtin_bit_cast(uint64_t, cur.sm[k]) & sm_pad_mask(lane, valid, k)) != 0;
                if (__ballot(padbad)) bad |= kBadPad;
            }
            const uint32_t M = cur.P[0] & cur.P[1] & cur.P[2];
            const uint32_t cnt = __builtin_popcount(M);
            const uint32_t incl = wave_inclusive_scan(cnt);
            if (readlane(incl, 63) != cur.span) bad |= kBadCount;
            if (!bad) {
                rebuild<!REDUCE>(cur, M, first + incl - cnt, escb, row, o);
                if (REDUCE) have = true;
                else store_values<TAIL>(a.out + sd.in_off, sd.n, g, lane, o);
            }
        }
        if (REDUCE && have) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const float lo = __uint_as_float(o[k][mm] << 16);
                    const float hi = __uint_as_float(o[k][mm] & 0xFFFF0000u);
                    float& a0 = acc[REDUCE ? 8 * k + 2 * mm : 0];
                    float& a1 = acc[REDUCE ? 8 * k + 2 * mm + 1 : 0];
                    a0 = s == 0 ? lo : a0 + lo;
                    a1 = s == 0 ? hi : a1 + hi;
                }
        }
        bad_all |= bad;
        if (REDUCE && s + 1 < a.nstreams) {
            cur = nxt;
            st = nst;
            cap = ncap;
        }
    }

    if (REDUCE && bad_all == 0 && a.nstreams > 0) {
        u32x4 o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
                o[k][mm] = to_bf16x2(acc[REDUCE ? 8 * k + 2 * mm : 0], acc[REDUCE ? 8 * k + 2 * mm + 1 : 0]);
        store_values<TAIL>(a.out + sd.in_off, sd.n, g, lane, o);
    }
    return bad_all;
}

template <bool REDUCE, bool SINGLE>
__device__ __forceinline__ void decode_kernel(const DecodeArgs& a) {
    __shared__ u32x4 s_row[4][64][2];   // per wave and lane: 32 exponent bytes
    __shared__ uint32_t s_esc[4][520];  // the group's escape bytes per wave (whole dwords)

    const uint32_t lane = lane_id(), wave = wave_id();
    const uint32_t gg = blockIdx.x * 4 + wave;
    if (gg >= a.ngroups) return;
    // (the fused reduce takes the descriptor from memory: the argument copy
    // costs it registers it does not have)
    // (a compile-time choice: selecting between the argument copy and the
    // table at run time would read the descriptor through vector loads)
    const ItemDesc gd = SINGLE ? ItemDesc{0u, gg} : a.groups[gg];
    const SegDesc sd = SINGLE ? a.seg0 : a.segs[gd.seg];
    const uint32_t g = gd.local;
    const uint32_t bad = (uint64_t)kGroup * (g + 1) > sd.n
                             ? decode_group_all<REDUCE, true>(a, sd, g, lane, s_esc[wave], s_row[wave][lane])
                             : decode_group_all<REDUCE, false>(a, sd, g, lane, s_esc[wave], s_row[wave][lane]);
    if (lane == 0) a.status[gg] = bad;
}

// One stream's group for the one-wave-per-shard reduce: decode into o (the
// lane's four words: tile k at word 64k + lane), returns the rejection bits.
// Decode one stream's group g into the wave's LDS area `vals` (word
// 64 k + lane: the lane's tile-k word); the area's first 4128 bytes hold
// the rows and escape bytes meanwhile (the wave reads them all before it
// writes a value: LDS operations of a wave run in order).  Returns the
// rejection bits (nothing written when non-zero).  The values are stored
// here, not returned, so no register copy of them outlives a branch.
template <bool TAIL>
__device__ __forceinline__ uint32_t decode_one(const uint8_t* st, uint64_t cap, const SegDesc& sd,
                                               uint32_t C, uint32_t g, uint32_t lane, const uint8_t* dummy,
                                               u32x4* vals) {
    uint32_t* esc_lds = reinterpret_cast<uint32_t*>(vals + 128);
    u32x4* row = vals + 2 * lane;
    GroupData d;
    fetch<true, true>(st, cap, sd, C, g, lane, dummy, d);
    if (d.bad == kRawStream) {  // uniform
        u32x4 o[4];
        raw_words<TAIL>(st, sd.n, g, lane, o);
#pragma unroll
        for (int k = 0; k < 4; ++k) vals[64 * k + lane] = o[k];
        return 0;
    }
    uint32_t first = 0;
    if (!d.bad) first = fetch_escapes(st, cap, sd.esc_off + d.t0 + d.rel, d.span, lane, esc_lds);
    uint32_t bad = d.bad;
    if (bad) return bad;
    if (TAIL) {
        const uint32_t valid = (uint32_t)(sd.n - (uint64_t)kGroup * g);
        const uint32_t V = valid_bits(lane, valid);
        bool padbad = ((d.P[0] | d.P[1] | d.P[2]) & ~V) != 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            padbad |= (__builtin_bit_cast(uint64_t, d.sm[k]) & sm_pad_mask(lane, valid, k)) != 0;
        if (__ballot(padbad)) bad |= kBadPad;
    }
    const uint32_t M = d.P[0] & d.P[1] & d.P[2];
    const uint32_t cnt = __builtin_popcount(M);
    const uint32_t incl = wave_inclusive_scan(cnt);
    if (readlane(incl, 63) != d.span) bad |= kBadCount;
    if (!bad) {
        u32x4 o[4];
        rebuild<false>(d, M, first + incl - cnt, reinterpret_cast<const uint8_t*>(esc_lds), row, o);
#pragma unroll
        for (int k = 0; k < 4; ++k) vals[64 * k + lane] = o[k];
    }
    return bad;
}

// OR of the 8 bytes of w.
__device__ __forceinline__ uint32_t or_bytes(uint64_t w) {
    const uint32_t x = (uint32_t)w | (uint32_t)(w >> 32);
    return (x | (x >> 8) | (x >> 16) | (x >> 24)) & 0xFFu;
}

// Output half-word i (values 512 (i / 128) + 8 ((i / 2) % 64) + 4 (i % 2)
// .. + 3 of group g: the half of area word i / 2).
template <bool TAIL>
__device__ __forceinline__ void store_half_word(uint16_t* __restrict__ out, uint64_t n, uint64_t g,
                                                uint32_t i, const u32x2 w) {
    const uint32_t wd = i >> 1;
    const uint64_t b = (uint64_t)kGroup * g + 512u * (wd >> 6) + 8u * (wd & 63u) + 4u * (i & 1u);
    if (!TAIL || b + 4 <= n) {
        *reinterpret_cast<u32x2*>(out + b) = w;
        return;
    }
    for (uint32_t j = 0; j < 4; ++j)
        if (b + j < n) out[b + j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
}

// Decompress-reduce with one wave per shard (up to 8 shards): wave s decodes
// shard s's group into its LDS area (the area first holds its exponent rows
// and escape bytes), then the workgroup sums the shards' values word by
// word in shard order, in fp32, and rounds to BF16.  Every shard's loads are
// in flight at once; a group costs two memory round trips.
template <int S, bool TAIL>
__device__ __forceinline__ void reduce_group_wide(const DecodeArgs& a, const SegDesc& sd, uint32_t g,
                                                  uint32_t gg, u32x4 (*s_area)[258], uint8_t* s_bad) {
    const uint32_t lane = lane_id(), wave = wave_id();
    const uint32_t bad = decode_one<TAIL>(a.in[wave], a.capacity, sd, a.chunk_elems, g, lane, a.dummy,
                                          s_area[wave]);
    // one byte per wave (rejection bits fit in 7), read back as one word;
    // the bytes of waves past S are masked off
    if (lane == 0) s_bad[wave] = (uint8_t)bad;
    __syncthreads();
    const uint64_t bytes = *reinterpret_cast<const uint64_t*>(s_bad);
    const uint32_t bad_all = or_bytes(S == 8 ? bytes : bytes & ((1ull << (8 * (S & 7))) - 1));
    if (bad_all == 0) {
        // every thread takes 4 values (half an area word), so all S waves
        // share the sum
#pragma unroll
        for (uint32_t i = threadIdx.x; i < 512; i += 64 * S) {
            float acc[4];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const u32x2 v = reinterpret_cast<const u32x2*>(s_area[s])[i];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const float lo = __uint_as_float(v[m] << 16), hi = __uint_as_float(v[m] & 0xFFFF0000u);
                    acc[2 * m] = s == 0 ? lo : acc[2 * m] + lo;
                    acc[2 * m + 1] = s == 0 ? hi : acc[2 * m + 1] + hi;
                }
            }
            u32x2 w;
#pragma unroll
            for (int m = 0; m < 2; ++m) w[m] = to_bf16x2(acc[2 * m], acc[2 * m + 1]);
            store_half_word<TAIL>(a.out + sd.in_off, sd.n, g, i, w);
        }
    }
    if (threadIdx.x == 0) a.status[gg] = bad_all;
}

template <int S>
__global__ __launch_bounds__(512) void zc_decode_reduce_wide(DecodeArgs a) {
    __shared__ u32x4 s_area[8][258];  // per wave: rows (2048 B) + escapes (2080 B); then values
    __shared__ __align__(8) uint8_t s_bad[8];
    const uint32_t gg = blockIdx.x;
    const SegDesc& sd = a.seg0;  // a reduce plan has one segment
    const uint32_t g = gg;
    if ((uint64_t)kGroup * (g + 1) > sd.n)
        reduce_group_wide<S, true>(a, sd, g, gg, s_area, s_bad);
    else
        reduce_group_wide<S, false>(a, sd, g, gg, s_area, s_bad);
}

template __global__ void zc_decode_reduce_wide<1>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<2>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<3>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<4>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<5>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<6>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<7>(DecodeArgs);
template __global__ void zc_decode_reduce_wide<8>(DecodeArgs);

// The native (uncompressed) reduce-scatter receive: S BF16 shards summed in
// fp32 in shard order and rounded as the fused reduce rounds, so the two
// paths give the same bits.  Each thread takes one 16-byte word (8 values)
// of every shard per step, all S loads in flight at once; the last n % 8
// values are summed one by one by the first threads of workgroup 0.
template <int S>
__global__ __launch_bounds__(256) void zc_reduce_native(NativeReduceArgs a) {
    const uint64_t words = a.n / 8;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words; w += step) {
        u32x4 v[S];
#pragma unroll
        for (int s = 0; s < S; ++s)  // non-temporal: read once (8 x 32M: 117 -> 109 us)
            v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.in[s]) + w);
        float acc[8];
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float lo = __uint_as_float(v[s][m] << 16), hi = __uint_as_float(v[s][m] & 0xFFFF0000u);
                acc[2 * m] = s == 0 ? lo : acc[2 * m] + lo;
                acc[2 * m + 1] = s == 0 ? hi : acc[2 * m + 1] + hi;
            }
        u32x4 o;
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = to_bf16x2(acc[2 * m], acc[2 * m + 1]);
        reinterpret_cast<u32x4*>(a.out)[w] = o;
    }
    const uint64_t i = 8 * words + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < 8 && i < a.n) {
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float x = __uint_as_float((uint32_t)a.in[s][i] << 16);
            acc = s == 0 ? x : acc + x;
        }
        a.out[i] = (uint16_t)to_bf16x2(acc, 0.f);
    }
}

template __global__ void zc_reduce_native<1>(NativeReduceArgs);
template __global__ void zc_reduce_native<2>(NativeReduceArgs);
template __global__ void zc_reduce_native<3>(NativeReduceArgs);
template __global__ void zc_reduce_native<4>(NativeReduceArgs);
template __global__ void zc_reduce_native<5>(NativeReduceArgs);
template __global__ void zc_reduce_native<6>(NativeReduceArgs);
template __global__ void zc_reduce_native<7>(NativeReduceArgs);
template __global__ void zc_reduce_native<8>(NativeReduceArgs);
template __global__ void zc_reduce_native<9>(NativeReduceArgs);
template __global__ void zc_reduce_native<10>(NativeReduceArgs);
template __global__ void zc_reduce_native<11>(NativeReduceArgs);
template __global__ void zc_reduce_native<12>(NativeReduceArgs);
template __global__ void zc_reduce_native<13>(NativeReduceArgs);
template __global__ void zc_reduce_native<14>(NativeReduceArgs);
template __global__ void zc_reduce_native<15>(NativeReduceArgs);
template __global__ void zc_reduce_native<16>(NativeReduceArgs);

// Eight waves per SIMD for the plain decoder (it fits in 64 VGPRs).
template <bool SINGLE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void zc_decode(DecodeArgs a) {
    decode_kernel<false, SINGLE>(a);
}

template __global__ void zc_decode<true>(DecodeArgs);
template __global__ void zc_decode<false>(DecodeArgs);

// Four waves per SIMD for the fused reduce (32 accumulators per lane).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void zc_decode_reduce(
    DecodeArgs a) {
    decode_kernel<true, false>(a);
}

}  // namespace zc
