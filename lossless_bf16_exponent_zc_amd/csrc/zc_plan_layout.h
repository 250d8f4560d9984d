// zc_plan_layout.h -- the host side of a plan: per-segment geometry, the
// kernels' item lists and the workspace carve-up, from the segment sizes and
// the chunk size alone.  Plain C++ (no HIP): the library builds it into
// zc_plan_create, and a sanitizer-instrumented host test drives it directly.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "zc_format.h"

namespace zc {

struct PlanLayout {
    uint32_t nseg = 0, chunk = 0, block = 0, flags = 0;
    std::vector<SegDesc> segs;
    std::vector<ItemDesc> chunks, groups, pairs, witems;  // pairs: encoder waves; witems: window workgroups
    std::vector<ItemDesc> fitems;  // the finish kernel's window workgroups: (segment, part)
    uint64_t input_elems = 0, out_bytes = 0;
    WsLayout ws{};
    // compress ends with the merged finish kernel: no segment over
    // kFinishMaxBlocks moment blocks, no raw fallback
    bool merged_tail = false;
};

constexpr uint32_t kPlanRawFallback = 1;  // ZC_PLAN_RAW_FALLBACK

// The ZC_ERR_* values of zc.h that a layout can give.
enum LayoutStatus : int { kLayoutOk = 0, kLayoutInvalidArg = 1, kLayoutUnsupported = 3, kLayoutNoMemory = 5 };

inline uint64_t layout_a256(uint64_t v) { return (v + 255) & ~uint64_t(255); }
inline uint64_t layout_cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Fills L for `nseg` segments of sizes[s] values (each < 2^32) and chunk
// size chunk_elems (0: 65536; else a power of two in 2048..65536).  Segments
// are laid side by side: inputs 8-element aligned, streams 256-byte aligned
// at their worst-case size.  Per segment: K chunks, G groups of 2048, moment
// blocks of 16,384 values (or the chunk, if smaller) whose partials take
// 2^ceil(log2 blocks) slots; encoder items of 4 waves x 2 groups (each
// segment padded to whole workgroups); window workgroups ~ items / 16, 1..256.
inline int build_layout(uint32_t nseg, const uint64_t* sizes, uint32_t chunk_elems, uint32_t flags,
                        PlanLayout& L) {
    if (nseg == 0 || !sizes) return kLayoutInvalidArg;
    const uint32_t C = chunk_elems ? chunk_elems : 65536u;
    if (C < kGroup || C > 65536u || (C & (C - 1))) return kLayoutUnsupported;
    uint64_t total_groups = 0;  // the lists index groups with 31 bits
    for (uint32_t s = 0; s < nseg; ++s) {
        if (sizes[s] >= (1ull << 32)) return kLayoutUnsupported;
        total_groups += layout_cdiv(sizes[s], kGroup);
    }
    if (total_groups >= (1ull << 31)) return kLayoutUnsupported;
    try {
        L = PlanLayout{};
        L.nseg = nseg;
        L.chunk = C;
        L.flags = flags;
        L.block = C < kSigmaBlock ? C : kSigmaBlock;
        uint64_t in_off = 0, out_off = 0, sb = 0;
        L.segs.reserve(nseg);
        for (uint32_t s = 0; s < nseg; ++s) {
            const uint64_t n = sizes[s];
            SegDesc d{};
            d.n = n;
            d.k = (uint32_t)layout_cdiv(n, C);
            d.g = (uint32_t)layout_cdiv(n, kGroup);
            d.nsb = (uint32_t)layout_cdiv(n, L.block);
            d.gtab_off = kHeaderBytes + 4ull * (d.k + 1);
            d.code_off = layout_a256(d.gtab_off + 2ull * d.g);
            d.sm_off = d.code_off + 768ull * d.g;
            d.esc_off = d.sm_off + 2048ull * d.g;
            d.max_bytes = d.esc_off + n;
            d.in_off = in_off;
            d.out_off = out_off;
            d.sb_base = (uint32_t)sb;
            uint64_t pb = 1;
            while (pb < d.nsb) pb <<= 1;
            sb += d.nsb ? pb : 0;  // leaf slots span the power of two
            d.group_base = (uint32_t)L.groups.size();
            d.chunk_base = (uint32_t)L.chunks.size();
            in_off += (n + 7) & ~uint64_t(7);
            out_off += layout_a256(d.max_bytes);
            for (uint32_t k = 0; k < d.k; ++k) L.chunks.push_back(ItemDesc{s, k});
            for (uint32_t g = 0; g < d.g; ++g) L.groups.push_back(ItemDesc{s, g});
            d.wg_base = (uint32_t)(L.pairs.size() / 4);
            for (uint32_t q = 0; q < (d.g + 1) / 2; ++q) L.pairs.push_back(ItemDesc{s, q});
            while (L.pairs.size() % 4) L.pairs.push_back(ItemDesc{0xFFFFFFFFu, 0});  // whole workgroups
            d.nwg = (uint32_t)(L.pairs.size() / 4) - d.wg_base;
            // window workgroups: enough to code the segment again at about 16
            // items each, at most 256 (each joins all of the segment's partials)
            d.wr = (uint32_t)std::min<uint64_t>(256, std::max<uint64_t>(1, layout_cdiv(d.nwg, 16)));
            for (uint32_t r = 0; r < d.wr; ++r) L.witems.push_back(ItemDesc{s, r});
            // the finish kernel joins a segment's moment blocks in parts of
            // kFinishPartBlocks (at least one part)
            const uint32_t parts = d.nsb > kFinishPartBlocks ? (d.nsb + kFinishPartBlocks - 1) / kFinishPartBlocks : 1u;
            for (uint32_t q = 0; q < parts && q < kFinishMaxParts; ++q) L.fitems.push_back(ItemDesc{s, q});
            L.segs.push_back(d);
        }
        L.merged_tail = !(flags & kPlanRawFallback);
        for (const SegDesc& d : L.segs) L.merged_tail = L.merged_tail && d.nsb <= kFinishMaxBlocks;
        L.input_elems = in_off;
        L.out_bytes = out_off;
        const uint64_t G = L.groups.size(), B = sb;
        uint64_t o = 0;
        WsLayout& w = L.ws;
        w.status = o;   o += layout_a256(4 * G);
        w.ps1 = o;      o += layout_a256(8 * B);
        w.ps2 = o;      o += layout_a256(8 * B);
        w.pn = o;       o += layout_a256(4 * B);
        w.pesc = o;     o += layout_a256(4 * B);
        w.stats = o;    o += layout_a256(sizeof(SegStat) * nseg);
        w.gcnt = o;     o += layout_a256(4 * G);
        w.pred = o;     o += layout_a256(4ull * nseg);
        w.done = o;     o += layout_a256(4ull * nseg);
        w.zero = o;     o += 256;
        w.staging = o;  o += layout_a256((uint64_t)kGroup * G + 16);
        w.flag = o;     o += layout_a256(4ull * nseg);
        w.agg = o;      o += layout_a256(8ull * L.chunks.size());
        w.fpart = o;    o += layout_a256(32ull * kFinishMaxParts * nseg);
        w.total = o;
        // decoders: the status words, then a 2048-byte stand-in (inside the
        // full layout too: the staging area alone is larger); a plan without
        // values decodes nothing and needs no stand-in
        w.dummy = layout_a256(4 * G);
        w.dec_total = G ? w.dummy + kGroup : 256;
    } catch (const std::bad_alloc&) {
        L = PlanLayout{};
        return kLayoutNoMemory;
    }
    return kLayoutOk;
}

}  // namespace zc
