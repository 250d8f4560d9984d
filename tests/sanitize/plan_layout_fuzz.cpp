// plan_layout_fuzz.cpp -- the library's host plan code under AddressSanitizer
// and UBSan.
//
// Test infrastructure: built with g++ -fsanitize=address,undefined by
// tests/test_plan_layout_sanitized.py from the library's own header
// (csrc/zc_plan_layout.h, plain C++).  Builds layouts for seeded random
// segment lists (empty segments, tiny and ragged ones, 2^32 - 1 values,
// 256 segments, every chunk size) and checks each against the format's
// closed forms and the kernels' indexing: regions aligned and disjoint,
// offsets as the stream format fixes them, item lists covering every group,
// chunk and encoder item once, workspace regions large enough for every
// index the kernels form.  Any out-of-bounds access, overflow or broken
// invariant ends the run with a report.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "zc_plan_layout.h"

using namespace zc;

static uint64_t rng = 0x243F6A8885A308D3ull;
static uint64_t next_u64() {  // xorshift64* (Vigna)
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return rng * 0x2545F4914F6CDD1Dull;
}

static int failures = 0;
#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            if (++failures > 20) exit(1);                                   \
        }                                                                   \
    } while (0)

static uint64_t a256(uint64_t v) { return (v + 255) / 256 * 256; }
static uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
static uint64_t pow2_at_least(uint64_t v) {
    uint64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

static void check_layout(const std::vector<uint64_t>& n, uint32_t chunk_arg, uint32_t flags = 0) {
    PlanLayout L;
    const int rc = build_layout((uint32_t)n.size(), n.data(), chunk_arg, flags, L);
    uint64_t G = 0;
    for (uint64_t v : n) G += cdiv(v, kGroup);
    const uint32_t C = chunk_arg ? chunk_arg : 65536u;
    const bool c_ok = C >= kGroup && C <= 65536u && (C & (C - 1)) == 0;
    if (!c_ok || G >= (1ull << 31)) {
        CHECK(rc == kLayoutUnsupported);
        return;
    }
    CHECK(rc == kLayoutOk);
    if (rc != kLayoutOk) return;
    CHECK(L.nseg == n.size() && L.chunk == C && L.block == (C < kSigmaBlock ? C : kSigmaBlock));
    CHECK(L.flags == flags);
    CHECK(L.segs.size() == n.size() && L.groups.size() == G);
    uint64_t in_end = 0, out_end = 0, K = 0, slots = 0, items = 0, wgs = 0;
    for (size_t s = 0; s < n.size(); ++s) {
        const SegDesc& d = L.segs[s];
        CHECK(d.n == n[s]);
        CHECK(d.k == cdiv(n[s], C) && d.g == cdiv(n[s], kGroup) && d.nsb == cdiv(n[s], L.block));
        // the stream format's offsets
        CHECK(d.gtab_off == 64 + 4ull * (d.k + 1));
        CHECK(d.code_off == a256(d.gtab_off + 2ull * d.g));
        CHECK(d.sm_off == d.code_off + 768ull * d.g && d.esc_off == d.sm_off + 2048ull * d.g);
        CHECK(d.max_bytes == d.esc_off + n[s]);
        // inputs 8-element aligned, streams 256-byte aligned, disjoint, in order
        CHECK(d.in_off % 8 == 0 && d.in_off >= in_end);
        CHECK(d.out_off % 256 == 0 && d.out_off >= out_end);
        in_end = d.in_off + n[s];
        out_end = d.out_off + d.max_bytes;
        // item lists: this segment's chunks and groups, consecutive
        CHECK(d.chunk_base == K && d.group_base + d.g <= L.groups.size());
        for (uint32_t k = 0; k < d.k; ++k)
            CHECK(L.chunks[d.chunk_base + k].seg == s && L.chunks[d.chunk_base + k].local == k);
        for (uint32_t g = 0; g < d.g; ++g)
            CHECK(L.groups[d.group_base + g].seg == s && L.groups[d.group_base + g].local == g);
        K += d.k;
        // moment-partial slots: the power of two above the block count
        CHECK(d.sb_base == slots);
        slots += d.nsb ? pow2_at_least(d.nsb) : 0;
        // encoder items: 4 waves of 2 groups, padded to whole workgroups
        CHECK(d.wg_base == items && d.nwg == cdiv((d.g + 1) / 2, 4));
        for (uint32_t w = 0; w < 4 * d.nwg; ++w) {
            const ItemDesc& it = L.pairs[4ull * d.wg_base + w];
            if (w < (d.g + 1) / 2) CHECK(it.seg == s && it.local == w);
            else CHECK(it.seg == 0xFFFFFFFFu);
        }
        // an item covers 16,384 values: whole moment blocks of its segment
        CHECK((16384u % L.block) == 0);
        items += d.nwg;
        // window workgroups: about 16 items each, 1..256
        CHECK(d.wr >= 1 && d.wr <= 256 && d.wr == (uint32_t)std::min<uint64_t>(256, std::max<uint64_t>(1, cdiv(d.nwg, 16))));
        for (uint32_t r = 0; r < d.wr; ++r)
            CHECK(L.witems[wgs + r].seg == s && L.witems[wgs + r].local == r);
        wgs += d.wr;
    }
    CHECK(L.chunks.size() == K && L.pairs.size() == 4 * items && L.witems.size() == wgs);
    // the merged finish kernel: no raw fallback, and segments of at most
    // kFinishMaxBlocks moment blocks
    bool merged = (flags & kPlanRawFallback) == 0;
    for (const SegDesc& d : L.segs) merged = merged && d.nsb <= kFinishMaxBlocks;
    CHECK(L.merged_tail == merged);
    // the finish kernel's window parts: each segment's blocks in parts of
    // kFinishPartBlocks, in segment order
    size_t fi = 0;
    for (size_t s = 0; s < n.size(); ++s) {
        const uint32_t nsb = L.segs[s].nsb;
        const uint64_t parts = nsb > kFinishPartBlocks ? cdiv(nsb, kFinishPartBlocks) : 1;
        for (uint64_t q = 0; q < std::min<uint64_t>(parts, kFinishMaxParts); ++q, ++fi)
            CHECK(fi < L.fitems.size() && L.fitems[fi].seg == s && L.fitems[fi].local == q);
        if (merged) CHECK(parts <= kFinishMaxParts);
    }
    CHECK(fi == L.fitems.size());
    CHECK(L.input_elems >= in_end && L.input_elems % 8 == 0 && L.out_bytes >= out_end);
    // workspace regions: aligned, in order, each as large as the kernels index
    const WsLayout& w = L.ws;
    const uint64_t S = n.size();
    const uint64_t start[] = {w.status, w.ps1, w.ps2, w.pn, w.pesc, w.stats, w.gcnt,
                              w.pred, w.done, w.zero, w.staging, w.flag, w.agg, w.fpart, w.total};
    const uint64_t need[] = {4 * G, 8 * slots, 8 * slots, 4 * slots, 4 * slots,
                             sizeof(SegStat) * S, 4 * G, 4 * S, 4 * S, 4,
                             (uint64_t)kGroup * G + 16, 4 * S, 8 * K, 32ull * kFinishMaxParts * S};
    for (int i = 0; i < 14; ++i) {
        CHECK(start[i] % 256 == 0);
        CHECK(start[i] + need[i] <= start[i + 1]);
    }
    // the decoders' workspace: status words, then a 2048-byte stand-in that
    // lies inside the full layout too
    CHECK(w.dummy == a256(4 * G) && w.dec_total == (G ? w.dummy + 2048 : 256));
    CHECK(w.dec_total <= w.total);
}

int main() {
    // edge cases
    check_layout({0}, 0);
    check_layout({1}, 0);
    check_layout({0, 0, 0}, 2048);
    check_layout({(1ull << 32) - 1}, 0);
    check_layout({(1ull << 32) - 1}, 2048);
    check_layout({(1ull << 32) - 1}, 0, kPlanRawFallback);
    check_layout({0, 1, 70000}, 4096, kPlanRawFallback);
    check_layout({7, 8, 2047, 2048, 2049, 16383, 16384, 16385, 65535, 65536, 65537}, 0);
    for (uint32_t c : {0u, 1000u, 1024u, 2048u, 3000u, 4096u, 8192u, 16384u, 32768u, 65536u, 131072u})
        check_layout({12345, 0, 99999}, c);
    {   // 256 segments (the MoE batch's count)
        std::vector<uint64_t> v;
        for (int s = 0; s < 256; ++s) v.push_back(7168ull * (21 + (s * 37) % 700));
        check_layout(v, 0);
    }
    {   // refused before anything is allocated: 2^31 groups
        std::vector<uint64_t> v(1024, (1ull << 32) - 1);
        PlanLayout L;
        CHECK(build_layout((uint32_t)v.size(), v.data(), 0, 0, L) == kLayoutUnsupported);
        const uint64_t big = 1ull << 32;
        CHECK(build_layout(1, &big, 0, 0, L) == kLayoutUnsupported);
        CHECK(build_layout(0, &big, 0, 0, L) == kLayoutInvalidArg);
        CHECK(build_layout(1, nullptr, 0, 0, L) == kLayoutInvalidArg);
    }
    // seeded random plans
    const uint32_t chunks[] = {0, 2048, 4096, 8192, 16384, 32768, 65536};
    int plans = 0;
    for (int t = 0; t < 3000; ++t) {
        const uint32_t nseg = 1 + (uint32_t)(next_u64() % (t % 10 == 0 ? 256 : 8));
        std::vector<uint64_t> v(nseg);
        for (auto& x : v) {
            const uint64_t r = next_u64();
            switch (r % 8) {
                case 0: x = 0; break;
                case 1: x = (r >> 8) % 16; break;
                case 2: x = (r >> 8) % 4096; break;
                case 3: x = (r >> 8) % 300000; break;
                case 4: x = 2048ull * ((r >> 8) % 64) + ((r >> 20) % 3) - 1 + 1; break;
                case 5: x = (r >> 8) % (nseg > 8 ? 2000000 : 60000000); break;
                default: x = (r >> 8) % 1000000; break;
            }
        }
        if (t % 500 == 7) v[0] = (1ull << 32) - 1 - (next_u64() % 5000);
        check_layout(v, chunks[next_u64() % 7], (next_u64() & 1) ? kPlanRawFallback : 0u);
        ++plans;
    }
    if (failures) return 1;
    printf("ok: %d random plans and the edge cases\n", plans);
    return 0;
}
