// zc_encode.hip -- the encoder's first pass and the escape placement.
//
// ZipCCL scribe notes, "Key idea and contribution", techniques 1 and 2.
//
// zc_encode: one workgroup item (zc_encoder.h) per workgroup, with the
// window predicted from the previous call (or the caller's fixed window);
// records the window it used per segment.  GW = 2: four waves of two groups
// (the common shape); GW = 1: eight waves of one group, for grids of at most
// 256 items, whose time is one wave's chain rather than the chip's bandwidth.  The window kernel checks the
// prediction and codes the segment again where it failed.
//
// zc_place_escapes, one workgroup per chunk, one wave per encoder wave: the
// group counts give the group table; the chunk's offset in the segment's
// escape stream comes from the chunk table; each wave's runs, whose source
// dwords are loaded before that offset is known, go to their place.
#include <type_traits>

#include "zc_place.h"

namespace zc {

template <bool MOMENTS, int GW>
__global__ __launch_bounds__(GW == 2 ? 256 : 512) void zc_encode(EncodeArgs a) {
    __shared__ typename std::conditional<GW == 2, EncodeLds, EncodeLds8>::type lds;
    encode_wg<MOMENTS, false, GW>(a, blockIdx.x, a.forced_L, lds);  // 0: the predicted window
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.zero = 0u;
    const ItemDesc first = a.single ? ItemDesc{0u, 4 * blockIdx.x} : a.pairs[blockIdx.x * 4];
    if (first.local == 0 && threadIdx.x == 0) {  // the segment's first item
        a.pred[first.seg] = a.forced_L ? a.forced_L : predicted_L(a.stats[first.seg].L);
        a.done[first.seg] = 0;
        a.flag[first.seg] = 0;
        for (uint32_t i = 0; i < 4 * kFinishMaxParts; ++i) a.fpart[4ull * kFinishMaxParts * first.seg + i] = ~0ull;
    }
    // the look-back words of the chunks that start in this item (16,384
    // values from value 4096 * first.local)
    const uint32_t per = kSigmaBlock / a.chunk_elems;  // chunks per item (0: an item per chunk part)
    const uint64_t v0 = 4096ull * first.local;
    if (threadIdx.x < (per ? per : 1u) && v0 % a.chunk_elems == 0) {
        const uint32_t base = a.single ? a.seg0.chunk_base : a.segs[first.seg].chunk_base;
        const uint32_t k = (uint32_t)(v0 / a.chunk_elems) + threadIdx.x;
        const uint32_t nk = a.single ? a.seg0.k : a.segs[first.seg].k;
        if (k < nk) a.agg[base + k] = 0;
    }
}

template __global__ void zc_encode<true, 2>(EncodeArgs);
template __global__ void zc_encode<false, 2>(EncodeArgs);
template __global__ void zc_encode<true, 1>(EncodeArgs);

template <int GPW>
__global__ __launch_bounds__(256) void zc_place_escapes(PlaceArgs a) {
    __shared__ PlaceLds<GPW> lds;
    for (uint32_t ci = blockIdx.x; ci < a.nchunks; ci += gridDim.x) {
        PlaceChunk<GPW> pc;
        place_begin(a, ci, pc);
        // the chunk's escape offset (chunk table, written from the group
        // counts before this kernel runs) and its raw verdict (flags byte 1,
        // set by the window kernel) go out before the staging loads: the
        // scan waits only for them
        const uint32_t prefix = reinterpret_cast<const uint32_t*>(pc.st + kHeaderBytes)[pc.local];
        const bool raw = (reinterpret_cast<const uint32_t*>(pc.st)[1] >> 24) == kFlagRaw;
        place_load<GPW, false>(a, pc);
        place_finish<GPW>(a, pc, prefix, raw, lds, [] { return true; });
    }
}

template __global__ void zc_place_escapes<1>(PlaceArgs);
template __global__ void zc_place_escapes<2>(PlaceArgs);
template __global__ void zc_place_escapes<4>(PlaceArgs);
template __global__ void zc_place_escapes<8>(PlaceArgs);

}  // namespace zc
