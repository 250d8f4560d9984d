// zc_format.h -- stream-format constants and the plain structs the host
// builds at plan time and the kernels read (no HIP types: the host-only plan
// code builds with any C++ compiler).
#pragma once

#include <stdint.h>

namespace zc {

constexpr uint32_t kGroup = 2048;
constexpr uint32_t kHeaderBytes = 64;
constexpr uint32_t kMagic = 0x3142435Au;  // "ZCB1"
constexpr uint32_t kVersion = 1;
constexpr uint32_t kFlagRaw = 1;  // header flags byte: the values stored as they are
constexpr uint32_t kMaxStreams = 16;
constexpr uint32_t kSigmaBlock = 16384;  // values per moment partial (or the chunk, if smaller)
// The merged finish kernel sums a chunk's escape offset from the moment
// blocks before it: segments up to kFinishMaxBlocks blocks (256M values)
// use it.  Its window workgroups each join kFinishPartBlocks of a segment's
// blocks (268,435,456 values: the compress call 236 -> 215.5 us with the
// merged tail instead of the window and placement kernels, a failed
// prediction's 510 -> 376 us).
constexpr uint32_t kFinishMaxBlocks = 16384;
constexpr uint32_t kFinishPartBlocks = 2048;
constexpr uint32_t kFinishMaxParts = kFinishMaxBlocks / kFinishPartBlocks;

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
    uint32_t sb_base;    // first entry of this segment's moment block arrays (2^ceil(log2 nsb) entries)
    uint32_t group_base; // first group of this segment in the plan's list
    uint32_t chunk_base; // first chunk of this segment in the plan's list
    uint32_t wg_base;    // first encoder workgroup item of this segment
    uint32_t nwg;        // encoder workgroup items (16,384 values each)
    uint32_t wr;         // window-kernel workgroups of this segment
    uint32_t pad;
};

struct ItemDesc {  // a moment block, chunk or group: its segment and index inside it
    uint32_t seg;
    uint32_t local;
};

struct Partials {  // per moment block, plan-wide arrays (segment s from sb_base)
    double* s1;     // moments, at the block's leaf slot (leaf_slot)
    double* s2;
    uint32_t* n;    // finite values, at the leaf slot
    uint32_t* esc;  // escapes of the last encoder pass, at the block index
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
    uint64_t ps1;       // f64 per moment block slot
    uint64_t ps2;       // f64 per moment block slot
    uint64_t pn;        // u32 per moment block slot
    uint64_t pesc;      // u32 per moment block
    uint64_t stats;     // SegStat per segment
    uint64_t gcnt;      // u32 per group: escape count
    uint64_t pred;      // u32 per segment: the window of the first encoder pass
    uint64_t done;      // u32 per segment: window workgroups done re-coding
    uint64_t zero;      // u32: zero (written by the encoder's first pass)
    uint64_t staging;   // 2048 bytes per group (+16): escape exponents before placement
    uint64_t flag;      // u32 per segment: the finish kernel's window verdict (0 until known)
    uint64_t agg;       // u64 per chunk: the finish kernel's look-back words
    uint64_t fpart;     // 8 x 4 u64 per segment: the finish kernel's moment parts
    uint64_t total;
    // the decoders use only the status words and, right after them, 2048
    // readable bytes they never write (the loads' stand-in): a decode-only
    // workspace is dec_total bytes; in the full layout the stand-in falls on
    // the regions after the status words
    uint64_t dummy;
    uint64_t dec_total;
};

}  // namespace zc
