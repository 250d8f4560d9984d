/*
 * zc.h -- lossless BF16 exponent coding on AMD MI355X (gfx950): C ABI.
 *
 * The codec (ZipCCL, SIGCOMM scribe notes, "Key idea and contribution",
 * technique 1): a BF16 tensor's frequent-exponent window is derived from its
 * standard deviation; each value whose 8-bit exponent falls in the 7-binade
 * window is stored as a 3-bit code plus its raw sign+mantissa byte, and every
 * other value (zeros, subnormals, Inf/NaN included) takes the escape code and
 * keeps its full exponent byte in a separate compacted stream, so decoding
 * is bit-exact at about 11 bits per value.  Technique 2 of the same section
 * asks for GPU kernels with a communication-aware, aligned layout; the
 * stream format (version 1) is:
 *
 *   [0,64) header | chunk table (K+1 u32) | group table (one u16 per 2048
 *   values) | code planes (768 B per 2048 values) | sign+mantissa bytes
 *   (2048 B per 2048 values) | escape bytes
 *
 * with the code planes and every region after them 256-byte aligned.  Chunk
 * table entry k is the number of escapes before chunk k (entry K = E); group
 * table entry g is the number of escapes in group g's chunk before group g.
 * Field by field:
 *   u32 magic "ZCB1" @0, u16 version=1 @4, u8 L @6, u8 flags=0 @7,
 *   u64 N @8, u32 C @16, u32 K @20, u64 E @24, u64 total @32,
 *   u64 code_off @40, u64 sm_off @48, u64 esc_off @56.
 *
 * A raw stream (only from plans made with ZC_PLAN_RAW_FALLBACK) has flags 1,
 * L 0, E 0, total 64 + 2N and the three offsets 0, and holds the N BF16
 * words as they are from byte 64.  It is written when the coded stream
 * would be longer (ties stay coded): mostly zeros, near-uniform bit
 * patterns, tensors of a few thousand values.  This is the notes' switch
 * between the compressed and the native path by compression benefit
 * (technique 3 of the same section), taken per stream.  Decoders accept
 * both kinds whatever their plan's flags.
 *
 * Conventions for every call below:
 *  - "d_" pointers are device memory owned by the caller; the library never
 *    frees, keeps or reallocates them.  Host pointers are read during the
 *    call only.
 *  - BF16 data are 16-bit patterns.  A plan lays several independent
 *    segments (each its own stream) side by side: segment s occupies BF16
 *    elements [zc_plan_input_offset(s), +segment_elems[s]) of the
 *    uncompressed buffer and bytes [zc_plan_stream_offset(s),
 *    +zc_plan_max_stream_bytes(s)) of the compressed buffer.
 *  - The compress / decompress calls only enqueue work on `stream`: they do
 *    not allocate, synchronise or read device memory on the host.  Results
 *    and data-dependent errors appear in device memory when the stream
 *    reaches them.  Calls that share a workspace must not overlap.
 *  - Argument errors are returned synchronously and enqueue nothing.
 *  - Alignment: uncompressed buffers 16 B, compressed buffers and the
 *    workspace 256 B.
 */
#ifndef ZC_H
#define ZC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum zc_status {
    ZC_OK = 0,
    ZC_ERR_INVALID_ARG = 1, /* null pointer, bad size or misalignment      */
    ZC_ERR_CAPACITY = 2,    /* a buffer is smaller than the plan needs      */
    ZC_ERR_UNSUPPORTED = 3, /* chunk size or segment size out of range      */
    ZC_ERR_FORMAT = 4,      /* zc_read_status found a rejected stream        */
    ZC_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed    */
} zc_status;

/* Bits reported by zc_read_status for a rejected stream. */
#define ZC_FMT_MAGIC  0x01u /* magic, version or flags wrong             */
#define ZC_FMT_WINDOW 0x02u /* L outside 1..248                           */
#define ZC_FMT_SHAPE  0x04u /* N, C, K or a region offset disagree        */
#define ZC_FMT_SIZE   0x08u /* E > N, or total bytes past the buffer      */
#define ZC_FMT_TABLE  0x10u /* chunk table not 0..E and non-decreasing, or
                               a chunk's first group entry is not 0        */
#define ZC_FMT_COUNT  0x20u /* a group's escape count differs from codes */
#define ZC_FMT_PAD    0x40u /* nonzero code bits or sm bytes past N       */

typedef struct zc_plan zc_plan; /* opaque, host-owned, immutable */

/* Library version (stream format version is 1). */
int zc_version(void);
const char *zc_status_string(zc_status s);

/*
 * Plan for `num_segments` segments of `segment_elems[s]` BF16 values each
 * (each < 2^32; zero allowed), chunk size `chunk_elems` (a power of two in
 * 2048..65536; 0 selects 65536).  The chunk is the unit of the escape
 * index (the chunk table).  Allocates a small device descriptor table on
 * the current device.  On success *out_plan must later be passed to
 * zc_plan_destroy.
 */
zc_status zc_plan_create(uint32_t num_segments, const uint64_t *segment_elems,
                         uint32_t chunk_elems, zc_plan **out_plan);

/* Plan flags. */
#define ZC_PLAN_RAW_FALLBACK 0x1u /* compress writes a raw stream for a segment
                                     whose coded stream would exceed 64 + 2N
                                     bytes (see the format above) */

/* zc_plan_create with flags (0 or ZC_PLAN_RAW_FALLBACK; other bits:
 * ZC_ERR_INVALID_ARG).  The raw copy happens in the escape-placement
 * kernel, after the header is written, so the compress call's work stays
 * the same three kernels; a raw segment costs one more pass over its
 * values. */
zc_status zc_plan_create_ex(uint32_t num_segments, const uint64_t *segment_elems,
                            uint32_t chunk_elems, uint32_t flags, zc_plan **out_plan);
void zc_plan_destroy(zc_plan *plan);

uint32_t zc_plan_num_segments(const zc_plan *plan);
uint32_t zc_plan_chunk_elems(const zc_plan *plan);
uint32_t zc_plan_flags(const zc_plan *plan);
/* BF16 element offset of segment s (a multiple of 8) and total elements. */
uint64_t zc_plan_input_offset(const zc_plan *plan, uint32_t s);
uint64_t zc_plan_input_elems(const zc_plan *plan);
/* Byte offset (multiple of 256) and worst-case size of segment s's stream. */
uint64_t zc_plan_stream_offset(const zc_plan *plan, uint32_t s);
uint64_t zc_plan_max_stream_bytes(const zc_plan *plan, uint32_t s);
/* Offsets, from the start of segment s's stream, of its code planes and of
 * its escape region; [code offset, escape offset) holds the code planes and
 * the sign+mantissa bytes (sizes fixed by the plan). */
uint64_t zc_plan_code_offset(const zc_plan *plan, uint32_t s);
uint64_t zc_plan_escape_offset(const zc_plan *plan, uint32_t s);
/* Bytes the compressed buffer must hold for every segment's worst case. */
uint64_t zc_plan_out_bytes(const zc_plan *plan);
/* Workspace bytes needed by any call with this plan: about one byte per
 * value (compress stages escape exponents there, 2048 bytes per 2048-value
 * group) plus a few bytes per group and chunk. */
uint64_t zc_plan_workspace_bytes(const zc_plan *plan);
/* Workspace bytes zc_decompress, zc_decompress_reduce and zc_read_status
 * need: 4 bytes per 2048-value group (the rejection bits), rounded up to 256,
 * plus 2048 bytes (256 for a plan without values).  A receiver that only
 * decodes can pass a workspace of this size; a workspace of
 * zc_plan_workspace_bytes, which is never smaller, serves every call. */
uint64_t zc_plan_decode_workspace_bytes(const zc_plan *plan);

/*
 * Compress every segment of d_in (BF16, zc_plan_input_elems elements) into
 * d_out (out_capacity >= zc_plan_out_bytes bytes).  Segment s's stream is
 * written at d_out + zc_plan_stream_offset(s) and its exact size in bytes to
 * d_stream_bytes[s] (device, one u64 per segment).  Bytes between a stream's
 * end and the next segment's offset are left untouched.
 * The window of each segment comes from its standard deviation (fp64
 * moments by a pairwise tree, population variance of the finite values,
 * the 7-binade window of largest Gaussian mass).
 * One pass over the input: it is coded with the window the workspace
 * recorded for the segment on the previous call (any value on a fresh
 * workspace) while the moments are taken; a segment whose window turns out
 * different is coded again in the same call.  The streams are the same
 * either way; a call after a change of window only takes longer.  Calls
 * that share a workspace must not overlap.
 */
zc_status zc_compress(const zc_plan *plan, const void *d_in, void *d_out,
                      uint64_t out_capacity, uint64_t *d_stream_bytes,
                      void *d_ws, uint64_t ws_bytes, hipStream_t stream);

/*
 * zc_compress for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * streams and sizes, with the workspace taken from a device array inside the
 * library (zc_static_workspace_bytes() = 80 MiB per GPU, reserved on each
 * GPU the library runs on until the process ends) instead of a caller's
 * buffer.  The call allocates and frees nothing; the caller still passes the
 * input, the output and d_stream_bytes as for zc_compress.  Plans whose
 * zc_plan_workspace_bytes exceed the array (about 80 million values) are
 * refused with ZC_ERR_CAPACITY; ZC_ERR_HIP if the array cannot be found on
 * the current device.  Every call on one GPU uses that GPU's one array: calls
 * that overlap on a GPU (other streams, other threads) race and must not be
 * made.  The array keeps the last call's contents; nothing in it needs to
 * start at zero (the window it holds from the previous call is only a
 * prediction, checked on every call).
 */
zc_status zc_compress_static(const zc_plan *plan, const void *d_in, void *d_out,
                             uint64_t out_capacity, uint64_t *d_stream_bytes,
                             hipStream_t stream);
uint64_t zc_static_workspace_bytes(void);

/*
 * As zc_compress, but every segment uses the window L (1..248) given here
 * instead of one derived from its standard deviation: no moments are taken
 * and no statistics are written.  The coding itself is the ZipCCL notes'
 * ("Key idea and contribution", technique 1): exponents in [L, L+6] become
 * 3-bit codes, the others escape with their full byte, so the stream is
 * lossless whatever L is; only its size depends on L.  This serves a window
 * known in advance, e.g. one carried over from an earlier iteration of the
 * same tensor (the exponent reuse across iterations named by the CIERA
 * title that the pages list).  Errors as zc_compress, plus
 * ZC_ERR_INVALID_ARG for L outside 1..248.
 */
zc_status zc_compress_window(const zc_plan *plan, const void *d_in, void *d_out,
                             uint64_t out_capacity, uint64_t *d_stream_bytes,
                             uint32_t window_L, void *d_ws, uint64_t ws_bytes,
                             hipStream_t stream);

/*
 * zc_compress that also records `fixed_ready` (a HIP event the caller
 * created) on `stream` as soon as, for every segment, the bytes before the
 * group table (header and chunk table), the bytes [code offset, escape
 * offset) and d_stream_bytes are final; the group table and the escape
 * region are final when the call's work completes.  A caller can wait on the
 * event from another stream and start the size exchange and the sending of
 * those regions while the escapes are still being placed (ZipCCL's
 * static/dynamic split, Fig. 5).  Plans with ZC_PLAN_RAW_FALLBACK are
 * refused (ZC_ERR_INVALID_ARG): a raw stream's bytes are written after the
 * event.
 */
zc_status zc_compress_split(const zc_plan *plan, const void *d_in, void *d_out,
                            uint64_t out_capacity, uint64_t *d_stream_bytes,
                            void *d_ws, uint64_t ws_bytes, hipStream_t stream,
                            hipEvent_t fixed_ready);

/*
 * For profiling: zc_compress with HIP events recorded on `stream` before,
 * between and after its kernels; waits for the call to finish and writes
 * the kernels' times in microseconds to us[0] (encoder pass: moments, codes,
 * staged escapes), us[1] (window, check of the prediction, chunk table; on
 * plans where one kernel does this and the escape placement, that kernel)
 * and us[2] (escape placement when it is a kernel of its own, else 0).
 * Each time spans a pair of events, so it includes the events' own overhead
 * (an empty pair reads about 4.4 us on an MI355X).  Same output as
 * zc_compress.
 */
zc_status zc_compress_timed(const zc_plan *plan, const void *d_in, void *d_out,
                            uint64_t out_capacity, uint64_t *d_stream_bytes,
                            void *d_ws, uint64_t ws_bytes, hipStream_t stream,
                            float *us);

/*
 * Decompression, the last step of the ZipCCL notes' compressed-collective
 * workflow (Fig. 5: compress, exchange sizes, communicate, decompress), as
 * the inverse of the exponent coding of "Key idea and contribution",
 * technique 1: e = L + code for codes 0..6, the next escape byte for code 7,
 * sign and mantissa from the raw byte; a raw stream's words are copied.
 * Decodes every segment's stream (at d_in + zc_plan_stream_offset(s); the
 * buffer holds in_capacity readable bytes, 256-B aligned) into d_out (BF16,
 * laid out as d_in of zc_compress, 16-B aligned).  d_ws: at least
 * zc_plan_decode_workspace_bytes bytes, 256-B aligned; it receives the
 * rejection bits.  Streams are validated on the device; a group of 2048
 * values whose checks fail writes no output and is reported by
 * zc_read_status, and other groups are decoded as usual.  Reads never leave
 * [d_in, d_in + in_capacity).  Argument errors: ZC_ERR_INVALID_ARG (null or
 * misaligned pointer), ZC_ERR_CAPACITY (workspace too small).
 */
zc_status zc_decompress(const zc_plan *plan, const void *d_in,
                        uint64_t in_capacity, void *d_out, void *d_ws,
                        uint64_t ws_bytes, hipStream_t stream);

/*
 * Receive side of a compressed reduce-scatter (the ZipCCL notes' "Key idea
 * and contribution", technique 3, names the reduce-scatter path; the UCCL-Zip
 * page's abstract argues for running decompression inside the collective's
 * kernel, which removes extra memory traffic and launches): every shard is
 * decoded (as zc_decompress) and summed in one kernel, so the only global
 * write is the sum.  The plan has one segment of N values; d_streams is a
 * HOST array of `nstreams` (1..16) device pointers (256-B aligned), each to
 * a stream of N values with stream_capacity readable bytes.  Writes
 * d_out[i] = bf16_rne(((x0[i] + x1[i]) + x2[i]) + ...) with the sum in fp32
 * in the given stream order (no flush of subnormals); any NaN sum gives
 * 0x7FC0.  A rejected stream makes the affected 2048-value groups write no
 * output (see zc_read_status).  d_ws as for zc_decompress.  Argument errors:
 * ZC_ERR_INVALID_ARG (plan with more than one segment, nstreams outside
 * 1..16, null or misaligned pointer), ZC_ERR_CAPACITY (workspace too small).
 */
zc_status zc_decompress_reduce(const zc_plan *plan, const void *const *d_streams,
                               uint32_t nstreams, uint64_t stream_capacity,
                               void *d_out, void *d_ws, uint64_t ws_bytes,
                               hipStream_t stream);

/*
 * Rejection report of the decompress step of the ZipCCL notes' workflow
 * (Fig. 5).  The pages define no stream validation; this is the library's
 * own error channel for data-dependent errors, which the enqueue-only calls
 * cannot return.  Synchronises `stream`, then ORs the ZC_FMT_* bits of the
 * most recent zc_decompress / zc_decompress_reduce that used this workspace
 * (any layout: the bits sit at its start) into *host_bits.  Returns
 * ZC_ERR_FORMAT if any bit is set, ZC_ERR_HIP if the stream or the copy
 * failed, ZC_ERR_INVALID_ARG for a null argument.
 */
zc_status zc_read_status(const zc_plan *plan, const void *d_ws,
                         hipStream_t stream, uint32_t *host_bits);

/*
 * Synchronises `stream`, then copies the window statistics of segment s from
 * the most recent zc_compress on this workspace: S1 = sum of values,
 * S2 = sum of squares (fp64 pairwise), n = finite values, var and L.
 * Any output pointer may be NULL.
 */
zc_status zc_read_sigma(const zc_plan *plan, const void *d_ws, uint32_t s,
                        hipStream_t stream, double *S1, double *S2,
                        uint64_t *n, double *var, uint32_t *L);

/*
 * Host-side switch between sending a tensor compressed and sending it raw
 * over a link of link_GBps (GB/s, > 0): returns 1 when
 *   compress_us + compressed_bytes / link + decompress_us < raw_bytes / link
 * (ZipCCL, "Key idea and contribution", technique 3: the reduce-scatter path
 * switches to the native collective when compression does not pay; for a
 * reduce-scatter, decompress_us is the fused decompress-reduce's time minus
 * the native reduce's).  Times are measured ones (microseconds).  When
 * break_even_GBps is not NULL it receives the link bandwidth below which
 * compression pays, (raw - compressed) / (compress_us + decompress_us), or 0
 * when the compressed form is not smaller.  Returns 0 for invalid arguments
 * (link_GBps <= 0, negative times).
 */
int zc_prefer_compressed(uint64_t raw_bytes, uint64_t compressed_bytes, double compress_us,
                         double decompress_us, double link_GBps, double *break_even_GBps);

/*
 * The native path of a reduce-scatter's receive side, the alternative that
 * the ZipCCL notes' switch ("Key idea and contribution", technique 3) weighs
 * the compressed path against: d_out[i] = bf16_rne(((x0[i] + x1[i]) + x2[i])
 * + ...) over `nshards` (1..16) uncompressed BF16 shards of n values each,
 * summed in fp32 in the given order with the rounding of
 * zc_decompress_reduce (so both give the same bits for the same values).
 * d_shards: HOST array of device pointers, each 16-B aligned; d_out: n BF16
 * values, 16-B aligned.  One kernel on `stream`, no workspace.  Errors:
 * ZC_ERR_INVALID_ARG (null or misaligned pointer, nshards outside 1..16).
 */
zc_status zc_reduce_native(const void *const *d_shards, uint32_t nshards, uint64_t n,
                           void *d_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ZC_H */
