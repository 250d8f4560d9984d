/*
 * zco.h -- CPU oracle for lossless BF16 exponent coding.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it.  It shares no code, header or constant
 * generator with the GPU library.
 *
 * Method (ZipCCL, SIGCOMM scribe notes, "Key idea and contribution",
 * first technique): the frequent-exponent range of a BF16 tensor is taken
 * from the tensor's standard deviation (no histogram, no sort); exponents in
 * that range become 3-bit codes, sign and mantissa stay raw, and exponents
 * outside it keep their full 8 bits in a separate stream, so decoding is
 * bit-exact at about 11 bits per value.
 *
 * Every pointer here is host memory.  Functions never allocate memory that
 * outlives the call and never keep state between calls.
 */
#ifndef ZCO_H
#define ZCO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format constants of stream version 1. */
#define ZCO_MAGIC        0x3142435Au /* bytes 'Z' 'C' 'B' '1' */
#define ZCO_VERSION      1u
#define ZCO_HEADER_BYTES 64u
#define ZCO_GROUP        2048u       /* values per code group */
#define ZCO_ESC          7u          /* the escape code */
#define ZCO_FLAG_RAW     1u          /* header flags: the values stored as they are */

/* Compression options (zco_compress_ex). */
#define ZCO_OPT_RAW_FALLBACK 1u /* a raw stream when the coded one is longer */

/* Decoder rejection bits (zco_decompress return value; 0 = accepted). */
#define ZCO_FMT_MAGIC    0x01u  /* magic, version or flags wrong            */
#define ZCO_FMT_WINDOW   0x02u  /* L outside [1, 248]                       */
#define ZCO_FMT_SHAPE    0x04u  /* N, C, K or a region offset disagree      */
#define ZCO_FMT_SIZE     0x08u  /* total bytes exceed the buffer            */
#define ZCO_FMT_TABLE    0x10u  /* chunk table not 0..E and monotone, or a
                                   chunk's first group-table entry not 0   */
#define ZCO_FMT_COUNT    0x20u  /* a chunk's or group's escape offsets
                                   differ from its codes                    */
#define ZCO_FMT_PAD      0x40u  /* nonzero code bits or sm bytes past N     */

/* The window constant C0: var >= C0 * 4^k  <=>  window k or higher. */
double zco_c0(void);

/* Exact value of each BF16 pattern as fp64 (Inf/NaN map to Inf/NaN). */
void zco_bf16_to_f64(const uint16_t *x, size_t n, double *out);

/* Pairwise fp64 sum: pad to the next power of two with +0.0, then add
 * neighbouring pairs level by level until one element remains. */
double zco_pairwise_sum(const double *a, size_t n);

/* Moments and variance of one tensor (finite values only).  Any output
 * pointer may be NULL. */
void zco_sigma(const uint16_t *x, size_t n, double *S1, double *S2,
               uint64_t *nfinite, double *var);

/* Window rule: lowest biased exponent L of the 7-binade window, 1..248. */
int zco_window(double var);

/* Stream geometry. */
uint64_t zco_code_off(uint64_t N, uint32_t C);
uint64_t zco_sm_off(uint64_t N, uint32_t C);
uint64_t zco_esc_off(uint64_t N, uint32_t C);
uint64_t zco_max_stream_bytes(uint64_t N, uint32_t C);

/* Compress N values with chunk size C (power of two, >= 2048).
 * forced_L < 0 applies the window rule; 1..248 forces that window.
 * Returns 0 on success, -1 on a bad argument, -2 if cap is too small. */
int zco_compress(const uint16_t *x, uint64_t N, uint32_t C, int forced_L,
                 uint8_t *out, uint64_t cap, uint64_t *out_len);

/* As zco_compress, with options (ZCO_OPT_*): with ZCO_OPT_RAW_FALLBACK a
 * tensor whose coded stream would exceed 64 + 2N bytes is stored as a raw
 * stream (header flags = 1, the N words after the header). */
int zco_compress_ex(const uint16_t *x, uint64_t N, uint32_t C, int forced_L,
                    uint32_t options, uint8_t *out, uint64_t cap, uint64_t *out_len);

/* Decode one stream of `len` readable bytes that must hold N values coded
 * with chunk size C.  Returns 0 and fills out[0..N) when the stream is
 * valid, else the OR of ZCO_FMT_* bits of the first failing check group
 * (out is then unspecified). */
uint32_t zco_decompress(const uint8_t *s, uint64_t len, uint64_t N, uint32_t C,
                        uint16_t *out);

/* BF16 round-to-nearest-even of an fp32 value; every NaN -> 0x7FC0. */
uint16_t zco_round_bf16(float f);

/* Decode S streams of N values each and sum them in shard order in fp32
 * (acc = x0; acc += x1; ...), then round each sum to BF16.  Returns the OR
 * of the streams' rejection bits (0 = all valid). */
uint32_t zco_decompress_reduce(const uint8_t *const *streams,
                               const uint64_t *lens, uint32_t S, uint64_t N,
                               uint32_t C, uint16_t *out);

#ifdef __cplusplus
}
#endif
#endif
