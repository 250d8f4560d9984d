/*
 * zco_fuzz.c -- the CPU oracle under AddressSanitizer and UBSan.
 *
 * Test infrastructure: built and run by tests/test_oracle_sanitized.py with
 * -fsanitize=address,undefined.  Round trips seeded tensors (coded and raw
 * streams), then decodes damaged copies -- every header byte changed, table
 * and region bytes flipped, every truncation of small streams -- from heap
 * buffers of exactly the stream's length, so any read past a buffer, or any
 * undefined arithmetic, stops the run.  Damaged streams may be accepted or
 * rejected; the point is that decoding never misbehaves.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zco.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    /* xorshift64* (Vigna) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (uint32_t)((rng * 0x2545F4914F6CDD1Dull) >> 32);
}

/* Near-Gaussian-looking BF16 data: small exponents around a centre, some
 * zeros, subnormals, Inf/NaN and wide outliers. */
static void fill(uint16_t *x, uint64_t n, unsigned centre, unsigned kind)
{
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t r = next_u32();
        unsigned e = centre + (r % 5) - 2;
        if (kind == 1)
            x[i] = (uint16_t)(r & 0xFFFF); /* uniform patterns */
        else if (kind == 2)
            x[i] = 0;
        else if ((r >> 8) % 100 == 0)
            x[i] = (uint16_t)(r >> 16); /* anything, Inf/NaN included */
        else if ((r >> 8) % 97 == 0)
            x[i] = (uint16_t)((r >> 31) << 15);
        else
            x[i] = (uint16_t)(((r >> 31) << 15) | (e << 7) | ((r >> 9) & 0x7F));
    }
}

static int check_decode(const uint8_t *s, uint64_t len, uint64_t N, uint32_t C, const uint16_t *x)
{
    uint8_t *exact = (uint8_t *)malloc(len ? len : 1);
    uint16_t *y = (uint16_t *)malloc((N ? N : 1) * sizeof(uint16_t));
    memcpy(exact, s, len);
    uint32_t bad = zco_decompress(exact, len, N, C, y);
    int ok = bad == 0 && (N == 0 || memcmp(x, y, N * sizeof(uint16_t)) == 0);
    free(exact);
    free(y);
    return ok;
}

/* decode a damaged copy; the result is not checked, only the behaviour */
static void damaged(const uint8_t *s, uint64_t len, uint64_t N, uint32_t C)
{
    uint8_t *exact = (uint8_t *)malloc(len ? len : 1);
    uint16_t *y = (uint16_t *)malloc((N ? N : 1) * sizeof(uint16_t));
    memcpy(exact, s, len);
    (void)zco_decompress(exact, len, N, C, y);
    free(exact);
    free(y);
}

int main(void)
{
    static const uint64_t sizes[] = {0, 1, 7, 2047, 2048, 2049, 5000, 8192 + 3, 3 * 8192};
    static const uint32_t chunks[] = {2048, 8192};
    long cases = 0, mutants = 0;
    for (unsigned si = 0; si < sizeof sizes / sizeof *sizes; ++si)
        for (unsigned ci = 0; ci < 2; ++ci)
            for (unsigned kind = 0; kind < 3; ++kind)
                for (uint32_t opt = 0; opt <= ZCO_OPT_RAW_FALLBACK; ++opt) {
                    uint64_t N = sizes[si];
                    uint32_t C = chunks[ci];
                    uint16_t *x = (uint16_t *)malloc((N ? N : 1) * sizeof(uint16_t));
                    fill(x, N, 100 + (unsigned)(next_u32() % 40), kind);
                    uint64_t cap = zco_max_stream_bytes(N, C), len = 0;
                    uint8_t *s = (uint8_t *)malloc(cap);
                    if (zco_compress_ex(x, N, C, -1, opt, s, cap, &len) != 0 || len > cap ||
                        !check_decode(s, len, N, C, x)) {
                        fprintf(stderr, "round trip failed: N=%llu C=%u kind=%u opt=%u\n",
                                (unsigned long long)N, C, kind, opt);
                        return 1;
                    }
                    ++cases;
                    /* every header byte through a few values */
                    for (uint64_t b = 0; b < 64 && b < len; ++b)
                        for (unsigned v = 0; v < 4; ++v) {
                            uint8_t *m = (uint8_t *)malloc(len);
                            memcpy(m, s, len);
                            m[b] = (uint8_t)(v == 0 ? m[b] ^ 1 : v == 1 ? 0 : v == 2 ? 0xFF : m[b] + 0x80);
                            damaged(m, len, N, C);
                            free(m);
                            ++mutants;
                        }
                    /* random flips past the header (tables, planes, bytes, escapes) */
                    for (unsigned t = 0; t < 200 && len > 64; ++t) {
                        uint8_t *m = (uint8_t *)malloc(len);
                        memcpy(m, s, len);
                        uint64_t at = 64 + next_u32() % (len - 64);
                        m[at] ^= (uint8_t)(1u << (next_u32() % 8));
                        damaged(m, len, N, C);
                        free(m);
                        ++mutants;
                    }
                    /* truncations (all of them for small streams) */
                    for (uint64_t l = 0; l < len; l += (len < 20000 ? 1 : 97)) {
                        damaged(s, l, N, C);
                        ++mutants;
                    }
                    free(s);
                    free(x);
                }
    /* the fused reduce over mixed coded and raw shards */
    {
        const uint64_t N = 9000;
        const uint32_t C = 2048;
        uint8_t *streams[3];
        uint64_t lens[3];
        uint16_t *x = (uint16_t *)malloc(N * sizeof(uint16_t)), *y = (uint16_t *)malloc(N * sizeof(uint16_t));
        for (int k = 0; k < 3; ++k) {
            fill(x, N, 120, k == 1 ? 1u : 0u);
            uint64_t cap = zco_max_stream_bytes(N, C);
            streams[k] = (uint8_t *)malloc(cap);
            if (zco_compress_ex(x, N, C, -1, ZCO_OPT_RAW_FALLBACK, streams[k], cap, &lens[k]) != 0)
                return 1;
        }
        if (zco_decompress_reduce((const uint8_t *const *)streams, lens, 3, N, C, y) != 0)
            return 1;
        for (int k = 0; k < 3; ++k)
            free(streams[k]);
        free(x);
        free(y);
    }
    printf("ok: %ld round trips, %ld damaged streams decoded\n", cases, mutants);
    return 0;
}
