/*
 * zco.c -- CPU oracle for lossless BF16 exponent coding (stream version 1).
 *
 * TEST INFRASTRUCTURE ONLY: the plain reference the GPU library is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code with the GPU library.  Build it with
 * -O2 -ffp-contract=off and without -ffast-math: every floating-point
 * operation below must be a separately rounded IEEE operation.
 *
 * Source of the method: ZipCCL (SIGCOMM scribe notes), section "Key idea and
 * contribution", first technique ("theoretically grounded exponent coding"):
 *   - the frequent-exponent range comes straight from the tensor's standard
 *     deviation, with no online histogram and no sorting;
 *   - a frequent BF16 exponent is coded in 3 bits instead of 8;
 *   - an infrequent exponent keeps all of its information in a separate
 *     place, so reconstruction is lossless;
 *   - ideally a value shrinks from 16 to about 11 bits (about 31% less data).
 * The same page's "Introduction" gives the data model behind the rule: LLM
 * communication tensors are near-Gaussian or log-normal.
 *
 * Where the page leaves a step open, this file takes the readings listed in
 * the design notes (window width 7 + escape, window from the Gaussian mass
 * argmax, population variance of the finite values, pairwise fp64 sums,
 * bit-plane code groups of 2048 values, escape bytes in code order).
 */
#include "zco.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Window constant.                                                    */
/*                                                                     */
/* For X ~ N(0, var) the 7-binade window [2^a, 2^(a+7)) holds the mass  */
/* g(a) = P(2^a <= |X| < 2^(a+7)).  Moving the window up one binade     */
/* pays off while P(2^(a+7) <= |X| < 2^(a+8)) > P(2^a <= |X| < 2^(a+1)),*/
/* i.e. while 2^a / sigma < u*, where u* solves                         */
/*     Phi(256 u) - Phi(128 u) = Phi(2 u) - Phi(u)                      */
/* (u* = 0.0189773116839826...).  The best integer a is therefore the   */
/* largest a with 2^(a-1) <= u* sigma, i.e. var >= C0 * 4^a with        */
/* C0 = 1 / (4 u*^2) = 694.17765124217978...  The literal is the fp64   */
/* value nearest to that number; oracle/derive_window_constant.py      */
/* recomputes it from the equation above.                               */
/* ------------------------------------------------------------------ */
static const double ZCO_C0 = 0x1.5b16bd46a1a0cp+9;

double zco_c0(void) { return ZCO_C0; }

/* ------------------------------------------------------------------ */
/* BF16 bit fields: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa  */
/* bits.  Exponent 0 holds zeros and subnormals, 255 holds Inf and NaN. */
/* ------------------------------------------------------------------ */
static unsigned bf16_exponent(uint16_t x) { return (x >> 7) & 0xFFu; }
static unsigned bf16_sign(uint16_t x) { return (x >> 15) & 1u; }
static unsigned bf16_mantissa(uint16_t x) { return x & 0x7Fu; }

/* Exact real value of a BF16 pattern. */
static double bf16_value(uint16_t x)
{
    unsigned e = bf16_exponent(x), m = bf16_mantissa(x);
    double mag;
    if (e == 255u)
        mag = (m == 0u) ? INFINITY : NAN;
    else if (e == 0u)
        mag = ldexp((double)m, -126 - 7);          /* 0.m * 2^-126 */
    else
        mag = ldexp((double)(128u + m), (int)e - 127 - 7); /* 1.m * 2^(e-127) */
    return bf16_sign(x) ? -mag : mag;
}

void zco_bf16_to_f64(const uint16_t *x, size_t n, double *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = bf16_value(x[i]);
}

/* ------------------------------------------------------------------ */
/* Pairwise sum: pad to P = 2^ceil(log2 max(n,1)) with +0.0, then       */
/* level[r+1][m] = level[r][2m] + level[r][2m+1] until one value is     */
/* left.  The order is fixed by the indices alone, which makes the sum  */
/* reproducible on any machine that rounds each fp64 add to nearest.    */
/* ------------------------------------------------------------------ */
static double pairwise_in_place(double *buf, size_t P)
{
    while (P > 1) {
        for (size_t m = 0; m < P / 2; ++m)
            buf[m] = buf[2 * m] + buf[2 * m + 1];
        P /= 2;
    }
    return buf[0];
}

static size_t pow2_at_least(size_t n)
{
    size_t P = 1;
    while (P < n)
        P *= 2;
    return P;
}

double zco_pairwise_sum(const double *a, size_t n)
{
    size_t P = pow2_at_least(n);
    double *buf = (double *)calloc(P, sizeof(double));
    if (!buf)
        return NAN;
    memcpy(buf, a, n * sizeof(double));
    double s = pairwise_in_place(buf, P);
    free(buf);
    return s;
}

/* ------------------------------------------------------------------ */
/* Standard deviation of the tensor (the page's only input to the      */
/* window).  Reading: population variance, mean subtracted, over the    */
/* finite values; zeros and subnormals count as values, Inf and NaN are */
/* left out (they would make the statistic NaN).                        */
/*   v_i = value of x_i if finite else +0.0,  q_i = v_i * v_i (exact:   */
/*   an 8-bit significand squared fits in 53 bits)                      */
/*   S1 = PW(v), S2 = PW(q), n = number of finite values                */
/*   mean = S1 / n, var = S2 / n - mean * mean (three rounded ops)      */
/* ------------------------------------------------------------------ */
void zco_sigma(const uint16_t *x, size_t n, double *S1o, double *S2o,
               uint64_t *nfo, double *varo)
{
    size_t P = pow2_at_least(n);
    double *buf = (double *)calloc(P, sizeof(double));
    uint64_t nf = 0;
    double S1 = NAN, S2 = NAN, var = 0.0;
    if (buf) {
        for (size_t i = 0; i < n; ++i) {
            double v = bf16_value(x[i]);
            if (isfinite(v)) {
                buf[i] = v;
                ++nf;
            } else {
                buf[i] = 0.0;
            }
        }
        S1 = pairwise_in_place(buf, P);
        memset(buf, 0, P * sizeof(double));
        for (size_t i = 0; i < n; ++i) {
            double v = bf16_value(x[i]);
            buf[i] = isfinite(v) ? v * v : 0.0;
        }
        S2 = pairwise_in_place(buf, P);
        free(buf);
        if (nf > 0) {
            double d = (double)nf;
            double mean = S1 / d;
            double ex2 = S2 / d;
            double sq = mean * mean;
            var = ex2 - sq;
            if (!(var > 0.0))
                var = 0.0;
        }
    }
    if (S1o) *S1o = S1;
    if (S2o) *S2o = S2;
    if (nfo) *nfo = nf;
    if (varo) *varo = var;
}

/* ------------------------------------------------------------------ */
/* Window rule.  The window is the 7 biased exponents L..L+6, i.e. the  */
/* magnitudes [2^(L-127), 2^(L-120)).  L = 127 + a with a the best      */
/* window under N(0, var) (see ZCO_C0), clamped to 1..248 so that       */
/* exponent 0 (zeros, subnormals) and 255 (Inf, NaN) always escape.     */
/* var = 0 (no finite spread) gives L = 1.                              */
/* ------------------------------------------------------------------ */
int zco_window(double var)
{
    if (!(var > 0.0))
        return 1;
    for (int L = 248; L >= 2; --L)
        if (var >= ldexp(ZCO_C0, 2 * (L - 127)))
            return L;
    return 1;
}

static unsigned code_of(unsigned e, unsigned L)
{
    return (e >= L && e <= L + 6u) ? e - L : ZCO_ESC;
}

/* ------------------------------------------------------------------ */
/* Stream layout, version 1 (all integers little-endian, pads zero):    */
/*   [0, 64)        header                                              */
/*   [64, ...)      chunk table: K+1 u32, entry k = escapes before      */
/*                  chunk k (entry K = E)                               */
/*   then           group table: G u16, entry g = escapes before group  */
/*                  g counted from the start of g's chunk               */
/*   code_off       = A256(64 + 4(K+1) + 2G); 768 bytes per group       */
/*   sm_off         = code_off + 768 G; 2048 bytes per group            */
/*   esc_off        = sm_off + 2048 G; E escape bytes                   */
/*   total          = esc_off + E                                       */
/* with K = ceil(N/C) chunks and G = ceil(N/2048) groups.               */
/*                                                                      */
/* Inside group g a value index r = i - 2048 g splits as                */
/*   r = 512 k + 8 l + j   (k = 0..3, l = 0..63, j = 0..7),            */
/* and its 3-bit code sits at bit p = 16 (j & 1) + 4 (j >> 1) + k of    */
/* the three u32 plane words at code_off + 768 g + 256 b + 4 l,         */
/* b = 0, 1, 2 (bit b of the code in plane b).  The sign+mantissa byte  */
/* (sign in bit 7) of value i is byte sm_off + i.  Escape bytes (the    */
/* full biased exponent of every value whose code is 7) are stored in   */
/* code order: by group, then plane-word index l, then bit p.           */
/* ------------------------------------------------------------------ */
static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
static uint64_t align256(uint64_t x) { return (x + 255u) & ~(uint64_t)255u; }

static uint64_t group_table_off(uint64_t N, uint32_t C)
{
    return ZCO_HEADER_BYTES + 4u * (ceil_div(N, C) + 1u);
}
uint64_t zco_code_off(uint64_t N, uint32_t C)
{
    return align256(group_table_off(N, C) + 2u * ceil_div(N, ZCO_GROUP));
}
uint64_t zco_sm_off(uint64_t N, uint32_t C)
{
    return zco_code_off(N, C) + 768u * ceil_div(N, ZCO_GROUP);
}
uint64_t zco_esc_off(uint64_t N, uint32_t C)
{
    return zco_sm_off(N, C) + 2048u * ceil_div(N, ZCO_GROUP);
}
uint64_t zco_max_stream_bytes(uint64_t N, uint32_t C)
{
    return zco_esc_off(N, C) + N;
}

static int chunk_ok(uint32_t C)
{
    return C >= ZCO_GROUP && (C & (C - 1u)) == 0u;
}

/* Value index of (group g, plane-word index l, bit p). */
static uint64_t index_of(uint64_t g, unsigned l, unsigned p)
{
    unsigned k = p & 3u;
    unsigned j = 2u * ((p >> 2) & 3u) + (p >> 4);
    return ZCO_GROUP * g + 512u * k + 8u * l + j;
}

/* Position of value i: plane-word index l and bit p inside group i/2048. */
static void place_of(uint64_t i, unsigned *l, unsigned *p)
{
    unsigned r = (unsigned)(i % ZCO_GROUP);
    unsigned k = r / 512u, j = r % 8u;
    *l = (r / 8u) % 64u;
    *p = 16u * (j & 1u) + 4u * (j >> 1) + k;
}

static void put_u16(uint8_t *b, uint16_t v) { b[0] = (uint8_t)v; b[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *b, uint32_t v) { for (int t = 0; t < 4; ++t) b[t] = (uint8_t)(v >> (8 * t)); }
static void put_u64(uint8_t *b, uint64_t v) { for (int t = 0; t < 8; ++t) b[t] = (uint8_t)(v >> (8 * t)); }
static uint16_t get_u16(const uint8_t *b) { return (uint16_t)(b[0] | (b[1] << 8)); }
static uint32_t get_u32(const uint8_t *b)
{
    uint32_t v = 0;
    for (int t = 3; t >= 0; --t) v = (v << 8) | b[t];
    return v;
}
static uint64_t get_u64(const uint8_t *b)
{
    uint64_t v = 0;
    for (int t = 7; t >= 0; --t) v = (v << 8) | b[t];
    return v;
}

/* ------------------------------------------------------------------ */
/* Raw streams.  The ZipCCL notes ("Key idea and contribution", third   */
/* technique) switch between the compressed and the native path by the  */
/* compression benefit.  Per stream this reads as: when the coded stream */
/* would be longer than the values themselves, send them as they are.   */
/* A raw stream is the 64-byte header with flags = 1, L = 0, E = 0,      */
/* total = 64 + 2N and the three region offsets 0, followed by the N    */
/* BF16 words, little-endian, from byte 64.  Compression picks it only  */
/* when asked to (ZCO_OPT_RAW_FALLBACK) and only when the coded total is */
/* strictly larger; decoders always accept both kinds.                 */
/* ------------------------------------------------------------------ */
static uint64_t raw_total(uint64_t N) { return ZCO_HEADER_BYTES + 2u * N; }

static void write_raw(const uint16_t *x, uint64_t N, uint32_t C, uint8_t *out)
{
    memset(out, 0, ZCO_HEADER_BYTES);
    put_u32(out + 0, ZCO_MAGIC);
    put_u16(out + 4, ZCO_VERSION);
    out[6] = 0;
    out[7] = ZCO_FLAG_RAW;
    put_u64(out + 8, N);
    put_u32(out + 16, C);
    put_u32(out + 20, (uint32_t)ceil_div(N, C));
    put_u64(out + 24, 0);
    put_u64(out + 32, raw_total(N));
    for (uint64_t i = 0; i < N; ++i)
        put_u16(out + ZCO_HEADER_BYTES + 2u * i, x[i]);
}

int zco_compress(const uint16_t *x, uint64_t N, uint32_t C, int forced_L,
                 uint8_t *out, uint64_t cap, uint64_t *out_len)
{
    return zco_compress_ex(x, N, C, forced_L, 0u, out, cap, out_len);
}

int zco_compress_ex(const uint16_t *x, uint64_t N, uint32_t C, int forced_L,
                    uint32_t options, uint8_t *out, uint64_t cap, uint64_t *out_len)
{
    if (!chunk_ok(C) || (forced_L >= 0 && (forced_L < 1 || forced_L > 248)) ||
        N >= ((uint64_t)1 << 32) || (options & ~ZCO_OPT_RAW_FALLBACK) != 0)
        return -1;

    /* 1. window from the standard deviation, or the forced one */
    unsigned L;
    if (forced_L >= 0) {
        L = (unsigned)forced_L;
    } else {
        double var;
        zco_sigma(x, (size_t)N, NULL, NULL, NULL, &var);
        L = (unsigned)zco_window(var);
    }

    /* 2. size: every value costs a 3-bit code and a byte, escapes a byte more */
    uint64_t E = 0;
    for (uint64_t i = 0; i < N; ++i)
        if (code_of(bf16_exponent(x[i]), L) == ZCO_ESC)
            ++E;
    uint64_t K = ceil_div(N, C), G = ceil_div(N, ZCO_GROUP);
    uint64_t code_off = zco_code_off(N, C), sm_off = zco_sm_off(N, C);
    uint64_t esc_off = zco_esc_off(N, C), total = esc_off + E;
    if ((options & ZCO_OPT_RAW_FALLBACK) && total > raw_total(N)) {
        if (out_len)
            *out_len = raw_total(N);
        if (raw_total(N) > cap)
            return -2;
        write_raw(x, N, C, out);
        return 0;
    }
    if (out_len)
        *out_len = total;
    if (total > cap)
        return -2;
    memset(out, 0, total);

    /* 3. header */
    put_u32(out + 0, ZCO_MAGIC);
    put_u16(out + 4, ZCO_VERSION);
    out[6] = (uint8_t)L;
    out[7] = 0;
    put_u64(out + 8, N);
    put_u32(out + 16, C);
    put_u32(out + 20, (uint32_t)K);
    put_u64(out + 24, E);
    put_u64(out + 32, total);
    put_u64(out + 40, code_off);
    put_u64(out + 48, sm_off);
    put_u64(out + 56, esc_off);

    /* 4. codes into the bit planes, sign+mantissa bytes */
    for (uint64_t i = 0; i < N; ++i) {
        unsigned c = code_of(bf16_exponent(x[i]), L), l, p;
        place_of(i, &l, &p);
        uint64_t g = i / ZCO_GROUP;
        for (unsigned b = 0; b < 3; ++b) {
            if ((c >> b) & 1u) {
                uint8_t *w = out + code_off + 768u * g + 256u * b + 4u * l;
                put_u32(w, get_u32(w) | (1u << p));
            }
        }
        out[sm_off + i] = (uint8_t)((bf16_sign(x[i]) << 7) | bf16_mantissa(x[i]));
    }

    /* 5. escape bytes in code order, chunk table, group table */
    uint64_t groups_per_chunk = C / ZCO_GROUP, pos = 0, chunk_start = 0;
    uint8_t *gtab = out + group_table_off(N, C);
    for (uint64_t g = 0; g < G; ++g) {
        if (g % groups_per_chunk == 0) {
            put_u32(out + ZCO_HEADER_BYTES + 4u * (g / groups_per_chunk), (uint32_t)pos);
            chunk_start = pos;
        }
        put_u16(gtab + 2u * g, (uint16_t)(pos - chunk_start));
        for (unsigned l = 0; l < 64; ++l)
            for (unsigned p = 0; p < 32; ++p) {
                uint64_t i = index_of(g, l, p);
                if (i < N && code_of(bf16_exponent(x[i]), L) == ZCO_ESC)
                    out[esc_off + pos++] = (uint8_t)bf16_exponent(x[i]);
            }
    }
    put_u32(out + ZCO_HEADER_BYTES + 4u * K, (uint32_t)pos);
    return 0;
}

static unsigned code_at(const uint8_t *s, uint64_t code_off, uint64_t i)
{
    unsigned l, p, c = 0;
    place_of(i, &l, &p);
    uint64_t g = i / ZCO_GROUP;
    for (unsigned b = 0; b < 3; ++b)
        c |= ((get_u32(s + code_off + 768u * g + 256u * b + 4u * l) >> p) & 1u) << b;
    return c;
}

/* A raw stream: header fields as write_raw sets them, then the words. */
static uint32_t decompress_raw(const uint8_t *s, uint64_t len, uint64_t N, uint32_t C,
                               uint16_t *out)
{
    uint32_t bad = 0;
    if (get_u32(s) != ZCO_MAGIC || get_u16(s + 4) != ZCO_VERSION)
        bad |= ZCO_FMT_MAGIC;
    if (s[6] != 0)
        bad |= ZCO_FMT_WINDOW;
    if (!chunk_ok(C) || get_u64(s + 8) != N || get_u32(s + 16) != C ||
        get_u32(s + 20) != ceil_div(N, C) || get_u64(s + 40) != 0 ||
        get_u64(s + 48) != 0 || get_u64(s + 56) != 0)
        bad |= ZCO_FMT_SHAPE;
    if (get_u64(s + 24) != 0 || get_u64(s + 32) != raw_total(N) || raw_total(N) > len)
        bad |= ZCO_FMT_SIZE;
    if (bad)
        return bad;
    for (uint64_t i = 0; i < N; ++i)
        out[i] = get_u16(s + ZCO_HEADER_BYTES + 2u * i);
    return 0;
}

uint32_t zco_decompress(const uint8_t *s, uint64_t len, uint64_t N, uint32_t C,
                        uint16_t *out)
{
    if (len < ZCO_HEADER_BYTES)
        return ZCO_FMT_SIZE;

    /* header checks */
    uint32_t bad = 0;
    if (s[7] == ZCO_FLAG_RAW)
        return decompress_raw(s, len, N, C, out);
    if (get_u32(s) != ZCO_MAGIC || get_u16(s + 4) != ZCO_VERSION || s[7] != 0)
        bad |= ZCO_FMT_MAGIC;
    unsigned L = s[6];
    if (L < 1 || L > 248)
        bad |= ZCO_FMT_WINDOW;
    uint64_t K = chunk_ok(C) ? ceil_div(N, C) : 0, G = ceil_div(N, ZCO_GROUP);
    uint64_t code_off = zco_code_off(N, C), sm_off = zco_sm_off(N, C);
    uint64_t esc_off = zco_esc_off(N, C);
    if (!chunk_ok(C) || get_u64(s + 8) != N || get_u32(s + 16) != C ||
        get_u32(s + 20) != K || get_u64(s + 40) != code_off ||
        get_u64(s + 48) != sm_off || get_u64(s + 56) != esc_off)
        bad |= ZCO_FMT_SHAPE;
    uint64_t E = get_u64(s + 24), total = get_u64(s + 32);
    if (E > N || total != esc_off + E || total > len)
        bad |= ZCO_FMT_SIZE;
    if (bad)
        return bad;

    /* chunk table checks */
    const uint8_t *tab = s + ZCO_HEADER_BYTES;
    if (get_u32(tab) != 0 || get_u32(tab + 4u * K) != E)
        bad |= ZCO_FMT_TABLE;
    for (uint64_t k = 0; k < K; ++k)
        if (get_u32(tab + 4u * k) > get_u32(tab + 4u * (k + 1)))
            bad |= ZCO_FMT_TABLE;
    if (bad)
        return bad;

    /* padding past N must be zero */
    for (uint64_t i = N; i < ZCO_GROUP * G; ++i)
        if (code_at(s, code_off, i) != 0 || s[sm_off + i] != 0)
            bad |= ZCO_FMT_PAD;

    /* every chunk's escape count must match its codes, and the group
     * table must hold each group's escape offset inside its chunk */
    uint64_t groups_per_chunk = C / ZCO_GROUP;
    const uint8_t *gtab = s + group_table_off(N, C);
    for (uint64_t k = 0; k < K; ++k) {
        uint64_t cnt = 0;
        for (uint64_t g = k * groups_per_chunk; g < G && g < (k + 1) * groups_per_chunk; ++g) {
            if (get_u16(gtab + 2u * g) != cnt)
                bad |= (g == k * groups_per_chunk) ? ZCO_FMT_TABLE : ZCO_FMT_COUNT;
            for (uint64_t i = g * ZCO_GROUP; i < N && i < (g + 1) * ZCO_GROUP; ++i)
                if (code_at(s, code_off, i) == ZCO_ESC)
                    ++cnt;
        }
        if (cnt != (uint64_t)get_u32(tab + 4u * (k + 1)) - get_u32(tab + 4u * k))
            bad |= ZCO_FMT_COUNT;
    }
    if (bad)
        return bad;

    /* reconstruction: escapes are consumed in code order */
    uint64_t pos = 0;
    for (uint64_t g = 0; g < G; ++g) {
        if (g % groups_per_chunk == 0)
            pos = get_u32(tab + 4u * (g / groups_per_chunk));
        for (unsigned l = 0; l < 64; ++l)
            for (unsigned p = 0; p < 32; ++p) {
                uint64_t i = index_of(g, l, p);
                if (i >= N)
                    continue;
                unsigned c = code_at(s, code_off, i);
                unsigned e = (c < ZCO_ESC) ? L + c : s[esc_off + pos++];
                unsigned sm = s[sm_off + i];
                out[i] = (uint16_t)(((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu));
            }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Round an fp32 value to BF16, nearest, ties to even.  BF16 keeps the  */
/* top 16 bits of the fp32 pattern.  Because the encoding is            */
/* sign-magnitude, the kept half t is the neighbour toward zero and     */
/* t + 1 the neighbour away from zero (a carry into the exponent gives  */
/* the next binade, and past the largest finite value it gives Inf).    */
/* The dropped 16 bits say how far the value is past t, in units of     */
/* 2^-16 of t's spacing; 0x8000 is exactly half way.                    */
/* ------------------------------------------------------------------ */
uint16_t zco_round_bf16(float f)
{
    if (isnan(f))
        return 0x7FC0u;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t t = (uint16_t)(u >> 16);
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (t & 1u)))
        t = (uint16_t)(t + 1u);
    return t;
}

uint32_t zco_decompress_reduce(const uint8_t *const *streams,
                               const uint64_t *lens, uint32_t S, uint64_t N,
                               uint32_t C, uint16_t *out)
{
    uint32_t bad = 0;
    uint16_t *tmp = (uint16_t *)malloc((N ? N : 1) * sizeof(uint16_t));
    float *acc = (float *)malloc((N ? N : 1) * sizeof(float));
    if (!tmp || !acc) {
        free(tmp);
        free(acc);
        return ZCO_FMT_SIZE;
    }
    for (uint32_t sidx = 0; sidx < S; ++sidx) {
        bad |= zco_decompress(streams[sidx], lens[sidx], N, C, tmp);
        for (uint64_t i = 0; i < N; ++i) {
            float v = (float)bf16_value(tmp[i]); /* exact: BF16 is a subset of fp32 */
            acc[i] = (sidx == 0) ? v : acc[i] + v;
        }
    }
    if (S > 0)
        for (uint64_t i = 0; i < N; ++i)
            out[i] = zco_round_bf16(acc[i]);
    free(tmp);
    free(acc);
    return bad;
}
