/*
 * uzip_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * split-exponent lossless BF16 codec.
 *
 * THIS IS TEST INFRASTRUCTURE. Only the test suite, the package's smoke check
 * and the benchmark's CPU-baseline leg may load it. The product path (the HIP
 * library) never calls, links or includes anything from this directory, and
 * this file includes nothing from the product.
 *
 * Sources (web pages; cited by title and section):
 *   [SZ]  "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
 *         Serving" (xllm-io paper review), section 3.2 (split/merge formulas,
 *         4-bit Top-16 codes two per byte, escapes as a 16-bit in-chunk position
 *         plus the raw 8-bit exponent, size B = N + N/2 + 3M), section 3.3
 *         (offline calibration: histogram, Top-16, three lookup tables),
 *         section 3.4 (all 16 codes are real exponents; escapes carry a dummy
 *         code and are overwritten from the position list), section 4.3
 *         Table 3 (Top-8 3-bit codes; the Top-8 section below).
 *   [UZ]  "UCCL-Zip: Lossless Compression Supercharged GPU Communication",
 *         section 3.4 / Figure 6: a receiver decompresses a slice, reduces it
 *         with its own slice, and recompresses the result; section 5.2 /
 *         Figure 9: two-shot all-reduce, whose reduce-scatter phase
 *         decompresses every received chunk before reducing it.
 *   [ZC]  "ZipCCL: Efficient Lossless Data Compression of Communication
 *         Collectives", adaptive communication strategies: a zipped
 *         all-to-all followed by a local reduction; exponent coding: the top
 *         7 exponents as 3-bit codes, code 000 a zero-point whose exponent
 *         is stored whole in a separate array (the Top-7 section below).
 *
 * Readings where the pages leave a point open (each is the plainest reading;
 * the same list stands in the design notes):
 *   - code k is the k-th most frequent exponent, ties to the smaller exponent;
 *     fewer than 16 non-zero bins are filled with zero-count exponents in
 *     ascending order;
 *   - the dummy code of an escape is 0;
 *   - element 2j sits in the low nibble of code byte j, 2j+1 in the high one;
 *     an odd N leaves the last high nibble 0;
 *   - escapes are stored as two arrays (all u16 positions, then all u8 raw
 *     exponents), chunk by chunk, ascending position inside a chunk, with a
 *     u32 exclusive offset per chunk plus the total at the end;
 *   - stream = 256-byte header, then the sign-mantissa, code, offset, position
 *     and value sections, each starting at a multiple of 256 bytes, padding 0;
 *   - reduce: one IEEE binary32 add of the two decoded values (round to
 *     nearest even, subnormals kept), then round-half-to-even to BF16; a NaN
 *     sum becomes 0x7FC0 (this last choice is ours: parity unpinned by the
 *     pages);
 *   - k-input reduce: the k values are added in binary32 in input order, one
 *     rounding per add, and the sum is rounded once to BF16 (the pages name
 *     the operation, a local reduction of received chunks, but not its
 *     arithmetic; this is the plainest reading that agrees with the
 *     two-input case).
 *
 * Everything here is scalar C on 16-bit words; floats appear only in the
 * reduce's binary32 add. Build: gcc -O2 -std=c99 -ffp-contract=off (no
 * -ffast-math: the add must be IEEE).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define ORC_HEADER 256u

/* ---------------------------------------------------------------- split -- */
/* [SZ] section 3.2: exponent e = (x >> 7) & 0xff, sign-mantissa byte
 * a = ((x >> 8) & 0x80) | (x & 0x7f). */
uint8_t orc_exponent(uint16_t x) { return (uint8_t)((x >> 7) & 0xffu); }
uint8_t orc_signmant(uint16_t x) { return (uint8_t)(((x >> 8) & 0x80u) | (x & 0x7fu)); }

/* [SZ] section 3.2: x = ((a & 0x80) << 8) | (e << 7) | (a & 0x7f). */
uint16_t orc_merge(uint8_t a, uint8_t e)
{
    return (uint16_t)((((unsigned)a & 0x80u) << 8) | ((unsigned)e << 7) | ((unsigned)a & 0x7fu));
}

/* ------------------------------------------------------------ histogram -- */
/* [SZ] section 3.3: count every exponent of the calibration set. Adds into
 * hist (the caller zeroes it), so two sets can be pooled. */
void orc_histogram(const uint16_t *x, uint64_t n, uint64_t *hist)
{
    for (uint64_t i = 0; i < n; i++)
        hist[orc_exponent(x[i])] += 1;
}

/* --------------------------------------------------------------- Top-16 -- */
/* [SZ] section 3.3: pick the 16 most frequent exponents and build the three
 * tables. Order: count descending, then exponent ascending, over all 256
 * values (zero counts included). Plain selection: 16 rounds, each taking the
 * best exponent not yet taken. */
void orc_top16(const uint64_t *hist, uint8_t *dec, uint8_t *enc, uint8_t *member)
{
    int taken[256];
    for (int e = 0; e < 256; e++) { taken[e] = 0; enc[e] = 0; member[e] = 0; }
    for (int k = 0; k < 16; k++) {
        int best = -1;
        for (int e = 0; e < 256; e++) {
            if (taken[e]) continue;
            if (best < 0 || hist[e] > hist[best]) best = e;   /* strict: ties keep smaller e */
        }
        taken[best] = 1;
        dec[k] = (uint8_t)best;
        enc[best] = (uint8_t)k;
        member[best] = 1;
    }
}

/* code of exponent e under dec[], or -1 if e is not in the codebook
 * (linear search: independent of any lookup table). */
static int orc_code_of(const uint8_t *dec, uint8_t e)
{
    for (int k = 0; k < 16; k++)
        if (dec[k] == e) return k;
    return -1;
}

/* ---------------------------------------------------------------- sizes -- */
static uint64_t orc_align(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

typedef struct {
    uint64_t sm, codes, offs, pos, val, total;
} orc_layout;

static uint64_t orc_nchunks(uint64_t n, uint32_t C) { return (n + C - 1) / C; }

static orc_layout orc_layout_of(uint64_t n, uint32_t C, uint64_t m)
{
    orc_layout L;
    uint64_t nch = orc_nchunks(n, C);
    L.sm = ORC_HEADER;
    L.codes = L.sm + orc_align(n);
    L.offs = L.codes + orc_align((n + 1) / 2);
    L.pos = L.offs + orc_align(4 * (nch + 1));
    L.val = L.pos + orc_align(2 * m);
    L.total = L.val + m;
    return L;
}

/* Worst-case stream size: every element an escape. */
uint64_t orc_max_bytes(uint64_t n, uint32_t C)
{
    if (n == 0 || C == 0) return 0;
    return orc_layout_of(n, C, n).total;
}

/* [SZ] section 3.2: payload bytes N + N/2 + 3M (N/2 rounded up for odd N). */
uint64_t orc_payload_bytes(uint64_t n, uint64_t m) { return n + (n + 1) / 2 + 3 * m; }

static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) { uint32_t v = 0; for (int i = 3; i >= 0; i--) v = (v << 8) | p[i]; return v; }
static uint64_t get_u64(const uint8_t *p) { uint64_t v = 0; for (int i = 7; i >= 0; i--) v = (v << 8) | p[i]; return v; }

/* --------------------------------------------------------------- encode -- */
/* [SZ] section 3.2, the two encode stages in the page's order:
 *  (1) dense transform: keep every sign-mantissa byte, look each exponent up
 *      in the codebook and pack two 4-bit codes per byte (escapes: dummy 0);
 *  (2) scan the raw exponents chunk by chunk and append every exponent that
 *      is not in the codebook to the escape arrays (in-chunk position, raw
 *      exponent).
 * Returns the stream size, or 0 if an argument is bad or cap is too small
 * for the worst case. */
uint64_t orc_encode(const uint16_t *x, uint64_t n, uint32_t C, const uint8_t *dec,
                    uint8_t *out, uint64_t cap)
{
    if (n == 0 || C == 0 || C > 65536u || n >= ((uint64_t)1 << 32)) return 0;
    if (cap < orc_max_bytes(n, C)) return 0;

    /* count escapes first so the section offsets are known */
    uint64_t m = 0;
    for (uint64_t i = 0; i < n; i++)
        if (orc_code_of(dec, orc_exponent(x[i])) < 0) m++;
    orc_layout L = orc_layout_of(n, C, m);
    memset(out, 0, L.total);

    /* stage (1): dense sections */
    for (uint64_t i = 0; i < n; i++) {
        out[L.sm + i] = orc_signmant(x[i]);
        int k = orc_code_of(dec, orc_exponent(x[i]));
        unsigned code = (k < 0) ? 0u : (unsigned)k;
        if (i % 2 == 0) out[L.codes + i / 2] |= (uint8_t)code;
        else            out[L.codes + i / 2] |= (uint8_t)(code << 4);
    }

    /* stage (2): escapes, chunk by chunk, ascending position */
    uint64_t nch = orc_nchunks(n, C);
    uint64_t j = 0;
    for (uint64_t c = 0; c < nch; c++) {
        put_u32(out + L.offs + 4 * c, (uint32_t)j);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t e = orc_exponent(x[i]);
            if (orc_code_of(dec, e) < 0) {
                put_u16(out + L.pos + 2 * j, (uint16_t)(i - lo));
                out[L.val + j] = e;
                j++;
            }
        }
    }
    put_u32(out + L.offs + 4 * nch, (uint32_t)j);

    /* header */
    out[0] = 0x55; out[1] = 0x5A; out[2] = 0x42; out[3] = 0x31;   /* "UZB1" */
    put_u16(out + 4, 1);
    put_u16(out + 6, 0);
    put_u32(out + 8, C);
    put_u32(out + 12, 0);
    put_u64(out + 16, n);
    put_u64(out + 24, m);
    put_u64(out + 32, L.total);
    memcpy(out + 40, dec, 16);
    return L.total;
}

/* --------------------------------------------------------------- decode -- */
/* [SZ] section 3.2: unpack both nibbles of every code byte, look the code up
 * in the 16-entry table and rebuild each word with its sign-mantissa byte;
 * then overwrite each escape's exponent with the recorded raw exponent.
 * Returns 0, or -1 on a bad argument or a stream that does not match. */
int orc_decode(const uint8_t *in, uint64_t in_bytes, uint64_t n, uint32_t C,
               const uint8_t *dec, uint16_t *y)
{
    if (in_bytes < ORC_HEADER || n == 0 || C == 0) return -1;
    if (get_u64(in + 16) != n || get_u32(in + 8) != C) return -1;
    if (memcmp(in + 40, dec, 16) != 0) return -1;
    uint64_t m = get_u64(in + 24);
    orc_layout L = orc_layout_of(n, C, m);
    if (in_bytes < L.total) return -1;

    for (uint64_t i = 0; i < n; i++) {
        uint8_t byte = in[L.codes + i / 2];
        unsigned code = (i % 2 == 0) ? (byte & 0x0fu) : (byte >> 4);
        y[i] = orc_merge(in[L.sm + i], dec[code]);
    }
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        if (j1 < j0 || j1 > m) return -1;
        for (uint32_t j = j0; j < j1; j++) {
            uint64_t i = c * C + get_u16(in + L.pos + 2 * (uint64_t)j);
            if (i >= n) return -1;
            y[i] = orc_merge(in[L.sm + i], in[L.val + j]);
        }
    }
    return 0;
}

/* --------------------------------------------------------------- reduce -- */
/* BF16 word -> binary32: the 16 bits become the high half. */
static float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 bits -> BF16, round half to even on the 16 dropped bits.
 * NaN -> 0x7FC0. A carry out of the mantissa moves into the exponent, which
 * turns the largest finite values into infinity when they round up. */
uint16_t orc_bf16_rne(uint32_t u)
{
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) return 0x7FC0;
    uint32_t hi = u >> 16, lo = u & 0xffffu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;
    return (uint16_t)hi;
}

/* One element of the reduce: binary32 sum of the two values, then BF16. */
uint16_t orc_add_bf16(uint16_t a, uint16_t b)
{
    volatile float s = orc_bf16_to_f32(a) + orc_bf16_to_f32(b);
    float sv = s;
    uint32_t u;
    memcpy(&u, &sv, 4);
    return orc_bf16_rne(u);
}

/* [UZ] section 3.4: decode both compressed inputs, add element-wise, and
 * encode the result with the same codebook and chunk size. tmp must hold 3n
 * words of scratch. Returns the output stream size or 0. */
uint64_t orc_reduce_add(const uint8_t *a, uint64_t a_bytes, const uint8_t *b, uint64_t b_bytes,
                        uint64_t n, uint32_t C, const uint8_t *dec,
                        uint8_t *out, uint64_t cap, uint16_t *tmp)
{
    uint16_t *ya = tmp, *yb = tmp + n, *r = tmp + 2 * n;
    if (orc_decode(a, a_bytes, n, C, dec, ya) != 0) return 0;
    if (orc_decode(b, b_bytes, n, C, dec, yb) != 0) return 0;
    for (uint64_t i = 0; i < n; i++) r[i] = orc_add_bf16(ya[i], yb[i]);
    return orc_encode(r, n, C, dec, out, cap);
}

/* One element of the k-input reduce: the k values added in binary32 in
 * input order (the first value is the starting sum; k - 1 IEEE adds, each
 * rounded to nearest even), then rounded once to BF16. v[i * stride] is the
 * element of input i. */
uint16_t orc_sum_bf16(const uint16_t *v, uint32_t k, uint64_t stride)
{
    volatile float s = orc_bf16_to_f32(v[0]);
    for (uint32_t i = 1; i < k; i++) s = s + orc_bf16_to_f32(v[(uint64_t)i * stride]);
    float sv = s;
    uint32_t u;
    memcpy(&u, &sv, 4);
    return orc_bf16_rne(u);
}

/* The k-input reduce: the local step of one GPU after a compressed exchange
 * ([ZC], adaptive communication strategies: a zipped all-to-all followed by
 * a local reduction; [UZ] section 5.2, Figure 9: in the reduce-scatter phase
 * of a two-shot all-reduce each received chunk is decompressed before it is
 * reduced). Decode the k inputs, sum each element as orc_sum_bf16 does, and
 * encode the sums with the same codebook and chunk size. k = 2 is
 * orc_reduce_add; k = 1 re-encodes the input with every NaN made 0x7FC0.
 * tmp must hold (k + 1) n words. Returns the output stream size or 0. */
uint64_t orc_reduce_k(const uint8_t *const *in, const uint64_t *in_bytes, uint32_t k,
                      uint64_t n, uint32_t C, const uint8_t *dec,
                      uint8_t *out, uint64_t cap, uint16_t *tmp)
{
    if (k == 0) return 0;
    for (uint32_t i = 0; i < k; i++)
        if (orc_decode(in[i], in_bytes[i], n, C, dec, tmp + (uint64_t)i * n) != 0) return 0;
    uint16_t *r = tmp + (uint64_t)k * n;
    for (uint64_t e = 0; e < n; e++) r[e] = orc_sum_bf16(tmp + e, k, n);
    return orc_encode(r, n, C, dec, out, cap);
}

/* ------------------------------------------------------------- validate -- */
/* Full structural check of a stream against the caller's codebook.
 * 0 = ok, -3 = malformed, -4 = codebook differs. */
int orc_validate(const uint8_t *in, uint64_t in_bytes, const uint8_t *dec)
{
    if (in_bytes < ORC_HEADER) return -3;
    if (!(in[0] == 0x55 && in[1] == 0x5A && in[2] == 0x42 && in[3] == 0x31)) return -3;
    if (get_u16(in + 4) != 1 || get_u16(in + 6) != 0 || get_u32(in + 12) != 0) return -3;
    uint32_t C = get_u32(in + 8);
    uint64_t n = get_u64(in + 16), m = get_u64(in + 24), total = get_u64(in + 32);
    if (C == 0 || C > 65536u || n == 0 || n >= ((uint64_t)1 << 32) || m > n) return -3;
    for (int i = 56; i < 256; i++) if (in[i] != 0) return -3;
    orc_layout L = orc_layout_of(n, C, m);
    if (total != L.total || in_bytes < L.total) return -3;
    if (memcmp(in + 40, dec, 16) != 0) return -4;
    /* codebook entries must be 16 distinct exponents */
    for (int k = 0; k < 16; k++)
        for (int q = k + 1; q < 16; q++)
            if (dec[k] == dec[q]) return -3;
    /* padding bytes are zero */
    for (uint64_t p = L.sm + n; p < L.codes; p++) if (in[p]) return -3;
    if (n % 2 == 1 && (in[L.codes + n / 2] >> 4) != 0) return -3;
    for (uint64_t p = L.codes + (n + 1) / 2; p < L.offs; p++) if (in[p]) return -3;
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t p = L.offs + 4 * (nch + 1); p < L.pos; p++) if (in[p]) return -3;
    for (uint64_t p = L.pos + 2 * m; p < L.val; p++) if (in[p]) return -3;
    /* offsets: start at 0, never decrease, end at m, fit their chunk */
    if (get_u32(in + L.offs) != 0 || get_u32(in + L.offs + 4 * nch) != m) return -3;
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        uint64_t len = (c + 1) * C <= n ? C : n - c * C;
        if (j1 < j0 || (uint64_t)(j1 - j0) > len) return -3;
        for (uint32_t j = j0; j < j1; j++) {
            uint16_t p = get_u16(in + L.pos + 2 * (uint64_t)j);
            if (p >= len) return -3;
            if (j > j0 && p <= get_u16(in + L.pos + 2 * (uint64_t)(j - 1))) return -3;
            if (orc_code_of(dec, in[L.val + j]) >= 0) return -3;   /* escape must be outside the codebook */
            uint64_t i = c * C + p;
            uint8_t byte = in[L.codes + i / 2];
            unsigned code = (i % 2 == 0) ? (byte & 0x0fu) : (byte >> 4);
            if (code != 0) return -3;                               /* dummy code is 0 */
        }
    }
    return 0;
}

/* Header reads, for tests. */
uint64_t orc_stream_m(const uint8_t *in) { return get_u64(in + 24); }
uint64_t orc_stream_total(const uint8_t *in) { return get_u64(in + 32); }

/* Array forms of the reduce arithmetic, for sweeps in the tests. */
void orc_bf16_rne_array(const uint32_t *u, uint64_t n, uint16_t *out)
{
    for (uint64_t i = 0; i < n; i++) out[i] = orc_bf16_rne(u[i]);
}

void orc_add_bf16_array(const uint16_t *a, const uint16_t *b, uint64_t n, uint16_t *r)
{
    for (uint64_t i = 0; i < n; i++) r[i] = orc_add_bf16(a[i], b[i]);
}

/* v holds k rows of n words; r[e] = orc_sum_bf16 of column e. */
void orc_sum_bf16_array(const uint16_t *v, uint32_t k, uint64_t n, uint16_t *r)
{
    for (uint64_t e = 0; e < n; e++) r[e] = orc_sum_bf16(v + e, k, n);
}

/* ==================================================== FP8 E5M2 variant === */
/* [SZ] section 4.2 / appendix C: E5M2 values (1 sign bit, 5 exponent bits,
 * 2 mantissa bits) in the same framework: each 5-bit exponent becomes a
 * 4-bit Top-16 code, the other 3 bits are kept, and an exponent outside the
 * codebook is an escape of 3 bytes (u16 in-chunk position, u8 raw exponent).
 * Readings (the page gives the framework and its numbers, not the layout):
 *   - the kept 3 bits are sign | mantissa, a = ((x >> 5) & 4) | (x & 3);
 *   - they are packed 3 bits per value, value i at bits 3i..3i+2 of the
 *     section, bit b of the section being bit b % 8 of byte b / 8 (so every
 *     8 values fill 3 bytes); unused bits of the last byte are 0;
 *   - codes, escape arrays, offsets and container are the BF16 ones, with
 *     header flags = 1 for the element type and the sign-mantissa section
 *     ceil(3N/8) bytes long;
 *   - payload = ceil(3N/8) + ceil(N/2) + 3M bytes, so the ratio is
 *     N / payload -> 8/7 with no escape (the page's 1.14x at 0.16 %). */
uint8_t orc8_exponent(uint8_t x) { return (uint8_t)((x >> 2) & 0x1fu); }
uint8_t orc8_signmant(uint8_t x) { return (uint8_t)(((x >> 5) & 0x4u) | (x & 0x3u)); }
uint8_t orc8_merge(uint8_t a, uint8_t e)
{
    return (uint8_t)((((unsigned)a & 0x4u) << 5) | (((unsigned)e & 0x1fu) << 2) | ((unsigned)a & 0x3u));
}

void orc8_histogram(const uint8_t *x, uint64_t n, uint64_t *hist)
{
    for (uint64_t i = 0; i < n; i++)
        hist[orc8_exponent(x[i])] += 1;
}

static uint64_t orc8_sm_bytes(uint64_t n) { return (3 * n + 7) / 8; }

static orc_layout orc8_layout_of(uint64_t n, uint32_t C, uint64_t m)
{
    orc_layout L;
    uint64_t nch = orc_nchunks(n, C);
    L.sm = ORC_HEADER;
    L.codes = L.sm + orc_align(orc8_sm_bytes(n));
    L.offs = L.codes + orc_align((n + 1) / 2);
    L.pos = L.offs + orc_align(4 * (nch + 1));
    L.val = L.pos + orc_align(2 * m);
    L.total = L.val + m;
    return L;
}

uint64_t orc8_max_bytes(uint64_t n, uint32_t C)
{
    if (n == 0 || C == 0) return 0;
    return orc8_layout_of(n, C, n).total;
}

uint64_t orc8_payload_bytes(uint64_t n, uint64_t m) { return orc8_sm_bytes(n) + (n + 1) / 2 + 3 * m; }

/* 3-bit field i of a sign-mantissa section, bit by bit. */
static void orc8_put3(uint8_t *sec, uint64_t i, unsigned v)
{
    for (unsigned k = 0; k < 3; k++) {
        uint64_t b = 3 * i + k;
        if ((v >> k) & 1u) sec[b / 8] |= (uint8_t)(1u << (b % 8));
    }
}

static unsigned orc8_get3(const uint8_t *sec, uint64_t i)
{
    unsigned v = 0;
    for (unsigned k = 0; k < 3; k++) {
        uint64_t b = 3 * i + k;
        v |= (unsigned)((sec[b / 8] >> (b % 8)) & 1u) << k;
    }
    return v;
}

/* The two encode stages of [SZ] section 3.2 on E5M2 values. Returns the
 * stream size, or 0 on a bad argument or too small a buffer. */
uint64_t orc8_encode(const uint8_t *x, uint64_t n, uint32_t C, const uint8_t *dec, uint8_t *out, uint64_t cap)
{
    if (n == 0 || C == 0 || C > 65536u || n >= ((uint64_t)1 << 32)) return 0;
    if (cap < orc8_max_bytes(n, C)) return 0;
    uint64_t m = 0;
    for (uint64_t i = 0; i < n; i++)
        if (orc_code_of(dec, orc8_exponent(x[i])) < 0) m++;
    orc_layout L = orc8_layout_of(n, C, m);
    memset(out, 0, L.total);
    for (uint64_t i = 0; i < n; i++) {
        orc8_put3(out + L.sm, i, orc8_signmant(x[i]));
        int k = orc_code_of(dec, orc8_exponent(x[i]));
        unsigned code = (k < 0) ? 0u : (unsigned)k;
        if (i % 2 == 0) out[L.codes + i / 2] |= (uint8_t)code;
        else            out[L.codes + i / 2] |= (uint8_t)(code << 4);
    }
    uint64_t nch = orc_nchunks(n, C);
    uint64_t j = 0;
    for (uint64_t c = 0; c < nch; c++) {
        put_u32(out + L.offs + 4 * c, (uint32_t)j);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t e = orc8_exponent(x[i]);
            if (orc_code_of(dec, e) < 0) {
                put_u16(out + L.pos + 2 * j, (uint16_t)(i - lo));
                out[L.val + j] = e;
                j++;
            }
        }
    }
    put_u32(out + L.offs + 4 * nch, (uint32_t)j);
    out[0] = 0x55; out[1] = 0x5A; out[2] = 0x42; out[3] = 0x31;
    put_u16(out + 4, 1);
    put_u16(out + 6, 1);                         /* element type: FP8 E5M2 */
    put_u32(out + 8, C);
    put_u32(out + 12, 0);
    put_u64(out + 16, n);
    put_u64(out + 24, m);
    put_u64(out + 32, L.total);
    memcpy(out + 40, dec, 16);
    return L.total;
}

/* Decode of an E5M2 stream: codes through dec[], merged with the 3 kept
 * bits, then the escape patch. Returns 0 or -1. */
int orc8_decode(const uint8_t *in, uint64_t in_bytes, uint64_t n, uint32_t C, const uint8_t *dec, uint8_t *y)
{
    if (in_bytes < ORC_HEADER || n == 0 || C == 0) return -1;
    if (get_u64(in + 16) != n || get_u32(in + 8) != C || get_u16(in + 6) != 1) return -1;
    if (memcmp(in + 40, dec, 16) != 0) return -1;
    uint64_t m = get_u64(in + 24);
    orc_layout L = orc8_layout_of(n, C, m);
    if (in_bytes < L.total) return -1;
    for (uint64_t i = 0; i < n; i++) {
        uint8_t byte = in[L.codes + i / 2];
        unsigned code = (i % 2 == 0) ? (byte & 0x0fu) : (byte >> 4);
        y[i] = orc8_merge((uint8_t)orc8_get3(in + L.sm, i), dec[code]);
    }
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        if (j1 < j0 || j1 > m) return -1;
        for (uint32_t j = j0; j < j1; j++) {
            uint64_t i = c * C + get_u16(in + L.pos + 2 * (uint64_t)j);
            if (i >= n) return -1;
            y[i] = orc8_merge((uint8_t)orc8_get3(in + L.sm, i), in[L.val + j]);
        }
    }
    return 0;
}

/* Structural check of an E5M2 stream: the BF16 rules, with flags = 1, the
 * shorter sign-mantissa section (its unused last bits 0) and every escape
 * value a 5-bit exponent. */
int orc8_validate(const uint8_t *in, uint64_t in_bytes, const uint8_t *dec)
{
    if (in_bytes < ORC_HEADER) return -3;
    if (!(in[0] == 0x55 && in[1] == 0x5A && in[2] == 0x42 && in[3] == 0x31)) return -3;
    if (get_u16(in + 4) != 1 || get_u16(in + 6) != 1 || get_u32(in + 12) != 0) return -3;
    uint32_t C = get_u32(in + 8);
    uint64_t n = get_u64(in + 16), m = get_u64(in + 24), total = get_u64(in + 32);
    if (C == 0 || C > 65536u || n == 0 || n >= ((uint64_t)1 << 32) || m > n) return -3;
    for (int i = 56; i < 256; i++) if (in[i] != 0) return -3;
    orc_layout L = orc8_layout_of(n, C, m);
    if (total != L.total || in_bytes < L.total) return -3;
    if (memcmp(in + 40, dec, 16) != 0) return -4;
    for (int k = 0; k < 16; k++)
        for (int q = k + 1; q < 16; q++)
            if (dec[k] == dec[q]) return -3;
    for (uint64_t b = 3 * n; b < 8 * orc8_sm_bytes(n); b++)
        if ((in[L.sm + b / 8] >> (b % 8)) & 1u) return -3;
    for (uint64_t p = L.sm + orc8_sm_bytes(n); p < L.codes; p++) if (in[p]) return -3;
    if (n % 2 == 1 && (in[L.codes + n / 2] >> 4) != 0) return -3;
    for (uint64_t p = L.codes + (n + 1) / 2; p < L.offs; p++) if (in[p]) return -3;
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t p = L.offs + 4 * (nch + 1); p < L.pos; p++) if (in[p]) return -3;
    for (uint64_t p = L.pos + 2 * m; p < L.val; p++) if (in[p]) return -3;
    if (get_u32(in + L.offs) != 0 || get_u32(in + L.offs + 4 * nch) != m) return -3;
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        uint64_t len = (c + 1) * C <= n ? C : n - c * C;
        if (j1 < j0 || (uint64_t)(j1 - j0) > len) return -3;
        for (uint32_t j = j0; j < j1; j++) {
            uint16_t p = get_u16(in + L.pos + 2 * (uint64_t)j);
            if (p >= len) return -3;
            if (j > j0 && p <= get_u16(in + L.pos + 2 * (uint64_t)(j - 1))) return -3;
            if (in[L.val + j] > 0x1f) return -3;                     /* a 5-bit exponent */
            if (orc_code_of(dec, in[L.val + j]) >= 0) return -3;
            uint64_t i = c * C + p;
            uint8_t byte = in[L.codes + i / 2];
            unsigned code = (i % 2 == 0) ? (byte & 0x0fu) : (byte >> 4);
            if (code != 0) return -3;
        }
    }
    return 0;
}

/* =========================================== Top-15 + sentinel format === */
/* [SZ] section 3.4 / Table 6, the alternative the page weighs against
 * Top-16: one codeword is an explicit escape token, so the decoder finds the
 * escapes in the code stream and no positions are stored. Readings:
 *   - codes 0..14 are the 15 most frequent exponents (dec[0..14] of the
 *     Top-16 ranking); code 15 marks an escape; dec[15] is not used;
 *   - each chunk's escapes are stored as their raw exponents (u8), in
 *     ascending position, chunk after chunk, with the u32 chunk offsets;
 *   - the container is the BF16 one with header flags = 2 and no position
 *     section: header | sm | codes | offsets | val;
 *   - payload = N + ceil(N/2) + M bytes. */
static int orcs_code_of(const uint8_t *dec, uint8_t e)
{
    for (int k = 0; k < 15; k++)
        if (dec[k] == e) return k;
    return -1;
}

static orc_layout orcs_layout_of(uint64_t n, uint32_t C, uint64_t m)
{
    orc_layout L;
    uint64_t nch = orc_nchunks(n, C);
    L.sm = ORC_HEADER;
    L.codes = L.sm + orc_align(n);
    L.offs = L.codes + orc_align((n + 1) / 2);
    L.pos = L.offs + orc_align(4 * (nch + 1));     /* no position section */
    L.val = L.pos;
    L.total = L.val + m;
    return L;
}

uint64_t orcs_max_bytes(uint64_t n, uint32_t C)
{
    if (n == 0 || C == 0) return 0;
    return orcs_layout_of(n, C, n).total;
}

uint64_t orcs_payload_bytes(uint64_t n, uint64_t m) { return n + (n + 1) / 2 + m; }

uint64_t orcs_encode(const uint16_t *x, uint64_t n, uint32_t C, const uint8_t *dec, uint8_t *out, uint64_t cap)
{
    if (n == 0 || C == 0 || C > 65536u || n >= ((uint64_t)1 << 32)) return 0;
    if (cap < orcs_max_bytes(n, C)) return 0;
    uint64_t m = 0;
    for (uint64_t i = 0; i < n; i++)
        if (orcs_code_of(dec, orc_exponent(x[i])) < 0) m++;
    orc_layout L = orcs_layout_of(n, C, m);
    memset(out, 0, L.total);
    for (uint64_t i = 0; i < n; i++) {
        out[L.sm + i] = orc_signmant(x[i]);
        int k = orcs_code_of(dec, orc_exponent(x[i]));
        unsigned code = (k < 0) ? 15u : (unsigned)k;          /* the sentinel */
        if (i % 2 == 0) out[L.codes + i / 2] |= (uint8_t)code;
        else            out[L.codes + i / 2] |= (uint8_t)(code << 4);
    }
    uint64_t nch = orc_nchunks(n, C);
    uint64_t j = 0;
    for (uint64_t c = 0; c < nch; c++) {
        put_u32(out + L.offs + 4 * c, (uint32_t)j);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t e = orc_exponent(x[i]);
            if (orcs_code_of(dec, e) < 0) out[L.val + j++] = e;
        }
    }
    put_u32(out + L.offs + 4 * nch, (uint32_t)j);
    out[0] = 0x55; out[1] = 0x5A; out[2] = 0x42; out[3] = 0x31;
    put_u16(out + 4, 1);
    put_u16(out + 6, 2);                         /* format: Top-15 + sentinel */
    put_u32(out + 8, C);
    put_u32(out + 12, 0);
    put_u64(out + 16, n);
    put_u64(out + 24, m);
    put_u64(out + 32, L.total);
    memcpy(out + 40, dec, 16);
    return L.total;
}

/* Decode: a code below 15 is looked up; a sentinel takes the next raw
 * exponent of its chunk (the chunk's offset plus the sentinels before it in
 * the chunk). Returns 0 or -1. */
int orcs_decode(const uint8_t *in, uint64_t in_bytes, uint64_t n, uint32_t C, const uint8_t *dec, uint16_t *y)
{
    if (in_bytes < ORC_HEADER || n == 0 || C == 0) return -1;
    if (get_u64(in + 16) != n || get_u32(in + 8) != C || get_u16(in + 6) != 2) return -1;
    if (memcmp(in + 40, dec, 16) != 0) return -1;
    uint64_t m = get_u64(in + 24);
    orc_layout L = orcs_layout_of(n, C, m);
    if (in_bytes < L.total) return -1;
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t c = 0; c < nch; c++) {
        uint64_t j = get_u32(in + L.offs + 4 * c);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t byte = in[L.codes + i / 2];
            unsigned code = (i % 2 == 0) ? (byte & 0x0fu) : (byte >> 4);
            if (code < 15) {
                y[i] = orc_merge(in[L.sm + i], dec[code]);
            } else {
                if (j >= m) return -1;
                y[i] = orc_merge(in[L.sm + i], in[L.val + j++]);
            }
        }
        if (j != get_u32(in + L.offs + 4 * (c + 1))) return -1;
    }
    return 0;
}

/* Structural check: header (flags 2), sizes, zero padding, offsets from 0
 * to m, each chunk's sentinel count equal to its offset difference, and
 * every stored exponent outside dec[0..14]. */
int orcs_validate(const uint8_t *in, uint64_t in_bytes, const uint8_t *dec)
{
    if (in_bytes < ORC_HEADER) return -3;
    if (!(in[0] == 0x55 && in[1] == 0x5A && in[2] == 0x42 && in[3] == 0x31)) return -3;
    if (get_u16(in + 4) != 1 || get_u16(in + 6) != 2 || get_u32(in + 12) != 0) return -3;
    uint32_t C = get_u32(in + 8);
    uint64_t n = get_u64(in + 16), m = get_u64(in + 24), total = get_u64(in + 32);
    if (C == 0 || C > 65536u || n == 0 || n >= ((uint64_t)1 << 32) || m > n) return -3;
    for (int i = 56; i < 256; i++) if (in[i] != 0) return -3;
    orc_layout L = orcs_layout_of(n, C, m);
    if (total != L.total || in_bytes < L.total) return -3;
    if (memcmp(in + 40, dec, 16) != 0) return -4;
    for (int k = 0; k < 16; k++)
        for (int q = k + 1; q < 16; q++)
            if (dec[k] == dec[q]) return -3;
    for (uint64_t p = L.sm + n; p < L.codes; p++) if (in[p]) return -3;
    if (n % 2 == 1 && (in[L.codes + n / 2] >> 4) != 0) return -3;
    for (uint64_t p = L.codes + (n + 1) / 2; p < L.offs; p++) if (in[p]) return -3;
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t p = L.offs + 4 * (nch + 1); p < L.val; p++) if (in[p]) return -3;
    if (get_u32(in + L.offs) != 0 || get_u32(in + L.offs + 4 * nch) != m) return -3;
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        uint64_t sentinels = 0;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t byte = in[L.codes + i / 2];
            unsigned code = (i % 2 == 0) ? (byte & 0x0fu) : (byte >> 4);
            if (code == 15) sentinels++;
        }
        if (j1 < j0 || j1 - j0 != sentinels) return -3;
        for (uint32_t j = j0; j < j1; j++)
            if (orcs_code_of(dec, in[L.val + j]) >= 0) return -3;     /* must be an escape */
    }
    return 0;
}

/* ======================================== Top-7 3-bit + zero-point ====== */
/* "ZipCCL: Efficient Lossless Data Compression of Communication
 * Collectives", exponent coding: the exponents among the 7 most frequent
 * take 3-bit codes 001..111; every other exponent takes the zero-point code
 * 000 and is stored whole in a separate zero-point array; 16 bits become 11
 * for most values. The same page's kernel section keeps the 3-bit codes as
 * three separate 1-bit arrays. Readings (the page gives the scheme, not the
 * stream):
 *   - code k + 1 for the k-th most frequent exponent (the Top-16 ranking,
 *     ties to the smaller exponent), k = 0..6; dec[7..15] are not used;
 *   - the codes are stored as three bit planes, one section each: bit b of
 *     value i's code is bit i % 8 of byte i / 8 of plane b;
 *   - the zero-point array holds the raw exponents chunk by chunk in
 *     ascending position, with u32 chunk offsets (no positions);
 *   - stream: header (flags = 3) | sm (N bytes) | plane 0 | plane 1 |
 *     plane 2 (ceil(N/8) bytes each) | offsets | values; payload
 *     N + 3 ceil(N/8) + M, so 16/11 with no zero-points. */
static int orcz_code_of(const uint8_t *dec, uint8_t e)
{
    for (int k = 0; k < 7; k++)
        if (dec[k] == e) return k + 1;
    return 0;
}

static uint64_t orcz_plane_bytes(uint64_t n) { return (n + 7) / 8; }
static unsigned orcz_bit(uint64_t i) { return (unsigned)(i % 8); }  /* least significant bit first */

static orc_layout orcz_layout_of(uint64_t n, uint32_t C, uint64_t m)
{
    orc_layout L;
    uint64_t nch = orc_nchunks(n, C);
    L.sm = ORC_HEADER;
    L.codes = L.sm + orc_align(n);                   /* plane 0; planes 1 and 2 follow */
    L.offs = L.codes + 3 * orc_align(orcz_plane_bytes(n));
    L.pos = L.offs + orc_align(4 * (nch + 1));      /* no position section */
    L.val = L.pos;
    L.total = L.val + m;
    return L;
}

static unsigned orcz_get_code(const uint8_t *in, const orc_layout *L, uint64_t n, uint64_t i)
{
    uint64_t P = orc_align(orcz_plane_bytes(n));
    unsigned code = 0;
    for (int b = 0; b < 3; b++)
        code |= ((in[L->codes + b * P + i / 8] >> orcz_bit(i)) & 1u) << b;
    return code;
}

uint64_t orcz_max_bytes(uint64_t n, uint32_t C)
{
    if (n == 0 || C == 0) return 0;
    return orcz_layout_of(n, C, n).total;
}

uint64_t orcz_payload_bytes(uint64_t n, uint64_t m) { return n + 3 * orcz_plane_bytes(n) + m; }

uint64_t orcz_encode(const uint16_t *x, uint64_t n, uint32_t C, const uint8_t *dec, uint8_t *out, uint64_t cap)
{
    if (n == 0 || C == 0 || C > 65536u || n >= ((uint64_t)1 << 32)) return 0;
    if (cap < orcz_max_bytes(n, C)) return 0;
    uint64_t m = 0;
    for (uint64_t i = 0; i < n; i++)
        if (orcz_code_of(dec, orc_exponent(x[i])) == 0) m++;
    orc_layout L = orcz_layout_of(n, C, m);
    uint64_t P = orc_align(orcz_plane_bytes(n));
    memset(out, 0, L.total);
    for (uint64_t i = 0; i < n; i++) {
        out[L.sm + i] = orc_signmant(x[i]);
        unsigned code = (unsigned)orcz_code_of(dec, orc_exponent(x[i]));
        for (int b = 0; b < 3; b++)
            if ((code >> b) & 1u) out[L.codes + b * P + i / 8] |= (uint8_t)(1u << orcz_bit(i));
    }
    uint64_t nch = orc_nchunks(n, C);
    uint64_t j = 0;
    for (uint64_t c = 0; c < nch; c++) {
        put_u32(out + L.offs + 4 * c, (uint32_t)j);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t e = orc_exponent(x[i]);
            if (orcz_code_of(dec, e) == 0) out[L.val + j++] = e;
        }
    }
    put_u32(out + L.offs + 4 * nch, (uint32_t)j);
    out[0] = 0x55; out[1] = 0x5A; out[2] = 0x42; out[3] = 0x31;
    put_u16(out + 4, 1);
    put_u16(out + 6, 3);                         /* format: Top-7 3-bit + zero-point */
    put_u32(out + 8, C);
    put_u32(out + 12, 0);
    put_u64(out + 16, n);
    put_u64(out + 24, m);
    put_u64(out + 32, L.total);
    memcpy(out + 40, dec, 16);
    return L.total;
}

int orcz_decode(const uint8_t *in, uint64_t in_bytes, uint64_t n, uint32_t C, const uint8_t *dec, uint16_t *y)
{
    if (in_bytes < ORC_HEADER || n == 0 || C == 0) return -1;
    if (get_u64(in + 16) != n || get_u32(in + 8) != C || get_u16(in + 6) != 3) return -1;
    if (memcmp(in + 40, dec, 16) != 0) return -1;
    uint64_t m = get_u64(in + 24);
    orc_layout L = orcz_layout_of(n, C, m);
    if (in_bytes < L.total) return -1;
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t c = 0; c < nch; c++) {
        uint64_t j = get_u32(in + L.offs + 4 * c);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            unsigned code = orcz_get_code(in, &L, n, i);
            if (code != 0) {
                y[i] = orc_merge(in[L.sm + i], dec[code - 1]);
            } else {
                if (j >= m) return -1;
                y[i] = orc_merge(in[L.sm + i], in[L.val + j++]);
            }
        }
        if (j != get_u32(in + L.offs + 4 * (c + 1))) return -1;
    }
    return 0;
}

int orcz_validate(const uint8_t *in, uint64_t in_bytes, const uint8_t *dec)
{
    if (in_bytes < ORC_HEADER) return -3;
    if (!(in[0] == 0x55 && in[1] == 0x5A && in[2] == 0x42 && in[3] == 0x31)) return -3;
    if (get_u16(in + 4) != 1 || get_u16(in + 6) != 3 || get_u32(in + 12) != 0) return -3;
    uint32_t C = get_u32(in + 8);
    uint64_t n = get_u64(in + 16), m = get_u64(in + 24), total = get_u64(in + 32);
    if (C == 0 || C > 65536u || n == 0 || n >= ((uint64_t)1 << 32) || m > n) return -3;
    for (int i = 56; i < 256; i++) if (in[i] != 0) return -3;
    orc_layout L = orcz_layout_of(n, C, m);
    if (total != L.total || in_bytes < L.total) return -3;
    if (memcmp(in + 40, dec, 16) != 0) return -4;
    for (int k = 0; k < 16; k++)
        for (int q = k + 1; q < 16; q++)
            if (dec[k] == dec[q]) return -3;
    for (uint64_t p = L.sm + n; p < L.codes; p++) if (in[p]) return -3;
    uint64_t P = orc_align(orcz_plane_bytes(n));
    for (int b = 0; b < 3; b++) {                    /* bits past n, then padding, are zero */
        const uint8_t *pl = in + L.codes + b * P;
        for (uint64_t i = n; i < 8 * P; i++)
            if ((pl[i / 8] >> (i % 8)) & 1u) return -3;
    }
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t p = L.offs + 4 * (nch + 1); p < L.val; p++) if (in[p]) return -3;
    if (get_u32(in + L.offs) != 0 || get_u32(in + L.offs + 4 * nch) != m) return -3;
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        uint64_t zeros = 0;
        for (uint64_t i = lo; i < hi; i++)
            if (orcz_get_code(in, &L, n, i) == 0) zeros++;
        if (j1 < j0 || j1 - j0 != zeros) return -3;
        for (uint32_t j = j0; j < j1; j++)
            if (orcz_code_of(dec, in[L.val + j]) != 0) return -3;     /* must be outside the top 7 */
    }
    return 0;
}

/* ======================================== Top-8 3-bit with positions ==== */
/* "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
 * Serving", section 4.3, Table 3 (Top-k exponent coding): the Top-16 codec
 * with 3-bit codes for the 8 most frequent exponents instead of 4-bit codes
 * for 16. Readings (the page gives the code width and the numbers, not the
 * stream): code k is dec[k] of the Top-16 ranking for k < 8; an escape is
 * every other exponent, with the dummy code 0 and the same chunked
 * (u16 position, u8 exponent) arrays; the page's 3-bit codes are not
 * byte-aligned, so they are packed back to back: value i's code at bits
 * 3i..3i+2 of the section, least significant bit first (the packing of the
 * E5M2 sign-mantissa bits); header flags = 4; payload N + ceil(3N/8) + 3M. */
static int orct8_code_of(const uint8_t *dec, uint8_t e)
{
    for (int k = 0; k < 8; k++)
        if (dec[k] == e) return k;
    return -1;
}

static orc_layout orct8_layout_of(uint64_t n, uint32_t C, uint64_t m)
{
    orc_layout L;
    uint64_t nch = orc_nchunks(n, C);
    L.sm = ORC_HEADER;
    L.codes = L.sm + orc_align(n);
    L.offs = L.codes + orc_align((3 * n + 7) / 8);
    L.pos = L.offs + orc_align(4 * (nch + 1));
    L.val = L.pos + orc_align(2 * m);
    L.total = L.val + m;
    return L;
}

uint64_t orct8_max_bytes(uint64_t n, uint32_t C)
{
    if (n == 0 || C == 0) return 0;
    return orct8_layout_of(n, C, n).total;
}

uint64_t orct8_payload_bytes(uint64_t n, uint64_t m) { return n + (3 * n + 7) / 8 + 3 * m; }

uint64_t orct8_encode(const uint16_t *x, uint64_t n, uint32_t C, const uint8_t *dec, uint8_t *out, uint64_t cap)
{
    if (n == 0 || C == 0 || C > 65536u || n >= ((uint64_t)1 << 32)) return 0;
    if (cap < orct8_max_bytes(n, C)) return 0;
    uint64_t m = 0;
    for (uint64_t i = 0; i < n; i++)
        if (orct8_code_of(dec, orc_exponent(x[i])) < 0) m++;
    orc_layout L = orct8_layout_of(n, C, m);
    memset(out, 0, L.total);
    /* stage 1: dense sections */
    for (uint64_t i = 0; i < n; i++) {
        out[L.sm + i] = orc_signmant(x[i]);
        int k = orct8_code_of(dec, orc_exponent(x[i]));
        orc8_put3(out + L.codes, i, k < 0 ? 0u : (unsigned)k);
    }
    /* stage 2: escapes chunk by chunk, ascending position */
    uint64_t nch = orc_nchunks(n, C);
    uint64_t j = 0;
    for (uint64_t c = 0; c < nch; c++) {
        put_u32(out + L.offs + 4 * c, (uint32_t)j);
        uint64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        for (uint64_t i = lo; i < hi; i++) {
            uint8_t e = orc_exponent(x[i]);
            if (orct8_code_of(dec, e) < 0) {
                put_u16(out + L.pos + 2 * j, (uint16_t)(i - lo));
                out[L.val + j] = e;
                j++;
            }
        }
    }
    put_u32(out + L.offs + 4 * nch, (uint32_t)j);
    out[0] = 0x55; out[1] = 0x5A; out[2] = 0x42; out[3] = 0x31;
    put_u16(out + 4, 1);
    put_u16(out + 6, 4);                         /* format: Top-8 3-bit with positions */
    put_u32(out + 8, C);
    put_u32(out + 12, 0);
    put_u64(out + 16, n);
    put_u64(out + 24, m);
    put_u64(out + 32, L.total);
    memcpy(out + 40, dec, 16);
    return L.total;
}

int orct8_decode(const uint8_t *in, uint64_t in_bytes, uint64_t n, uint32_t C, const uint8_t *dec, uint16_t *y)
{
    if (in_bytes < ORC_HEADER || n == 0 || C == 0) return -1;
    if (get_u64(in + 16) != n || get_u32(in + 8) != C || get_u16(in + 6) != 4) return -1;
    if (memcmp(in + 40, dec, 16) != 0) return -1;
    uint64_t m = get_u64(in + 24);
    orc_layout L = orct8_layout_of(n, C, m);
    if (in_bytes < L.total) return -1;
    /* dense lookup: escapes first decode to dec[0] */
    for (uint64_t i = 0; i < n; i++) y[i] = orc_merge(in[L.sm + i], dec[orc8_get3(in + L.codes, i)]);
    /* sparse patch */
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        for (uint32_t j = j0; j < j1; j++) {
            uint64_t i = c * C + get_u16(in + L.pos + 2 * j);
            if (i >= n || j >= m) return -1;
            y[i] = orc_merge(in[L.sm + i], in[L.val + j]);
        }
    }
    return 0;
}

int orct8_validate(const uint8_t *in, uint64_t in_bytes, const uint8_t *dec)
{
    if (in_bytes < ORC_HEADER) return -3;
    if (!(in[0] == 0x55 && in[1] == 0x5A && in[2] == 0x42 && in[3] == 0x31)) return -3;
    if (get_u16(in + 4) != 1 || get_u16(in + 6) != 4 || get_u32(in + 12) != 0) return -3;
    uint32_t C = get_u32(in + 8);
    uint64_t n = get_u64(in + 16), m = get_u64(in + 24), total = get_u64(in + 32);
    if (C == 0 || C > 65536u || n == 0 || n >= ((uint64_t)1 << 32) || m > n) return -3;
    for (int i = 56; i < 256; i++) if (in[i] != 0) return -3;
    orc_layout L = orct8_layout_of(n, C, m);
    if (total != L.total || in_bytes < L.total) return -3;
    if (memcmp(in + 40, dec, 16) != 0) return -4;
    for (int k = 0; k < 16; k++)
        for (int q = k + 1; q < 16; q++)
            if (dec[k] == dec[q]) return -3;
    for (uint64_t p = L.sm + n; p < L.codes; p++) if (in[p]) return -3;
    for (uint64_t b = 3 * n; b < 8 * ((3 * n + 7) / 8); b++)
        if ((in[L.codes + b / 8] >> (b % 8)) & 1u) return -3;
    for (uint64_t p = L.codes + (3 * n + 7) / 8; p < L.offs; p++) if (in[p]) return -3;
    uint64_t nch = orc_nchunks(n, C);
    for (uint64_t p = L.offs + 4 * (nch + 1); p < L.pos; p++) if (in[p]) return -3;
    for (uint64_t p = L.pos + 2 * m; p < L.val; p++) if (in[p]) return -3;
    if (get_u32(in + L.offs) != 0 || get_u32(in + L.offs + 4 * nch) != m) return -3;
    for (uint64_t c = 0; c < nch; c++) {
        uint32_t j0 = get_u32(in + L.offs + 4 * c), j1 = get_u32(in + L.offs + 4 * (c + 1));
        uint64_t len = (c + 1) * C <= n ? C : n - c * C;
        if (j1 < j0 || j1 - j0 > len) return -3;
        for (uint32_t j = j0; j < j1; j++) {
            uint32_t p = get_u16(in + L.pos + 2 * j);
            if (p >= len || (j > j0 && p <= get_u16(in + L.pos + 2 * (j - 1)))) return -3;
            if (orct8_code_of(dec, in[L.val + j]) >= 0) return -3;
            if (orc8_get3(in + L.codes, c * C + p) != 0) return -3;
        }
    }
    return 0;
}
