/*
 * uzip.h -- C-ABI of a lossless split-exponent codec for BF16 tensors on
 * AMD Instinct MI355X (gfx950).
 *
 * The codec (source: "SplitZip: Ultra Fast Lossless KV Compression for
 * Disaggregated LLM Serving", xllm-io paper review, section 3.2):
 * every BF16 word x splits into an exact sign-mantissa byte
 *     a = ((x >> 8) & 0x80) | (x & 0x7f)
 * and an 8-bit exponent
 *     e = (x >> 7) & 0xff.
 * The 16 most frequent exponents of a calibration set (section 3.3) get 4-bit
 * codes, packed two per byte. Any other exponent is an escape. It keeps a
 * dummy code in the dense stream (section 3.4). Its in-chunk position (u16)
 * and raw exponent (u8) go to per-chunk escape arrays. Payload: N + N/2 + 3M
 * bytes for N values and M escapes. Decoding looks up all codes in a 16-entry
 * table, rebuilds the words, then overwrites each escape's exponent.
 *
 * Stream format (all little-endian; A(v) = v rounded up to a multiple of 256):
 *   header   256 bytes:  "UZB1" | u16 version=1 | u16 flags=0 | u32 chunk C |
 *                        u32 0 | u64 n | u64 M | u64 total_bytes | u8 dec[16] |
 *                        zeros to byte 256
 *   sm       at 256                        n bytes       sign-mantissa bytes
 *   codes    at sm + A(n)                  ceil(n/2)     element 2j -> low nibble
 *                                                        of byte j, 2j+1 -> high
 *   offsets  at codes + A(ceil(n/2))       4*(nch+1)     u32 escapes before each
 *                                                        chunk, then M
 *   pos      at offsets + A(4*(nch+1))     2*M           u16 in-chunk positions,
 *                                                        ascending per chunk
 *   val      at pos + A(2*M)               M             u8 raw exponents
 *   total_bytes = offset(val) + M; every padding byte is zero.
 *   nch = ceil(n / C). Escapes carry code 0.
 *
 * The code for exponent rank k (count descending, ties to the smaller
 * exponent) is k.
 *
 * Conventions for every call:
 *   - Device pointers (d_*) are device memory the caller owns. They must be
 *     16-byte aligned. The library allocates no device memory and keeps no
 *     state between calls.
 *   - "async" calls only enqueue work on stream s and return. Their outputs
 *     are valid once s reaches that point. "blocking" calls synchronise s
 *     before returning.
 *   - Arguments are checked on the host before anything is enqueued. A failed
 *     check returns a negative UZIP_E* code and enqueues nothing.
 *   - Calls on different streams may run concurrently when their buffers do
 *     not overlap.
 *   - 1 <= n < 2^32. chunk C is a power of two in [64, 65536].
 */
#ifndef UZIP_H
#define UZIP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UZIP_VERSION 1u

#define UZIP_OK          0
#define UZIP_EINVAL     -1   /* null or misaligned pointer, bad n or chunk */
#define UZIP_ENOSPC     -2   /* output capacity or workspace too small */
#define UZIP_ECORRUPT   -3   /* stream fails a structural check */
#define UZIP_ECODEBOOK  -4   /* stream's dec[16] differs from the codebook */
#define UZIP_EHIP       -5   /* a HIP runtime call or kernel launch failed */
#define UZIP_ESCRATCH   -6   /* input too large for uzip_encode_noalloc's fixed scratch */

/* Codebook: the three tables of the page's offline calibration (section 3.3)
 * and the histogram they came from. Plain data, owned by the caller. It is
 * copied into kernel arguments at each launch.
 *   dec[k]    exponent of code k (k = 0..15)
 *   enc[e]    code of exponent e, 0 when e has no code
 *   member[e] 1 when e has a code, else 0
 */
typedef struct uzip_codebook {
    uint32_t version;          /* UZIP_VERSION */
    uint8_t  dec[16];
    uint8_t  enc[256];
    uint8_t  member[256];
    uint64_t hist[256];
    uint64_t n_cal;            /* sum of hist */
} uzip_codebook_t;

/* Optional per-call settings. A NULL pointer means all defaults.
 *   events/n_events  If not NULL, the call records events[0] before its first
 *                    kernel and events[i] after kernel i (i >= 1), up to
 *                    n_events, all on the call's stream. The caller creates
 *                    the events. Used to time single kernels.
 *   flags            UZIP_F_SEPARATE_PATCH: decode with a dense kernel, then a
 *                    separate sparse patch kernel, instead of the fused
 *                    kernel. The output is the same.
 */
#define UZIP_F_SEPARATE_PATCH 0x1u
typedef struct uzip_opts {
    hipEvent_t *events;
    uint32_t    n_events;
    uint32_t    flags;
} uzip_opts_t;

/* ---------------------------------------------------------- host only -- */

/* Largest stream for n values at chunk C: the format above with M = n.
 * The page's size formula B = N + N/2 + 3M ("SplitZip: Ultra Fast Lossless
 * KV Compression for Disaggregated LLM Serving", section 3.2) is the payload;
 * this adds the header, the chunk offsets and the padding, at the worst case
 * M = n (4.5 bytes per value: the pages define no raw fallback for inputs
 * that expand). M is known only after the encode, so every encode's out_cap
 * must reach this. Returns 0 when n or C is invalid. */
uint64_t uzip_max_bytes(uint64_t n, uint32_t chunk);

/* Device workspace that uzip_encode / uzip_reduce_add / uzip_reduce_k need
 * for (n, C). A format helper with no passage of its own: it is scratch for
 * the escape arrays of section 3.2 (per-tile escape counts and prefixes, and
 * a staging area for each tile's escape list) that lets the library allocate
 * nothing itself. Returns 0 when n or C is invalid. */
uint64_t uzip_workspace_bytes(uint64_t n, uint32_t chunk);

/* Builds the codebook from a 256-bin exponent histogram (page section 3.3).
 * Order: count descending, then exponent ascending, over all 256 values.
 * The first 16 are codes 0..15. Zero-count exponents fill the codebook when
 * fewer than 16 bins are non-zero. Returns UZIP_OK or UZIP_EINVAL (NULL). */
int uzip_codebook_from_hist(const uint64_t hist[256], uzip_codebook_t *cb);

/* Builds the codebook whose decode table is dec[16] (for instance the one a
 * stream's header carries, from uzip_parse_header), enc and member from it,
 * hist and n_cal zero. Enough to decode, validate or reduce that stream.
 * Returns UZIP_OK, or UZIP_EINVAL (NULL, or entries not distinct). */
int uzip_codebook_from_dec(const uint8_t dec[16], uzip_codebook_t *cb);

/* A format helper with no passage of its own: the pages check a bit-exact
 * round trip before they time anything ("SplitZip: Ultra Fast Lossless KV
 * Compression for Disaggregated LLM Serving", section 4.1), and a receiver of
 * an untrusted stream needs the same guarantee without the original tensor.
 * Full structural check of a stream held in host memory (any format: BF16,
 * FP8 E5M2 with header flags 1, Top-15 + sentinel with flags 2, Top-7 +
 * zero-point with flags 3, Top-8 3-bit with flags 4): header fields, section sizes, zero padding,
 * offsets monotone and ending at M, positions ascending and inside their
 * chunk, every escape value outside the codebook with code 0 in the dense
 * stream (for the position-free formats: as many stored values per chunk as
 * sentinels or zero-points, each outside the codes in use). Returns UZIP_OK, UZIP_ECORRUPT,
 * UZIP_ECODEBOOK or UZIP_EINVAL. */
int uzip_validate_host(const void *h_stream, uint64_t bytes, const uzip_codebook_t *cb);

/* Parses a 256-byte header in host memory. Any output pointer may be NULL.
 * Returns UZIP_OK or UZIP_ECORRUPT (bad magic or version). */
int uzip_parse_header(const void *h_header, uint64_t *n, uint32_t *chunk,
                      uint64_t *m, uint64_t *total_bytes, uint8_t dec[16]);

/* Static text for an error code (never NULL). */
const char *uzip_strerror(int code);

/* ------------------------------------------------------------- device -- */

/* async. Adds the exponent histogram of d_x[0..n) to d_hist[256]. The caller
 * zeroes d_hist first, or keeps earlier counts to pool several sets (page
 * section 3.3, the histogram step of calibration). */
int uzip_histogram(const uint16_t *d_x, uint64_t n, uint64_t *d_hist, hipStream_t s);

/* async. As uzip_histogram, over a sample of d_x: the first `sample` words
 * of every block of `block` words (the last block may be partial). block and
 * sample are multiples of 8 with 8 <= sample <= block; block = 0 means all
 * of d_x. This is the sampled estimate of the exponent distribution that
 * "CCCL" (section 4.3, localized frequency tables) builds from the first
 * part of each block's data range (256 KB in its example). */
int uzip_histogram_sampled(const uint16_t *d_x, uint64_t n, uint64_t block, uint64_t sample,
                           uint64_t *d_hist, hipStream_t s);

/* blocking. Calibrates a codebook on d_x[0..n) (page section 3.3).
 * It runs the histogram on the device into d_hist_ws (256 x u64 scratch the
 * caller owns), copies the histogram back, and builds *cb on the host. */
int uzip_calibrate(const uint16_t *d_x, uint64_t n, uint64_t *d_hist_ws,
                   uzip_codebook_t *cb, hipStream_t s);

/* async. Encodes d_x[0..n) into d_out with chunk C (page section 3.2: the
 * dense transform, then the chunked escape arrays).
 *   d_out    stream buffer of out_cap >= uzip_max_bytes(n, C) bytes. Bytes
 *            past the stream's total_bytes are left as they were.
 *   d_ws     workspace of ws_bytes >= uzip_workspace_bytes(n, C) bytes. Its
 *            contents are scratch and are not preserved.
 * The stream's size is in its header: see uzip_stream_bytes. */
int uzip_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s);
int uzip_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                   const uzip_opts_t *opts, hipStream_t s);

/* async. uzip_encode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The call allocates nothing: its workspace
 * is a fixed array of UZIP_NOALLOC_SCRATCH_BYTES in the library's device
 * memory, one per GPU, held from the library's first use on that GPU until
 * the process ends. Inputs with uzip_workspace_bytes(n, chunk) larger than
 * that are rejected with UZIP_ESCRATCH before anything is enqueued. Every call
 * on one GPU uses that GPU's array, so calls that overlap on one GPU (two
 * streams, or two host threads) race and must be serialised by the caller.
 * The array keeps the last call's contents; the result does not depend on
 * them (the encode may load stale bytes past a tile's staged escapes, but
 * never uses them). Output, arguments and the other errors are those of
 * uzip_encode (the device is the current one). */
#define UZIP_NOALLOC_SCRATCH_BYTES (64ull << 20)
int uzip_encode_noalloc(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                        void *d_out, uint64_t out_cap, hipStream_t s);

/* ------------------------------------------------ FP8 E5M2 variant ---- */
/* "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
 * Serving", section 4.2 / appendix C: FP8 E5M2 values (1 sign, 5 exponent,
 * 2 mantissa bits; one byte each) in the same framework. The 5-bit exponent
 * e = (x >> 2) & 0x1f takes a 4-bit Top-16 code, two per byte as above; the
 * other three bits a = ((x >> 5) & 4) | (x & 3) are packed 3 bits per value
 * (value i at bits 3i..3i+2 of the section, least significant bit first:
 * every 8 values fill 3 bytes; unused bits 0); escapes are the BF16 ones
 * (u16 in-chunk position + u8 raw exponent). Stream: the BF16 container with
 * header flags (offset 6) = 1 and a sign-mantissa section of ceil(3n/8)
 * bytes. Payload ceil(3n/8) + ceil(n/2) + 3M bytes: 8/7 with no escape.
 * Codebooks are built from an FP8 exponent histogram; every entry of dec
 * must be below 32 (else UZIP_EINVAL). The workspace is uzip_workspace_bytes. */

/* Largest E5M2 stream for n values at chunk C (M = n); 0 if n or C is invalid. */
uint64_t uzip_fp8_max_bytes(uint64_t n, uint32_t chunk);

/* async. Adds the 5-bit exponent histogram of d_x[0..n) (bytes, 16-byte
 * aligned) to d_hist[256], as uzip_histogram does for BF16. */
int uzip_fp8_histogram(const uint8_t *d_x, uint64_t n, uint64_t *d_hist, hipStream_t s);

/* blocking. As uzip_calibrate, on E5M2 values. */
int uzip_fp8_calibrate(const uint8_t *d_x, uint64_t n, uint64_t *d_hist_ws, uzip_codebook_t *cb,
                       hipStream_t s);

/* async. Encodes n E5M2 values; arguments, ownership and errors as for
 * uzip_encode (out_cap >= uzip_fp8_max_bytes). */
int uzip_fp8_encode(const uint8_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s);
int uzip_fp8_encode_ex(const uint8_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       const uzip_opts_t *opts, hipStream_t s);

/* async. Decodes an E5M2 stream of n values into d_y[0..n) (16-byte
 * aligned); bounds and errors as for uzip_decode (fused patch only). */
int uzip_fp8_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                    const uzip_codebook_t *cb, uint8_t *d_y, hipStream_t s);
int uzip_fp8_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                       const uzip_codebook_t *cb, uint8_t *d_y, const uzip_opts_t *opts, hipStream_t s);

/* ------------------------------------- Top-15 + sentinel (ablation) ---- */
/* "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
 * Serving", section 3.4 / Table 6: the format the page weighs against
 * Top-16, kept here to measure that trade-off. Codes 0..14 are dec[0..14];
 * code 15 marks an escape, whose raw exponent is the next stored one of its
 * chunk; no positions are stored. Stream: header (flags = 2) | sm | codes |
 * offsets | values (u8, chunk by chunk, ascending position); payload
 * N + ceil(N/2) + M. The codebook is a Top-16 one (dec[15] is not used).
 * chunk must be at most 4096 (a decode tile starts a chunk); otherwise as
 * uzip_encode / uzip_decode. */
uint64_t uzip_s15_max_bytes(uint64_t n, uint32_t chunk);
int uzip_s15_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s);
int uzip_s15_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       const uzip_opts_t *opts, hipStream_t s);
int uzip_s15_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                    const uzip_codebook_t *cb, uint16_t *d_y, hipStream_t s);
int uzip_s15_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                       const uzip_codebook_t *cb, uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s);

/* ------------------------------ Top-8 3-bit with positions (ablation) -- */
/* "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
 * Serving", section 4.3 / Table 3 (Top-k exponent coding): the Top-16
 * stream with 3-bit codes for dec[0..7] instead of 4-bit codes for
 * dec[0..15]; every other exponent is an escape (dummy code 0, u16 in-chunk
 * position, u8 raw exponent, as in uzip_encode). The page notes that its
 * 3-bit codes are not byte-aligned; here they are packed back to back: value
 * i's code at bits 3i..3i+2 of the section, least significant bit first.
 * Stream: header (flags = 4) | sm | codes (ceil(3n/8) bytes) | offsets |
 * pos | val, each section 256-byte aligned; payload n + ceil(3n/8) + 3M.
 * The codebook is a Top-16 one (dec[8..15] are not used). Any chunk valid
 * for uzip_encode; otherwise as uzip_encode / uzip_decode. */
uint64_t uzip_t8_max_bytes(uint64_t n, uint32_t chunk);
int uzip_t8_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s);
int uzip_t8_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                      void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                      const uzip_opts_t *opts, hipStream_t s);
int uzip_t8_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                   const uzip_codebook_t *cb, uint16_t *d_y, hipStream_t s);
int uzip_t8_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                      const uzip_codebook_t *cb, uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s);

/* ------------------------------ Top-7 3-bit + zero-point (ablation) ---- */
/* "ZipCCL: Efficient Lossless Data Compression of Communication
 * Collectives", exponent coding: the seven most frequent exponents take
 * 3-bit codes 1..7 (code k + 1 for dec[k], k < 7); any other exponent takes
 * code 0, a zero-point, and its raw exponent is the next stored one of its
 * chunk; no positions are stored. The page's kernels split the 3-bit codes
 * into three 1-bit arrays; the stream keeps that split: bit b of value i's
 * code is bit i % 8 of byte i / 8 of plane b. Stream: header (flags = 3) |
 * sm (n bytes) | plane 0 | plane 1 | plane 2 (ceil(n/8) bytes each, each
 * section 256-byte aligned) | offsets | values (u8, chunk by chunk, ascending
 * position); payload n + 3 ceil(n/8) + M: 16 -> 11 bits per value with no
 * zero-point. The codebook is a Top-16 one (dec[7..15] are not used). chunk
 * must be at most 4096 (a decode tile starts a chunk); otherwise as
 * uzip_encode / uzip_decode. */
uint64_t uzip_z7_max_bytes(uint64_t n, uint32_t chunk);
int uzip_z7_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s);
int uzip_z7_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                      void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                      const uzip_opts_t *opts, hipStream_t s);
int uzip_z7_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                   const uzip_codebook_t *cb, uint16_t *d_y, hipStream_t s);
int uzip_z7_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                      const uzip_codebook_t *cb, uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s);

/* blocking. Reads a device stream's header. Returns its size and M.
 * Either output pointer may be NULL. A format helper: compression changes the
 * size of the data a sender ships, so the transfer has to learn it from the
 * stream ("UCCL-Zip: Lossless Compression Supercharged GPU Communication",
 * section 4, the metadata of compressed sends); the size is also what the
 * ratio 2N / total_bytes is reported on. Returns UZIP_OK, UZIP_EINVAL (NULL
 * stream), UZIP_ECORRUPT (bad magic or version) or UZIP_EHIP. */
int uzip_stream_bytes(const void *d_stream, uint64_t *total_bytes, uint64_t *m, hipStream_t s);

/* async. Encode with a codebook calibrated on the input itself, entirely on
 * the device (no host round trip): the exponent histogram of a sample of
 * d_x (the first `sample` words of every `block` words; block = 0: all of
 * d_x, as for uzip_histogram_sampled), its Top-16 and tables by the same
 * rule as uzip_codebook_from_hist, then uzip_encode with those tables. This
 * is the per-input "dynamic Top-16" that "SplitZip: Ultra Fast Lossless KV
 * Compression for Disaggregated LLM Serving" measures against offline
 * calibration (section 4.3, Table 7), with the sampled estimate of "CCCL"
 * (section 4.3, localized frequency tables) as an option. The stream header
 * carries dec[16]; a receiver rebuilds the codebook with
 * uzip_codebook_from_dec. If d_cb is not NULL (8-byte aligned device
 * memory) the whole codebook is also written there. d_out, d_ws and the
 * errors are as for uzip_encode; the workspace also holds the histogram.
 * Events (uzip_opts_t): [0] before the first kernel, [1] after the three
 * calibration kernels, [2] after the dense pass, [3] after the tile sums,
 * [4] after the escape placement. */
int uzip_encode_online(const uint16_t *d_x, uint64_t n, uint32_t chunk, uint64_t block, uint64_t sample,
                       uzip_codebook_t *d_cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       hipStream_t s);
int uzip_encode_online_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, uint64_t block, uint64_t sample,
                          uzip_codebook_t *d_cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                          const uzip_opts_t *opts, hipStream_t s);

/* async. Decodes a stream of n values at chunk C into d_y[0..n) (page
 * section 3.2: nibble unpack, 16-entry lookup, merge with the sign-mantissa
 * byte, then the sparse escape patch). in_bytes is the size of the readable
 * buffer at d_in (at least the stream's total_bytes). The kernels read
 * nothing past it and never write past d_y[n-1], whatever the header holds.
 * A stream that fails uzip_validate gives unspecified output values. n, C
 * and the codebook must be the ones the stream was encoded with. */
int uzip_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                const uzip_codebook_t *cb, uint16_t *d_y, hipStream_t s);
int uzip_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                   const uzip_codebook_t *cb, uint16_t *d_y, const uzip_opts_t *opts,
                   hipStream_t s);

/* async. Fused decode-add-reencode: the one-GPU share of a compressed
 * all-reduce hop ("UCCL-Zip: Lossless Compression Supercharged GPU
 * Communication", section 3.4 / Figure 6: decompress a received slice, reduce
 * it with the local slice, recompress).
 *   r[i] = bf16_rne( (float)A[i] + (float)B[i] )
 * The sum is one IEEE binary32 add (round to nearest even, subnormals kept).
 * The result rounds half-to-even to BF16. A NaN sum becomes 0x7FC0. A and B
 * are streams of n values at chunk C under codebook cb. The result is
 * encoded with the same n, C and cb into d_out (out_cap >= uzip_max_bytes),
 * with workspace as for uzip_encode. a_bytes and b_bytes bound the reads, as
 * in_bytes does for uzip_decode. */
int uzip_reduce_add(const void *d_a, uint64_t a_bytes, const void *d_b, uint64_t b_bytes,
                    uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                    hipStream_t s);
int uzip_reduce_add_ex(const void *d_a, uint64_t a_bytes, const void *d_b, uint64_t b_bytes,
                       uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       const uzip_opts_t *opts, hipStream_t s);

/* async. k-input fused reduce: the local step of one GPU after a compressed
 * exchange, for instance its shard of the reduce-scatter phase of a two-shot
 * all-reduce ("UCCL-Zip: Lossless Compression Supercharged GPU
 * Communication", section 5.2 / Figure 9: every received chunk is
 * decompressed before it is reduced; "ZipCCL: Efficient Lossless Data
 * Compression of Communication Collectives", adaptive communication
 * strategies: a zipped all-to-all followed by a local reduction).
 *   r[i] = bf16_rne( (...((float)X0[i] + (float)X1[i]) + ...) + (float)Xk-1[i] )
 * The k values are added in binary32 in input order, each add rounded to
 * nearest even with subnormals kept, and the sum is rounded once,
 * half-to-even, to BF16; a NaN sum becomes 0x7FC0. k = 2 gives exactly
 * uzip_reduce_add; k = 1 re-encodes the input with every NaN made 0x7FC0.
 * d_in is a host array of k device stream pointers (16-byte aligned) and
 * in_bytes a host array of their readable sizes; both are read during the
 * call only. 1 <= k <= UZIP_MAX_K. Every input is a stream of n values at
 * chunk C under codebook cb; the result is encoded with the same n, C and cb
 * into d_out (out_cap >= uzip_max_bytes), with workspace as for uzip_encode.
 * Errors: UZIP_EINVAL (k out of range, a null or misaligned pointer, an
 * input smaller than an escape-free stream) and UZIP_ENOSPC, detected on the
 * host before any launch; UZIP_EHIP. As for uzip_decode, the input headers
 * are not checked: use uzip_validate for untrusted input. */
#define UZIP_MAX_K 16
int uzip_reduce_k(const void *const *d_in, const uint64_t *in_bytes, uint32_t k, uint64_t n, uint32_t chunk,
                  const uzip_codebook_t *cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                  hipStream_t s);
int uzip_reduce_k_ex(const void *const *d_in, const uint64_t *in_bytes, uint32_t k, uint64_t n, uint32_t chunk,
                     const uzip_codebook_t *cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                     const uzip_opts_t *opts, hipStream_t s);

/* blocking. Copies a device stream of `bytes` bytes to the host and runs
 * uzip_validate_host on it (the same format helper, for a stream in device
 * memory). */
int uzip_validate(const void *d_stream, uint64_t bytes, const uzip_codebook_t *cb, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* UZIP_H */
