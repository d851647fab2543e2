// uzip.hip -- HIP kernels (gfx950, wave64) and the C-ABI host library for the
// split-exponent lossless BF16 codec. The C-ABI is declared in include/uzip.h.
//
// Method: "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
// Serving" (xllm-io paper review):
//   section 3.2: split x into a = ((x>>8)&0x80)|(x&0x7f) and e = (x>>7)&0xff.
//                Top-16 exponents become 4-bit codes, two per byte. Other
//                exponents are escapes: u16 in-chunk position + u8 exponent.
//                Encode = dense transform, then escape arrays. Decode = nibble
//                unpack + 16-entry lookup + merge, then sparse patch.
//   section 3.3: offline calibration (histogram, Top-16, three tables).
//   section 3.4: every code is a real exponent; escapes carry a dummy code.
// Reduce step: "UCCL-Zip: Lossless Compression Supercharged GPU
// Communication", section 3.4 / Figure 6 (decompress, reduce, recompress).
//
// Kernels:
//   k_hist          exponent histogram. Per-wave LDS sub-histograms, one
//                   global 64-bit atomic per bin per workgroup.
//   k_encode_tile   one pass over the input. 16-byte loads of 8 words per
//                   lane, and the exponent->code table in LDS. Writes the
//                   sign-mantissa and code sections. Counts escapes per wave
//                   with 64-lane ballots, ranks them in element order, and
//                   stages each tile's escapes (position, exponent) compactly
//                   in the workspace.
//   k_group_sums    sums the per-tile escape counts of each group of tiles.
//   k_place_escapes each wave takes a run of consecutive tiles: their escape
//                   prefixes (group sums before their group + tile counts
//                   before each in the group), the chunk offsets, and the
//                   escapes of the tiles with few of them; a heavier tile's
//                   staged escapes go to their final position and value
//                   slots from a wave of its own, by 16-byte shifted block
//                   copies. Wave 0 also writes the header, the last chunk
//                   offset and the zero padding.
//   k_decode_tile   one pass: 8-byte sign-mantissa loads, 4-byte code loads,
//                   16-entry lookup in registers (v_perm). A tile with
//                   escapes writes its exponent bytes to LDS, each escape
//                   overwrites its own byte, and the bytes are read back
//                   before the merge and the single store of the output.
//   k_patch         standalone sparse patch (the two-kernel decode variant).
//   k_reduce_tile   decodes both inputs of a tile as above, adds in binary32,
//                   rounds to BF16 (half to even), then encodes like
//                   k_encode_tile.
//   k_reduce_k_tile the same for k inputs summed in order, one rounding.
//   k8_encode_tile, k8_decode_tile   the FP8 E5M2 variant.
//   k_s15_decode_tile, kz_encode_tile, kz_decode_tile   the Top-15 +
//                   sentinel and Top-7 3-bit + zero-point formats.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "uzip.h"

namespace {

// ------------------------------------------------------------------ layout --
constexpr uint64_t kHeader = 256;

__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255u) & ~uint64_t(255u); }

// Stream formats (header flags): Top-16 codes with escape positions on BF16
// words or on FP8 E5M2 bytes; Top-15 + sentinel on BF16 words (no position
// section); Top-7 3-bit codes + zero-points on BF16 words (three bit planes,
// no position section); Top-8 3-bit codes packed 3 bits per value, with the
// Top-16 escape arrays.
enum : uint8_t { kFmtBF16 = 0, kFmtFP8 = 1, kFmtS15 = 2, kFmtZ7 = 3, kFmtT8 = 4 };

struct Layout {
    uint64_t n, nch;
    uint32_t C, logC;
    uint8_t fmt;
    uint64_t off_codes, off_offs, off_pos;   // off_sm is kHeader; S15 and Z7 values start at off_pos
    uint64_t code_bytes, plane;              // one code section (or plane) and its 256-aligned stride
    uint32_t nplanes;                        // 1, or 3 bit planes for Z7
};

__host__ __device__ inline bool has_pos(uint8_t fmt) { return fmt == kFmtBF16 || fmt == kFmtFP8 || fmt == kFmtT8; }
__host__ __device__ inline uint64_t off_val_of(const Layout &L, uint64_t m)
{
    return L.off_pos + (has_pos(L.fmt) ? align256(2 * m) : 0);
}
__host__ __device__ inline uint64_t total_of(const Layout &L, uint64_t m) { return off_val_of(L, m) + m; }

// fp8: the E5M2 variant, whose sign-mantissa section holds 3 bits per value.
__host__ __device__ inline uint64_t sm_bytes_of(uint64_t n, bool fp8) { return fp8 ? (3 * n + 7) / 8 : n; }

Layout make_layout(uint64_t n, uint32_t C, uint8_t fmt = kFmtBF16)
{
    const bool fp8 = fmt == kFmtFP8;
    Layout L;
    L.n = n;
    L.C = C;
    L.fmt = fmt;
    L.logC = 0;
    while ((1u << L.logC) < C) L.logC++;
    L.nch = (n + C - 1) / C;
    L.off_codes = kHeader + align256(sm_bytes_of(n, fp8));
    L.nplanes = fmt == kFmtZ7 ? 3 : 1;
    L.code_bytes = fmt == kFmtZ7 ? (n + 7) / 8 : fmt == kFmtT8 ? (3 * n + 7) / 8 : (n + 1) / 2;
    L.plane = align256(L.code_bytes);
    L.off_offs = L.off_codes + L.nplanes * L.plane;
    L.off_pos = L.off_offs + align256(4 * (L.nch + 1));
    return L;
}

// ------------------------------------------------------------ tile shapes --
// Compile-time shapes (defaults measured on MI355X; override with -D to sweep).
#ifndef UZIP_ENC_THREADS
#define UZIP_ENC_THREADS 256
#endif
#ifndef UZIP_ENC_GROUPS
#define UZIP_ENC_GROUPS 4          // groups of 8 words per thread
#endif
#ifndef UZIP_DEC_THREADS
#define UZIP_DEC_THREADS 128
#endif
#ifndef UZIP_DEC_GROUPS
#define UZIP_DEC_GROUPS 2          // groups of 16 words per thread
#endif
#ifndef UZIP_DEC_FETCH
#define UZIP_DEC_FETCH 2           // escapes per thread a decode tile loads with its first patch round
#endif
#ifndef UZIP_RED_FETCH
#define UZIP_RED_FETCH 2           // the same, per input, in the reduce
#endif
#ifndef UZIP_NT
#define UZIP_NT 1                  // non-temporal streaming loads/stores
#endif

constexpr int kEncThreads = UZIP_ENC_THREADS;
constexpr int kEncGroups = UZIP_ENC_GROUPS;
constexpr int kEncTile = kEncThreads * kEncGroups * 8;
constexpr int kDecThreads = UZIP_DEC_THREADS;
constexpr int kDecGroups = UZIP_DEC_GROUPS;
constexpr int kDecTile = kDecThreads * kDecGroups * 16;
constexpr int kThreads = 256;               // histogram, placement and patch kernels
constexpr int kDecFetch = UZIP_DEC_FETCH;
constexpr int kRedFetch = UZIP_RED_FETCH;

static_assert((kEncTile & (kEncTile - 1)) == 0 && kEncTile <= 65536, "encode tile: power of two <= 65536");

// A tile's escapes wait in its staging slot between the tile kernel and the
// placement: the raw exponents (kEncTile bytes at most), and kAux bytes that
// hold either the list of their in-chunk positions (a tile with at most
// kPosListMax escapes) or, for a heavier tile, the tile's escape bitmap (bit
// i set when tile value i is an escape), which is smaller than its list; the
// placement rebuilds such a tile's positions from the bitmap.
constexpr int kAux = kEncTile / 8;
constexpr int kPosListMax = kAux / 2;
static_assert((kDecTile & (kDecTile - 1)) == 0 && kDecTile >= 64, "decode tile: power of two");

// Encode workspace (see uzip_workspace_bytes).
struct EncWs {
    unsigned long long *hist;  // [256] exponent histogram (online calibration)
    uint8_t *lut;          // [256] code table built on the device (online calibration)
    uint8_t *dec;          // [16] its decode table
    uint32_t *counts;      // [ntiles] escapes per tile
    uint32_t *gsum;        // [ngroups] escapes per group of 2^gshift tiles
    uint32_t *tpre;        // [ntiles] escapes of the tiles before it inside its group
    uint32_t *chunk_pre;   // [nch] escapes in the tile before each chunk start
    uint8_t  *stage_aux;   // [ntiles * kAux] per tile: its position list, or its escape bitmap
    uint8_t  *stage_val;   // [ntiles * kEncTile] raw exponents, per tile
};

struct WsLayout {
    uint64_t hist, lut, dec, counts, gsum, tpre, chunk_pre, stage_aux, stage_val, total;
};

// Tiles are summed in groups of 2^gshift, with gshift about half of log2(ntiles)
// (at least 6), so a tile's prefix reads at most ~2*sqrt(ntiles) counts.
uint32_t group_shift(uint64_t ntiles)
{
    uint32_t lg = 0;
    while ((1ull << lg) < ntiles) lg++;
    const uint32_t g = (lg + 1) / 2;
    return g < 6 ? 6 : g;
}

WsLayout ws_layout(uint64_t n, uint32_t C)
{
    uint64_t ntiles = (n + kEncTile - 1) / kEncTile;
    uint64_t ngroups = (ntiles + (1ull << group_shift(ntiles)) - 1) >> group_shift(ntiles);
    uint64_t nch = (n + C - 1) / C;
    WsLayout w;
    w.hist = 0;
    w.lut = w.hist + 256 * 8;
    w.dec = w.lut + 256;
    w.counts = w.dec + 256;
    w.gsum = w.counts + align256(4 * ntiles);
    w.tpre = w.gsum + align256(4 * ngroups);
    w.chunk_pre = w.tpre + align256(4 * ntiles);
    w.stage_aux = w.chunk_pre + align256(4 * nch);
    w.stage_val = w.stage_aux + align256(ntiles * kAux);
    w.total = w.stage_val + align256(ntiles * kEncTile) + 256;   // slack for 16-byte over-reads
    return w;
}

// Per-launch constants of an encoder (kernel argument, by value).
struct EncParams {
    uint8_t lut[256];      // code of e in bits 0..3, bit 7 set when e is an escape
    const uint8_t *dlut;   // if not null: the code table in device memory (used instead of lut)
    const uint8_t *ddec;   // if not null: dec[16] in device memory, for the stream header
    uint64_t sm_bytes;     // length of the sign-mantissa section
    uint64_t code_bytes;   // length of a code section (each of nplanes, plane bytes apart)
    uint64_t plane;
    uint32_t nplanes;
    uint32_t posw;         // bytes per escape position: 2, or 0 for streams without positions
    uint64_t n, nch, ntiles, ngroups;
    uint32_t Cmask, logC, gshift;
    uint64_t off_codes, off_offs, off_pos;
};

// Per-launch constants of a decoder.
struct DecParams {
    uint32_t dec[4];       // dec[16] packed little-endian, 4 codes per word
    uint64_t n, nch;
    uint32_t C, logC;
    uint64_t off_codes, off_offs, off_pos;
    uint64_t plane;        // bytes from one code plane to the next (Z7)
};

struct HeaderParams {
    uint8_t tmpl[256];     // header with M and total_bytes left zero
};

// Native vector types for 8- and 16-byte memory operations.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming loads/stores: every byte is touched once per call.
template <typename T>
__device__ __forceinline__ T ld_stream(const T *p)
{
#if UZIP_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void st_stream(T v, T *p)
{
#if UZIP_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// --------------------------------------------------------- bit helpers -----
#ifndef UZIP_PLACE_NT
#define UZIP_PLACE_NT 1
#endif
// Stores of the escape placement: non-temporal (ordinary write-back stores
// with UZIP_PLACE_NT = 0). Write-back stores make the kernel itself finish
// sooner, but part of what it writes then stays dirty in the memory-side
// cache and is written back during the next operation, which costs more
// than it saved.
template <typename T>
__device__ __forceinline__ void st_place(T v, T *p)
{
    if constexpr (UZIP_PLACE_NT != 0) st_stream(v, p);
    else *p = v;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b)
{
    return (a & mask) | (b & ~mask);
}

// Bit j of the nibble b to bit 0 of byte j (the four shifted copies of b
// that the multiply adds occupy disjoint bits, so nothing carries).
__device__ __forceinline__ uint32_t spread4(uint32_t b) { return (b * 0x00204081u) & 0x01010101u; }

// 0xFF in byte j where bit j of the nibble b is set, else 0 (byte permute
// selectors 12 and 13 give 0x00 and 0xFF).
__device__ __forceinline__ uint32_t bytemask4(uint32_t b) { return perm(0u, 0u, 0x0C0C0C0Cu + spread4(b)); }

// 4 three-bit values held one per byte -> a0 | a1 << 3 | a2 << 6 | a3 << 9.
__device__ __forceinline__ uint32_t pack12(uint32_t a)
{
    const uint32_t t = (a | (a >> 5)) & 0x003F003Fu;
    return (t | (t >> 10)) & 0xFFFu;
}

// Inverse of pack12.
__device__ __forceinline__ uint32_t unpack12(uint32_t c)
{
    const uint32_t t = (c & 0x3Fu) | ((c & 0xFC0u) << 10);
    return (t & 0x00070007u) | ((t & 0x00380038u) << 5);
}

// Sign-mantissa bytes of 4 words held in two dwords (word 2i in the low half).
__device__ __forceinline__ uint32_t signmant4(uint32_t v0, uint32_t v1)
{
    // low byte of each half: bits 0..6 from the word, bit 7 = word bit 15
    uint32_t t0 = bfi(0x007F007Fu, v0, v0 >> 8);
    uint32_t t1 = bfi(0x007F007Fu, v1, v1 >> 8);
    return perm(t1, t0, 0x06040200u);
}

// Exponent-table entries of 4 consecutive words: byte j = lut[e_j].
__device__ __forceinline__ uint32_t lut4(const uint8_t *s_lut, uint32_t v0, uint32_t v1)
{
    uint32_t b0 = s_lut[(v0 >> 7) & 0xFFu];
    uint32_t b1 = s_lut[(v0 >> 23) & 0xFFu];
    uint32_t b2 = s_lut[(v1 >> 7) & 0xFFu];
    uint32_t b3 = s_lut[(v1 >> 23) & 0xFFu];
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// The table bytes of 8 words, L0 (words 0..3) and L1 (words 4..7), gathered
// by parity into two dwords (words 0, 2, 4, 6 and words 1, 3, 5, 7, one per
// byte). From them, the packed code nibbles (word 2j in the low nibble of
// byte j, word 2j + 1 in the high one) and the escape flags (bit 7 of each
// table byte), word j's at bit 4j + 3 (the even words' flags moved down 4
// bits), so that one loop over the set bits of a whole group meets them in
// word order.
struct Codes8 {
    uint32_t codes, flags;
};
__device__ __forceinline__ Codes8 codes_flags8(uint32_t L0, uint32_t L1)
{
    const uint32_t fe = perm(L1, L0, 0x06040200u), fo = perm(L1, L0, 0x07050301u);
    Codes8 c;
    c.codes = (fe & 0x0F0F0F0Fu) | ((fo & 0x0F0F0F0Fu) << 4);
    c.flags = ((fe >> 4) & 0x08080808u) | (fo & 0x80808080u);
    return c;
}

// The 8 escape flags of a group (codes_flags8's layout, word j at bit
// 4j + 3) as one byte, word j at bit j.
__device__ __forceinline__ uint32_t flags_byte(uint32_t fl)
{
    uint32_t x = (fl >> 3) & 0x11111111u;          // word j at bit 4j
    x = (x | (x >> 3)) & 0x03030303u;              // words 2i, 2i + 1 at bits 8i, 8i + 1
    x = (x | (x >> 6)) & 0x000F000Fu;              // words 4h..4h + 3 at bits 16h..16h + 3
    return (x | (x >> 12)) & 0xFFu;
}

// Exponents of 4 words from 4 code nibbles held one per byte (values 0..15),
// through the 16-entry table dec (4 dwords).
__device__ __forceinline__ uint32_t dec4(const uint32_t dec[4], uint32_t nib)
{
    uint32_t sel = nib & 0x07070707u;
    uint32_t lo = perm(dec[1], dec[0], sel);
    uint32_t hi = perm(dec[3], dec[2], sel);
    // pick hi for bytes whose code has bit 3 set: selector byte k -> k or 4+k
    uint32_t pick = ((nib >> 1) & 0x04040404u) | 0x03020100u;
    return perm(hi, lo, pick);
}

// Rebuild 2 words from a dword of interleaved bytes [a0, e0, a1, e1].
__device__ __forceinline__ uint32_t merge2(uint32_t w)
{
    // per half: bits 0..6 = a & 0x7f, bits 7..14 = e, bit 15 = a bit 7
    uint32_t t = bfi(0x80008000u, w << 8, w);
    return bfi(0x7F807F80u, w >> 1, t);
}

// Exponents of 8 words from their 8 code nibbles, one per byte: e[0] holds
// words 0..3, e[1] words 4..7.
__device__ __forceinline__ void decode8_e(uint32_t codes, const uint32_t dec[4], uint32_t e[2])
{
    const uint32_t lo = codes & 0x0F0F0F0Fu;          // nibbles of words 0,2,4,6
    const uint32_t hi = (codes >> 4) & 0x0F0F0F0Fu;   // nibbles of words 1,3,5,7
    e[0] = dec4(dec, perm(hi, lo, 0x05010400u));      // [c0, c1, c2, c3]
    e[1] = dec4(dec, perm(hi, lo, 0x07030602u));      // [c4, c5, c6, c7]
}

// 8 words from their sign-mantissa bytes (2 dwords) and exponents (e[2]).
__device__ __forceinline__ void merge8(uint32_t sm0, uint32_t sm1, const uint32_t e[2], uint32_t y[4])
{
    y[0] = merge2(perm(e[0], sm0, 0x05010400u));
    y[1] = merge2(perm(e[0], sm0, 0x07030602u));
    y[2] = merge2(perm(e[1], sm1, 0x05010400u));
    y[3] = merge2(perm(e[1], sm1, 0x07030602u));
}

// The binary32 values of 8 words from their sign-mantissa bytes (sm0: words
// 0..3, sm1: words 4..7, one per byte) and exponents (e[2]), without forming
// the words: value j is the word shifted up 16 bits, i.e. the bytes
// [0, 0, lo_j, hi_j] with hi_j = sign | e >> 1 and lo_j = (e & 1) << 7 |
// mantissa. Each shift of the exponent bytes moves bits into a neighbouring
// byte only at positions the sign-mantissa byte fills in the following bfi,
// and one byte permute (selector 12 gives 0x00) places each value.
__device__ __forceinline__ void floats8(uint32_t sm0, uint32_t sm1, const uint32_t e[2], float f[8])
{
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t a = h ? sm1 : sm0;
        const uint32_t hi = bfi(0x80808080u, a, e[h] >> 1);
        const uint32_t lo = bfi(0x7F7F7F7Fu, a, e[h] << 7);
#pragma unroll
        for (int j = 0; j < 4; j++)
            f[4 * h + j] = __uint_as_float(perm(hi, lo, ((4u + j) << 24) | ((uint32_t)j << 16) | 0x0C0Cu));
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two binary32 values rounded to BF16, s0 in the low half, NaN -> 0x7FC0.
// Rounding is half to even on the bit pattern: add 0x7FFF plus the lowest
// kept bit, keep the high 16 bits (a carry out of the mantissa rounds up
// into the exponent, up to infinity). One v_cvt_pk_bf16_f32 does exactly
// that for every non-NaN binary32 pattern (checked on MI355X over all 2^32
// patterns in both halves) but keeps a NaN's payload, so NaNs are fixed
// after it.
__device__ __forceinline__ uint32_t bf16x2_rne(float s0, float s1)
{
    const f32x2 v = {s0, s1};
    uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    if (s0 != s0) r = (r & 0xFFFF0000u) | 0x7FC0u;
    if (s1 != s1) r = (r & 0x0000FFFFu) | 0x7FC00000u;
    return r;
}

// bf16x2_rne without the NaN fix, which is final unless s0 or s1 is a NaN:
// nan is set then (one unordered compare covers both). Callers redo the
// values of a wave whose ballot of nan is not empty with bf16x2_rne.
__device__ __forceinline__ uint32_t bf16x2_rne_fast(float s0, float s1, bool &nan)
{
    const f32x2 v = {s0, s1};
    nan = __builtin_isunordered(s0, s1);
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}


// =========================================================== histogram ====
// Exponent histogram of a sample of x: the first S values of every block of
// B values (S = B: all of x). EB is the element width: 2 for BF16 (exponent
// bits 7..14), 1 for FP8 E5M2 (bits 2..6). B and S are multiples of the
// values per 16 bytes (VG = 16 / EB) with S <= B. Each wave counts into
// kHistCopies copies of a 256-bin table in LDS, lane l into copy
// l % kHistCopies: exponents of neighbouring values are mostly equal, and
// lanes adding to one LDS word are served one after another, so more copies
// mean fewer lanes per word. The counters are 16 bits, two bins per word
// (bin e in the half e & 1 of word e >> 1), which keeps 16 copies per wave
// within the LDS of 4 resident workgroups: a lane counts at most 8,192
// values plus one partial group (the grid holds 2^19 threads whenever a lane
// would get more than one round), so a copy's 4 lanes never carry a bin
// past 32,828. Copies are 129 words
// apart, so word w of different copies sits in different banks. Each
// workgroup adds its counts to hist (one 64-bit atomic per non-empty bin).
// (Measured on 2^28 BF16 words: 135 us with 8 copies of 32-bit counters,
// 107 us with 16 copies of 16-bit ones.)
constexpr int kHistCopies = 16;
constexpr int kHistStride = 129;
constexpr int kHistUnroll = 8;
template <int EB>
__device__ __forceinline__ uint32_t hist_exponent(uint32_t v)
{
    return EB == 2 ? (v >> 7) & 0xFFu : (v >> 2) & 0x1Fu;
}

template <int EB>
__global__ __launch_bounds__(kThreads) void k_hist(const uint8_t *__restrict__ x, uint64_t n, uint64_t B,
                                                   uint64_t S, unsigned long long *__restrict__ hist)
{
    constexpr uint32_t VG = 16 / EB;                         // values per 16-byte group
    __shared__ uint32_t sh[kThreads / 64][kHistCopies * kHistStride];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < (kThreads / 64) * kHistCopies * kHistStride; i += kThreads) (&sh[0][0])[i] = 0;
    __syncthreads();
    uint32_t *mine = &sh[wave][(lane % kHistCopies) * kHistStride];
    // groups of VG values, numbered block by block (n < 2^32, so 32 bits hold
    // them); kHistUnroll groups per thread and round, all loads issued first
    const uint32_t nblk = (uint32_t)((n + B - 1) / B);
    const uint32_t gps = (uint32_t)(S / VG);                 // groups per block sample
    const uint32_t ngroups = nblk * gps;
    const uint32_t stride = gridDim.x * kThreads * kHistUnroll;
    for (uint32_t g0 = blockIdx.x * kThreads * kHistUnroll + tid; g0 < ngroups; g0 += stride) {
        u32x4 v[kHistUnroll];
        uint64_t w0[kHistUnroll];
#pragma unroll
        for (int u = 0; u < kHistUnroll; u++) {
            const uint32_t g = g0 + u * kThreads;
            w0[u] = (uint64_t)(g / gps) * B + (uint64_t)(g % gps) * VG;   // first value of the group
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (g < ngroups && w0[u] + VG <= n) v[u] = ld_stream(reinterpret_cast<const u32x4 *>(x + EB * w0[u]));
        }
#pragma unroll
        for (int u = 0; u < kHistUnroll; u++) {
            const uint32_t g = g0 + u * kThreads;
            if (g >= ngroups) continue;
            if (w0[u] + VG <= n) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int q = 0; q < 4; q++)
#pragma unroll
                    for (int h = 0; h < 4 / EB; h++) {
                        const uint32_t e = hist_exponent<EB>(w[q] >> (8 * EB * h));
                        atomicAdd(&mine[e >> 1], 1u << (16 * (e & 1)));
                    }
            } else {
                for (uint64_t i = w0[u]; i < n; i++) {
                    const uint32_t val = EB == 2 ? reinterpret_cast<const uint16_t *>(x)[i] : x[i];
                    const uint32_t e = hist_exponent<EB>(val);
                    atomicAdd(&mine[e >> 1], 1u << (16 * (e & 1)));
                }
            }
        }
    }
    __syncthreads();
    for (int b = tid; b < 256; b += kThreads) {
        uint32_t s = 0;
        for (int q = 0; q < kThreads / 64; q++)
            for (int c = 0; c < kHistCopies; c++) s += (sh[q][c * kHistStride + (b >> 1)] >> (16 * (b & 1))) & 0xFFFFu;
        if (s) atomicAdd(&hist[b], (unsigned long long)s);
    }
}

// Online calibration, step 1: zero the workspace histogram (a kernel, not a
// memset, so that the call can be captured in a graph).
__global__ void k_zero_hist(unsigned long long *__restrict__ hist)
{
    hist[threadIdx.x] = 0ull;
}

// Online calibration, step 3 (one workgroup of 256 threads, thread e for
// exponent e): the Top-16 of the histogram under the total order (count
// descending, exponent ascending) -- e's rank is the number of exponents
// before it in that order -- and the tables built from it: lut[e] = code, or
// 0x80 for an exponent outside the codebook, and dec[16]. If cb is not null
// the whole codebook (the same fields as on the host) is written there too.
__global__ __launch_bounds__(256) void k_top16(const unsigned long long *__restrict__ hist,
                                               uint8_t *__restrict__ lut, uint8_t *__restrict__ dec,
                                               uzip_codebook_t *__restrict__ cb)
{
    __shared__ unsigned long long h[256];
    __shared__ unsigned long long part[4];
    const uint32_t e = threadIdx.x;
    const unsigned long long he = hist[e];
    h[e] = he;
    __syncthreads();
    uint32_t rank = 0;
    for (uint32_t q = 0; q < 256; q++) {
        const unsigned long long hq = h[q];
        rank += (hq > he || (hq == he && q < e)) ? 1u : 0u;
    }
    lut[e] = rank < 16 ? (uint8_t)rank : (uint8_t)0x80;
    if (rank < 16) dec[rank] = (uint8_t)e;
    if (cb) {
        cb->enc[e] = rank < 16 ? (uint8_t)rank : (uint8_t)0;
        cb->member[e] = rank < 16 ? (uint8_t)1 : (uint8_t)0;
        cb->hist[e] = he;
        if (rank < 16) cb->dec[rank] = (uint8_t)e;
        unsigned long long t = he;
        for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
        if ((e & 63) == 0) part[e >> 6] = t;
        __syncthreads();
        if (e == 0) {
            cb->n_cal = part[0] + part[1] + part[2] + part[3];
            cb->version = UZIP_VERSION;
        }
    }
}

// ============================================================== encode ====
// LDS of the encode back end.
// (NT threads per workgroup, NG groups of 8 words per thread.)
template <int NT = kEncThreads, int NG = kEncGroups>
struct EncSharedT {
    uint8_t lut[256];                       // the code table (one copy: a barrier publishes it)
    uint32_t wtot[NG][NT / 64];
};
using EncShared = EncSharedT<>;
// A tile's escapes in element order (compacted), written out with 16-byte
// stores: the exponents of all of them, the positions of a tile with at most
// kPosListMax (a heavier tile's positions go out as its bitmap).
struct alignas(16) EscBuf {
    uint16_t pos[kPosListMax];
    uint8_t val[kEncTile];
};

// Copies the code table to LDS (threads 0..63, 4 bytes each); a workgroup
// barrier must follow before any wave reads it.
template <typename Sh>
__device__ __forceinline__ void load_shared_lut(Sh &sh, const uint8_t *lut)
{
    if (threadIdx.x < 64)
        reinterpret_cast<uint32_t *>(sh.lut)[threadIdx.x] = reinterpret_cast<const uint32_t *>(lut)[threadIdx.x];
}

// Inclusive prefix sum of v within each row of 16 lanes (a lane whose
// source lies before its row's start adds 0).
__device__ __forceinline__ uint32_t row_inclusive_sum(uint32_t v)
{
    v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    return v;
}

// Inclusive prefix sum of v over the 64 lanes of a wave: row shifts by 1, 2,
// 4 and 8 within each row of 16 lanes, then lane 15 of each row added to the
// next row and lane 31 to the upper two rows (DPP row broadcasts).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v)
{
    v = row_inclusive_sum(v);
    v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}


// Words of tile t0 (at most kEncTile), a scalar.
__device__ __forceinline__ uint32_t enc_tile_words(uint64_t t0, const EncParams &p)
{
    return (uint32_t)((p.n - t0 < (uint64_t)kEncTile) ? p.n - t0 : (uint64_t)kEncTile);
}

// Bit b (b = 0..2) of the 3-bit codes of 8 words (code bytes of words 0..3
// in L0, 4..7 in L1), gathered into byte b of the result: bit j of byte b is
// bit b of word j's code. The two code fields of byte i of m8 (word i in bits
// 0..2, word 4 + i in bits 4..6) put bit b of word i at 8i and of word 4 + i
// at 8i + 4; one multiply by 2^24 + 2^17 + 2^10 + 2^3 moves word j to bit
// 24 + j, and no two partial products meet, so nothing carries.
__device__ __forceinline__ uint32_t plane_bytes8(uint32_t L0, uint32_t L1)
{
    const uint32_t m8 = (L0 & 0x07070707u) | ((L1 & 0x07070707u) << 4);
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 3; b++) v |= ((((m8 >> b) & 0x11111111u) * 0x01020408u) >> 24) << (8 * b);
    return v;
}

// Quad transpose of plane bytes: lane q of each group of 4 lanes (q < 3)
// returns the dword of plane q made of byte q of the 4 lanes' v, lane 0's
// byte lowest (DPP quad broadcasts, then two byte permutes).
__device__ __forceinline__ uint32_t quad_planes(uint32_t v, uint32_t q)
{
    const uint32_t a0 = __builtin_amdgcn_update_dpp(0u, v, 0x00, 0xF, 0xF, false);   // quad_perm [0,0,0,0]
    const uint32_t a1 = __builtin_amdgcn_update_dpp(0u, v, 0x55, 0xF, 0xF, false);   // quad_perm [1,1,1,1]
    const uint32_t a2 = __builtin_amdgcn_update_dpp(0u, v, 0xAA, 0xF, 0xF, false);   // quad_perm [2,2,2,2]
    const uint32_t a3 = __builtin_amdgcn_update_dpp(0u, v, 0xFF, 0xF, 0xF, false);   // quad_perm [3,3,3,3]
    const uint32_t sel = 0x0C0C0000u | ((4u + q) << 8) | q;
    return perm(a1, a0, sel) | (perm(a3, a2, sel) << 16);
}

// Encode front half shared by k_encode_tile and k_reduce_tile. Each thread
// holds kEncGroups groups of 8 words (group k covers tile words
// k*kEncThreads*8 + tid*8 .. +8) in xw[k][0..3] (word 2q in the low half of
// xw[k][q]); the tile has rem words. Writes the dense sections and lists the
// tile's escapes in element order in LDS (eb). Returns the tile's escape
// count m (the same in every thread). cstart[k] is the number of the tile's
// escapes before group k when group k starts a chunk, else ~0u. Ends without
// a barrier after the LDS writes of eb. kCodes: kCodeNib, 4-bit codes two per
// byte; kCodePlanes, 3-bit codes (lut bits 0..2) in three bit planes
// (p.plane bytes apart); kCodePack3, 3-bit codes packed 3 bits per value.
// With 3-bit codes every thread of the workgroup must take part (quad
// exchanges).
enum { kCodeNib = 0, kCodePlanes = 1, kCodePack3 = 2 };

// The packed 3-bit codes of a quad of lanes (24 bits each, 8 values, lane
// 0's lowest): lane q < 3 returns dword q of the quad's 12 bytes (its own
// bits from bit 8q on, then the next lane's).
__device__ __forceinline__ uint32_t quad_pack3(uint32_t v, uint32_t q)
{
    const uint32_t nxt = __builtin_amdgcn_update_dpp(0u, v, 0xF9, 0xF, 0xF, false);   // quad_perm [1,2,3,3]
    return (v >> (8 * q)) | (nxt << (24 - 8 * q));
}

template <int kCodes = kCodeNib, int NT = kEncThreads, int NG = kEncGroups>
__device__ __forceinline__ uint32_t encode_dense_rank(const uint32_t xw[NG][4], uint64_t t0, uint32_t rem,
                                                      uint8_t *__restrict__ out, const EncParams &p,
                                                      EncSharedT<NT, NG> &sh, EscBuf &eb, uint32_t cstart[NG],
                                                      uint8_t *__restrict__ aux)
{
    static_assert(NT * NG * 8 == kEncTile, "a workgroup encodes one tile");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the tile's bases (scalar); lanes index them with 32-bit offsets
    uint8_t *smt = out + kHeader + t0;
    uint8_t *cdt = out + p.off_codes + t0 / 2;
    const uint32_t t0m = (uint32_t)(t0 & p.Cmask);      // offset of the tile in its chunk
    uint32_t fl[NG], sm[NG][2], cw[NG];
    // table lookups and dense values for every group, then all the stores
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const uint32_t lo = (uint32_t)(k * (NT * 8) + tid * 8);
        uint32_t L0 = 0, L1 = 0;
        if (lo < rem) {
            L0 = lut4(sh.lut, xw[k][0], xw[k][1]);
            L1 = lut4(sh.lut, xw[k][2], xw[k][3]);
            if (lo + 8 > rem) {       // tail group: words past n are not escapes
                const uint32_t valid = rem - lo;   // 1..7
                const uint64_t keep = (1ull << (8 * valid)) - 1ull;
                const uint64_t both = ((uint64_t)L1 << 32 | L0) & keep;
                L0 = (uint32_t)both;
                L1 = (uint32_t)(both >> 32);
            }
        }
        const Codes8 c8 = codes_flags8(L0, L1);
        fl[k] = c8.flags;
        sm[k][0] = signmant4(xw[k][0], xw[k][1]);
        sm[k][1] = signmant4(xw[k][2], xw[k][3]);
        if constexpr (kCodes == kCodePlanes) cw[k] = quad_planes(plane_bytes8(L0, L1), (uint32_t)(lane & 3));
        else if constexpr (kCodes == kCodePack3)
            cw[k] = quad_pack3(pack12(L0 & 0x07070707u) | (pack12(L1 & 0x07070707u) << 12), (uint32_t)(lane & 3));
        else cw[k] = c8.codes;
    }
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const uint32_t lo = (uint32_t)(k * (NT * 8) + tid * 8);
        if (lo < rem) {
            u32x2 smv;
            smv.x = sm[k][0];
            smv.y = sm[k][1];
            st_stream(smv, reinterpret_cast<u32x2 *>(smt + lo));
            if constexpr (kCodes == kCodeNib) st_stream(cw[k], reinterpret_cast<uint32_t *>(cdt + lo / 2));
        }
        if constexpr (kCodes == kCodePack3) {
            // lane q < 3 of a quad stores dword q of the quad's 12 code
            // bytes (32 words from lq); a quad whose first group is past the
            // end stores nothing; bits past n are 0
            const uint32_t q = (uint32_t)(lane & 3), lq = lo - 8 * q;
            if (q < 3 && lq < rem)
                st_stream(cw[k], reinterpret_cast<uint32_t *>(out + p.off_codes + (3 * (t0 + lq)) / 8 + 4 * q));
        }
        if constexpr (kCodes == kCodePlanes) {
            // lane q < 3 of a quad stores the quad's dword of plane q (its
            // bytes are the 4 lanes' 8-word groups); a quad whose first group
            // is past the end stores nothing
            const uint32_t q = (uint32_t)(lane & 3), lq = lo - 8 * q;
            if (q < 3 && lq < rem)
                st_stream(cw[k], reinterpret_cast<uint32_t *>(out + p.off_codes + q * p.plane + t0 / 8 + lq / 8));
        }
    }
    // escape count of each group -> exclusive prefix over the wave's lanes
    uint32_t pre[NG];
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const uint32_t cnt = __builtin_popcount(fl[k]);
        uint32_t wt = 0, pr = 0;
        if (__ballot(cnt != 0) != 0ull) {
            const uint32_t inc = wave_inclusive_sum(cnt);
            pr = inc - cnt;
            wt = __builtin_amdgcn_readlane(inc, 63);
        }
        pre[k] = pr;
        if (lane == 0) sh.wtot[k][wave] = wt;
    }
    __syncthreads();
    // element order inside the tile is (group k, wave, lane, word): each row
    // of 16 lanes takes the exclusive prefix of the group-major totals, and
    // the wave reads its own entries out of it (wave-uniform values)
    constexpr int kTot = NG * (NT / 64);
    static_assert(kTot <= 16, "the wave totals fit one row of 16 lanes");
    const uint32_t tv = (lane & 15) < kTot ? (&sh.wtot[0][0])[lane & 15] : 0u;
    const uint32_t tinc = row_inclusive_sum(tv), texc = tinc - tv;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t base[NG];
#pragma unroll
    for (int k = 0; k < NG; k++)
        base[k] = __builtin_amdgcn_readlane(texc, k * (NT / 64) + wv);
    const uint32_t run = __builtin_amdgcn_readlane(tinc, kTot - 1);
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const uint32_t lo = (uint32_t)(k * (NT * 8) + tid * 8);
        cstart[k] = (lo < rem && ((t0m + lo) & p.Cmask) == 0) ? base[k] + pre[k] : ~0u;
    }
    // the list in LDS: every escape's exponent, and its position as well
    // when the tile has at most kPosListMax escapes (run is the same in
    // every thread); a heavier tile's positions go to its staging slot as
    // the tile's escape bitmap, one byte per group of 8 words (byte lo / 8;
    // groups past the end have no escapes, so their bytes are 0)
    const bool want_pos = p.posw != 0;
    const bool lst = want_pos && run <= (uint32_t)kPosListMax;
    if (want_pos && !lst) {
#pragma unroll
        for (int k = 0; k < NG; k++)
            aux[(uint32_t)(k * (NT * 8) + tid * 8) >> 3] = (uint8_t)flags_byte(fl[k]);
    }
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const uint32_t lo = (uint32_t)(k * (NT * 8) + tid * 8);
        uint32_t rank = base[k] + pre[k];
        const uint32_t g0m = (t0m + lo) & p.Cmask;          // a multiple of 8, below C
        uint32_t mask = fl[k];
        if (mask == 0) continue;
        // exponents of words 0..7, one per byte of ex1:ex0
        const uint32_t ex0 = perm(xw[k][1] >> 7, xw[k][0] >> 7, 0x06040200u);
        const uint32_t ex1 = perm(xw[k][3] >> 7, xw[k][2] >> 7, 0x06040200u);
        while (mask) {
            const uint32_t j = __builtin_ctz(mask) >> 2;       // the word, 0..7
            if (lst) eb.pos[rank] = (uint16_t)(g0m + j);
            eb.val[rank] = (uint8_t)perm(ex1, ex0, j);
            rank++;
            mask &= mask - 1;
        }
    }
    return run;
}

// Staging back half: the tile's count, its in-tile prefix at each chunk
// start, and its escape list copied to the tile's staging slot with 16-byte
// stores: the exponents, and the positions of a tile with at most
// kPosListMax escapes (the last store of each array may carry stale bytes
// past m: the slot is scratch and only its first m entries are read). The
// stores are temporal: the placement kernel reads the slot back right away,
// from the Infinity Cache.
// G groups of GW values per thread (group k of thread tid starts at tile
// value k*kEncThreads*GW + tid*GW).
template <int G = kEncGroups, int GW = 8, int NT = kEncThreads>
__device__ __forceinline__ void stage_escapes(uint32_t m, const uint32_t cstart[G], uint64_t t0,
                                              uint64_t tile, const EncWs &ws, const EncParams &p,
                                              const EscBuf &eb)
{
    const int tid = threadIdx.x;
    if (tid == 0) ws.counts[tile] = m;
    if (p.Cmask + 1 < (uint32_t)kEncTile) {
        uint32_t *cpt = ws.chunk_pre + (t0 >> p.logC);     // chunks no larger than the tile start at t0
#pragma unroll
        for (int k = 0; k < G; k++) {
            const uint32_t lo = (uint32_t)(k * (NT * GW) + tid * GW);
            if (cstart[k] != ~0u) cpt[lo >> p.logC] = cstart[k];
        }
    }
    if (m == 0) return;
    __syncthreads();
    if (p.posw && m <= (uint32_t)kPosListMax) {
        u32x4 *sp = reinterpret_cast<u32x4 *>(ws.stage_aux + tile * kAux);
        const u32x4 *lp = reinterpret_cast<const u32x4 *>(eb.pos);
        for (uint32_t q = tid; q < (m + 7) / 8; q += NT) sp[q] = lp[q];
    }
    u32x4 *sv = reinterpret_cast<u32x4 *>(ws.stage_val + tile * kEncTile);
    const u32x4 *lv = reinterpret_cast<const u32x4 *>(eb.val);
    for (uint32_t q = tid; q < (m + 15) / 16; q += NT) sv[q] = lv[q];
}

template <int kCodes>
__device__ __forceinline__ void encode_tile(const uint16_t *__restrict__ x, uint8_t *__restrict__ out,
                                            const EncWs &ws, const EncParams &p)
{
    __shared__ EncShared sh;
    __shared__ EscBuf eb;
    const int tid = threadIdx.x;
    const uint64_t tile = blockIdx.x;
    const uint64_t t0 = tile * kEncTile;
    const uint32_t rem = enc_tile_words(t0, p);
    const uint16_t *xt = x + t0;
    uint32_t xw[kEncGroups][4];
#pragma unroll
    for (int k = 0; k < kEncGroups; k++) {
        const uint32_t lo = (uint32_t)(k * (kEncThreads * 8) + tid * 8);
        if (lo + 8 <= rem) {
            const u32x4 v = ld_stream(reinterpret_cast<const u32x4 *>(xt + lo));
            xw[k][0] = v.x; xw[k][1] = v.y; xw[k][2] = v.z; xw[k][3] = v.w;
        } else {
            uint16_t h[8];
#pragma unroll
            for (int j = 0; j < 8; j++) h[j] = (lo + j < rem) ? xt[lo + j] : (uint16_t)0;
#pragma unroll
            for (int q = 0; q < 4; q++) xw[k][q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
        }
    }
    // the code table goes to LDS after the data loads are in flight: one
    // copy for the workgroup, at a constant address that the byte reads'
    // offset absorbs
    load_shared_lut(sh, p.dlut ? p.dlut : p.lut);
    __syncthreads();
    uint32_t cstart[kEncGroups];
    const uint32_t m = encode_dense_rank<kCodes>(xw, t0, rem, out, p, sh, eb, cstart, ws.stage_aux + tile * kAux);
    stage_escapes(m, cstart, t0, tile, ws, p, eb);
}

__global__ __launch_bounds__(kEncThreads) void k_encode_tile(const uint16_t *__restrict__ x,
                                                             uint8_t *__restrict__ out, EncWs ws, EncParams p)
{
    encode_tile<kCodeNib>(x, out, ws, p);
}

// Top-7 3-bit + zero-point streams: the same pass with the codes written as
// three bit planes.
__global__ __launch_bounds__(kEncThreads) void kz_encode_tile(const uint16_t *__restrict__ x,
                                                              uint8_t *__restrict__ out, EncWs ws, EncParams p)
{
    encode_tile<kCodePlanes>(x, out, ws, p);
}

// Top-8 3-bit streams: the same pass with the codes packed 3 bits per value.
__global__ __launch_bounds__(kEncThreads) void kt8_encode_tile(const uint16_t *__restrict__ x,
                                                               uint8_t *__restrict__ out, EncWs ws, EncParams p)
{
    encode_tile<kCodePack3>(x, out, ws, p);
}

// One workgroup per group of 2^gshift tiles: gsum[g] = escapes in the group,
// tpre[t] = escapes of the group's tiles before t (each thread scans a run
// of consecutive tiles, then the runs are scanned across the workgroup).
__global__ __launch_bounds__(kThreads) void k_group_sums(EncWs ws, EncParams p)
{
    __shared__ uint32_t s_wave[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t glo = (uint64_t)blockIdx.x << p.gshift;
    uint64_t ghi = glo + (1ull << p.gshift);
    if (ghi > p.ntiles) ghi = p.ntiles;
    const uint64_t per = ((1ull << p.gshift) + kThreads - 1) / kThreads;
    const uint64_t lo = glo + tid * per;
    const uint64_t hi = (lo + per < ghi) ? lo + per : (lo < ghi ? ghi : lo);
    uint32_t sum = 0;
    for (uint64_t t = lo; t < hi; t++) sum += ws.counts[t];
    const uint32_t inc = wave_inclusive_sum(sum);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    uint32_t run = inc - sum, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) {
        if (w < wave) run += s_wave[w];
        total += s_wave[w];
    }
    for (uint64_t t = lo; t < hi; t++) {
        const uint32_t c = ws.counts[t];
        ws.tpre[t] = run;
        run += c;
    }
    if (tid == 0) ws.gsum[blockIdx.x] = total;
}

// Bytes [r, r + 16) of the 32 bytes lo|hi (r in 0..15, the same in every
// lane of the wave: the switch does not diverge).
__device__ __forceinline__ u32x4 extract16(u32x4 lo, u32x4 hi, uint32_t r)
{
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const uint32_t b = r & 3;
    u32x4 o;
    switch (r >> 2) {
    case 0:
        o.x = __builtin_amdgcn_alignbyte(d[1], d[0], b); o.y = __builtin_amdgcn_alignbyte(d[2], d[1], b);
        o.z = __builtin_amdgcn_alignbyte(d[3], d[2], b); o.w = __builtin_amdgcn_alignbyte(d[4], d[3], b);
        break;
    case 1:
        o.x = __builtin_amdgcn_alignbyte(d[2], d[1], b); o.y = __builtin_amdgcn_alignbyte(d[3], d[2], b);
        o.z = __builtin_amdgcn_alignbyte(d[4], d[3], b); o.w = __builtin_amdgcn_alignbyte(d[5], d[4], b);
        break;
    case 2:
        o.x = __builtin_amdgcn_alignbyte(d[3], d[2], b); o.y = __builtin_amdgcn_alignbyte(d[4], d[3], b);
        o.z = __builtin_amdgcn_alignbyte(d[5], d[4], b); o.w = __builtin_amdgcn_alignbyte(d[6], d[5], b);
        break;
    default:
        o.x = __builtin_amdgcn_alignbyte(d[4], d[3], b); o.y = __builtin_amdgcn_alignbyte(d[5], d[4], b);
        o.z = __builtin_amdgcn_alignbyte(d[6], d[5], b); o.w = __builtin_amdgcn_alignbyte(d[7], d[6], b);
        break;
    }
    return o;
}

// Geometry of a copy of len bytes to dst (any alignment) from a 16-byte
// aligned source: whole destination blocks d4[0..nblk), whose block k holds
// source bytes [r + 16k, r + 16k + 16); and at most 31 edge bytes, the
// first `head` bytes and the bytes from tail0 to len. Without a whole block
// (len <= 30), head = min(len, 16) and tail0 = 16.
struct ShiftPlan {
    uint8_t *dst;
    u32x4 *d4;
    uint64_t len, head, tail0, nblk;
    uint32_t r;
};

__device__ __forceinline__ ShiftPlan shift_plan(uint8_t *dst, uint64_t len)
{
    ShiftPlan q;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t first = (d0 + 15) & ~uintptr_t(15);
    const uintptr_t last = (d0 + len) & ~uintptr_t(15);
    q.dst = dst;
    q.len = len;
    if (first < last) {
        q.head = first - d0;
        q.tail0 = last - d0;
        q.nblk = (last - first) / 16;
    } else {
        q.head = len < 16 ? len : 16;
        q.tail0 = 16;
        q.nblk = 0;
    }
    q.d4 = reinterpret_cast<u32x4 *>(dst + (first - d0));   // derived from dst: stays a global pointer
    q.r = (uint32_t)(q.head & 15);
    return q;
}

// Edge byte e (0..31) of a copy: its offset, or ~0 when there is none
// (e < 16: head bytes; e >= 16: tail bytes).
__device__ __forceinline__ uint64_t edge_offset(uint64_t head, uint64_t tail0, uint64_t len, int e)
{
    const uint64_t j = (e < 16) ? (uint64_t)e : tail0 + (uint64_t)(e - 16);
    const bool ok = (e < 16) ? j < head : j < len;
    return ok ? j : ~0ull;
}

// Whole destination block k of a plan from source blocks lo = k, hi = k + 1.
__device__ __forceinline__ void put_block(const ShiftPlan &q, uint64_t k, u32x4 lo, u32x4 hi)
{
    st_place(q.r == 0 ? lo : extract16(lo, hi, q.r), q.d4 + k);
}

// A tile with more than 64 escapes is placed by a wave of its own. Its
// escape prefix P = (group sums before the tile's group) + (the tile's
// prefix inside its group). Once its count is known, the group sums, the
// in-group prefix and the staged bytes it needs come in one load round:
// with at most 64 * kDirectR escapes, entry `lane` of its staged list and
// exponents, and the tile is written one escape per lane (place_direct);
// otherwise the first KiB of each part of its staging slot (its position
// list or bitmap, and its exponents; 16 bytes per lane) and, with at least
// kValPre escapes, the exponent copy's first round of blocks; then:
//  - positions, a tile with at most kPosListMax escapes: its list is all in
//    the prefetched bytes. Each whole 16-byte destination block of pos[P..]
//    is built from two lanes' bytes (a cross-lane read and a byte funnel)
//    and stored; the partial blocks at the two ends, which the neighbouring
//    tiles share, by byte stores;
//  - positions, a heavier tile: from its escape bitmap, in four passes of
//    2,048 values. Each lane takes 32 values, counts their escapes, and,
//    after a wave scan of the counts, writes their in-chunk positions into
//    the wave's LDS buffer in value order; the buffer's whole 16-byte blocks
//    go out with one store each (the buffer starts on a 16-byte boundary of
//    the destination: the tile's first block is preceded by the entries of
//    the tile before it, which are not written), and the at most 7 entries
//    of a partial last block move to the buffer's start for the next pass;
//  - exponents: like a short position list for the blocks within the
//    prefetched KiB, then 64 blocks per round from the slot (the first
//    round preloaded as above), the loads of each round issued before the
//    stores of the round before it (a wait for a load also waits for every
//    store issued before it).
// Lanes 0..31 store a short list's edge bytes, lanes 32..63 the exponents'.
// The tile's chunk offsets are written by the wave of its run (place_run).
constexpr int kPassVals = 2048;                    // values per bitmap pass: 32 per lane
// With at least this many escapes a tile's exponents span more than 64 whole
// 16-byte destination blocks wherever they start, so the copy's first round
// past the prefetched KiB reads source blocks 63 + lane and 64 + lane.
constexpr uint32_t kValPre = 16 * 64 + 30;
static_assert(kEncTile >= 16 * 128, "the preloaded exponent blocks lie in the slot");
static_assert(kEncTile % kPassVals == 0 && kAux == 16 * 64, "the slot's first KiB is 16 bytes per lane");
static_assert(kEncTile >= 16 * 65, "placement reads at most 65 blocks past a round start");

// Byte j (j < 1024) of the bytes held 16 per lane in pf (lane l: bytes
// 16l..16l + 15); every lane must call it (cross-lane reads).
__device__ __forceinline__ uint32_t byte_from_lanes(u32x4 pf, uint32_t j)
{
    const int sl = (int)((j >> 4) & 63);
    const uint32_t comp = (j >> 2) & 3u;
    const uint32_t x = __shfl(pf.x, sl, 64), y = __shfl(pf.y, sl, 64);
    const uint32_t z = __shfl(pf.z, sl, 64), w = __shfl(pf.w, sl, 64);
    const uint32_t d = comp == 0 ? x : comp == 1 ? y : comp == 2 ? z : w;
    return (d >> (8 * (j & 3))) & 0xFFu;
}

// The next lane's 16 bytes (lane 63 gets its own back).
__device__ __forceinline__ u32x4 next_lane(u32x4 v)
{
    const int nl = ((int)(threadIdx.x & 63) + 1) & 63;
    return u32x4{(uint32_t)__shfl(v.x, nl, 64), (uint32_t)__shfl(v.y, nl, 64), (uint32_t)__shfl(v.z, nl, 64),
                 (uint32_t)__shfl(v.w, nl, 64)};
}

#ifndef UZIP_PLACE_LIGHT_T
#define UZIP_PLACE_LIGHT_T 16
#endif
// One placement wave takes a run of kLightT consecutive tiles: their chunk
// offsets, and the escapes of those with at most 64, go out from one wave in
// runs rather than as short pieces from many. A tile with more escapes is
// placed by the wave of its own index; the other waves past the runs exit at
// once.
constexpr int kLightT = UZIP_PLACE_LIGHT_T;
static_assert(kLightT >= 1 && kLightT <= 64 && 64 % kLightT == 0, "a wave's tiles lie in one group of 2^gshift >= 64 tiles");
#ifndef UZIP_PLACE_WAVES
#define UZIP_PLACE_WAVES 4
#endif
constexpr int kPlaceThreads = 64 * UZIP_PLACE_WAVES;  // one wave per tile, UZIP_PLACE_WAVES per workgroup
#ifndef UZIP_PLACE_DIRECT
#define UZIP_PLACE_DIRECT 2
#endif
// A tile with at most 64 * kDirectR escapes is placed one escape per lane
// (a 2-byte and a 1-byte store each, coalesced across the wave) instead of
// by shifted 16-byte blocks.
constexpr int kDirectR = UZIP_PLACE_DIRECT;
static_assert(kDirectR >= 1 && 64 * kDirectR <= kPosListMax, "a directly placed tile has its positions listed");

// What the first load round fetches for one tile.
struct PlaceIn {
    u32x4 ap, vp;                                  // the slot's first KiB of each part, 16 bytes per lane
    u32x4 bl, bh;                                  // exponent blocks 63 + lane and 64 + lane (m >= kValPre)
    uint32_t dp, dv;                               // entry `lane` of the slot's position list and exponents
};

// A tile with m <= 64 * kDirectR escapes (its positions listed in the slot,
// when the format has them): escape k is written by lane k mod 64, its
// position to pos[P + k] and its exponent to val[P + k]; entry `lane` came
// with the first load round, the others are loaded here.
__device__ __forceinline__ void place_direct(const EncWs &ws, uint8_t *__restrict__ out, const EncParams &p,
                                             uint64_t tile, uint32_t m, uint32_t P, uint64_t M, const PlaceIn &in)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t off_val = p.off_pos + (p.posw ? align256(2 * M) : 0);
    uint16_t *dpos = reinterpret_cast<uint16_t *>(out + p.off_pos) + P;
    uint8_t *dval = out + off_val + P;
    const uint16_t *spos = reinterpret_cast<const uint16_t *>(ws.stage_aux + tile * kAux);
    const uint8_t *sval = ws.stage_val + tile * kEncTile;
    uint32_t ps[kDirectR], vs[kDirectR];
    ps[0] = in.dp;
    vs[0] = in.dv;
#pragma unroll
    for (int r = 1; r < kDirectR; r++) {
        const uint32_t k = lane + 64u * r;
        ps[r] = (p.posw && k < m) ? spos[k] : 0u;
        vs[r] = k < m ? sval[k] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kDirectR; r++) {
        const uint32_t k = lane + 64u * r;
        if (k < m) {
            if (p.posw) st_place((uint16_t)ps[r], dpos + k);
            st_place((uint8_t)vs[r], dval + k);
        }
    }
}

// buf: the wave's LDS position buffer (a pass plus the carried block); bm:
// its 1 KiB LDS copy of a heavy tile's escape bitmap.
__device__ __forceinline__ void place_tile(const EncWs &ws, uint8_t *__restrict__ out, const EncParams &p,
                                           uint64_t tile, uint32_t m, uint32_t P, uint64_t M, const PlaceIn &in,
                                           uint16_t *buf, uint32_t *bm)
{
    const int lane = threadIdx.x & 63;
    const uint64_t t0 = tile * kEncTile;
    const u32x4 ap = in.ap, vp = in.vp;
    const uint8_t *src_v = ws.stage_val + tile * kEncTile;
    const u32x4 *sv4 = reinterpret_cast<const u32x4 *>(src_v);
    const uint64_t off_val = p.off_pos + (p.posw ? align256(2 * M) : 0);
    // ---- positions
    const ShiftPlan qp = shift_plan(out + p.off_pos + 2 * (uint64_t)P, (p.posw && m <= kPosListMax) ? 2 * (uint64_t)m : 0);
    if (qp.nblk) {                                  // a short list, from the prefetched bytes
        const u32x4 nxt = next_lane(ap);
        if ((uint64_t)lane < qp.nblk) st_place(qp.r == 0 ? ap : extract16(ap, nxt, qp.r), qp.d4 + lane);
    }
    if (p.posw && m > (uint32_t)kPosListMax) {      // from the bitmap
        const uint32_t t0m = (uint32_t)(t0 & p.Cmask);
        const uint64_t d0 = p.off_pos + 2 * (uint64_t)P;
        uint8_t *base = out + (d0 & ~15ull);        // destination of buffer entry 0
        const uint32_t phantom = (uint32_t)((d0 & 15u) >> 1);   // entries of the tile before
        uint32_t carry = phantom, done = 0;         // entries waiting at the buffer's start; blocks stored
        // the bitmap to LDS once (16 bytes per lane), read a dword per lane and pass
        reinterpret_cast<u32x4 *>(bm)[lane] = ap;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int c = 0; c < kEncTile / kPassVals; c++) {
            // this lane's 32 values: dword 64c + lane of the bitmap
            uint32_t bits = bm[64 * c + lane];
            const uint32_t cnt = __builtin_popcount(bits);
            const uint32_t inc = wave_inclusive_sum(cnt);
            const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane(inc, 63);
            uint32_t slot = carry + inc - cnt;
            const uint32_t v0 = t0m + (uint32_t)(c * kPassVals) + 32u * (uint32_t)lane;
            while (bits) {
                buf[slot++] = (uint16_t)((v0 + (uint32_t)__builtin_ctz(bits)) & p.Cmask);
                bits &= bits - 1;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint32_t ntot = carry + tot, nb = ntot >> 3;
            for (uint32_t k = (uint32_t)lane; k < nb; k += 64) {
                const u32x4 blk = *reinterpret_cast<const u32x4 *>(buf + 8 * k);
                uint8_t *dst = base + 16 * (uint64_t)(done + k);
                if (done + k == 0 && phantom) {     // the first block: skip the tile before's bytes
                    for (uint32_t b = 2 * phantom; b < 16; b++)
                        dst[b] = (uint8_t)((b < 8 ? (b < 4 ? blk.x : blk.y) : (b < 12 ? blk.z : blk.w)) >> (8 * (b & 3)));
                } else {
                    st_place(blk, reinterpret_cast<u32x4 *>(dst));
                }
            }
            const uint32_t left = ntot & 7u;        // entries of a partial last block
            uint32_t keep = 0;
            if ((uint32_t)lane < left) keep = buf[8 * nb + lane];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if ((uint32_t)lane < left) buf[lane] = (uint16_t)keep;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            done += nb;
            carry = left;
        }
        // the partial last block: its entries' bytes (after the tile
        // before's, if it is also the first block)
        const uint32_t b0 = done == 0 ? 2 * phantom : 0, b1 = 2 * carry;
        if ((uint32_t)lane >= b0 && (uint32_t)lane < b1)
            base[16 * (uint64_t)done + lane] = (uint8_t)(buf[lane >> 1] >> (8 * (lane & 1)));
    }
    // ---- exponents
    const ShiftPlan qv = shift_plan(out + off_val + P, m);
    // blocks whose two source blocks are both prefetched (k + 1 < 64)
    const uint64_t nreg = qv.nblk < 63 ? qv.nblk : 63;
    {
        const u32x4 nxt = next_lane(vp);
        if ((uint64_t)lane < nreg) st_place(qv.r == 0 ? vp : extract16(vp, nxt, qv.r), qv.d4 + lane);
    }
    // edge bytes: this lane's byte (lanes 0..31: a short position list's,
    // 32..63: the exponents'), from the prefetched bytes or else loaded
    const bool is_p = lane < 32;
    const uint64_t ej = edge_offset(is_p ? qp.head : qv.head, is_p ? qp.tail0 : qv.tail0,
                                    is_p ? qp.len : qv.len, lane & 31);
    const uint32_t jj = (ej == ~0ull || ej >= (uint64_t)kAux) ? 0u : (uint32_t)ej;
    const uint32_t bp = byte_from_lanes(ap, jj), bv = byte_from_lanes(vp, jj);
    uint32_t eb = is_p ? bp : bv;
    if (!is_p && ej != ~0ull && ej >= (uint64_t)kAux) eb = src_v[ej];
    // the rest of the exponents, 64 blocks per round from the slot (the
    // first round came with the slot's first KiB when m >= kValPre)
    u32x4 blo = in.bl, bhi = in.bh;
    if (m < kValPre) {
        const uint64_t k = nreg + lane;
        if (k < qv.nblk) {
            blo = sv4[k];
            bhi = sv4[k + 1];
        }
    }
    for (uint64_t k0 = nreg; k0 < qv.nblk; k0 += 64) {
        const uint64_t k = k0 + lane, kn = k + 64;
        u32x4 nblo = blo, nbhi = bhi;
        if (kn < qv.nblk) {
            nblo = sv4[kn];
            nbhi = sv4[kn + 1];
        }
        if (k < qv.nblk) put_block(qv, k, blo, bhi);
        blo = nblo;
        bhi = nbhi;
    }
    if (ej != ~0ull) {
        uint8_t *edst = is_p ? qp.dst : qv.dst;
        edst[ej] = (uint8_t)eb;
    }
}

// The first KiB of each staged part of a heavy tile (16 bytes per lane), as
// far as its count says it is used, and with at least kValPre escapes the
// exponent copy's first round of blocks past that KiB.
__device__ __forceinline__ void place_load_blocks(const EncWs &ws, const EncParams &p, uint64_t tile, uint32_t m,
                                                  PlaceIn &in)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t need_a = p.posw ? (m <= (uint32_t)kPosListMax ? 2 * m : (uint32_t)kAux) : 0u;
    const uint32_t need_v = m < (uint32_t)kAux ? m : (uint32_t)kAux;
    const u32x4 *sv4 = reinterpret_cast<const u32x4 *>(ws.stage_val + tile * kEncTile);
    in.ap = in.vp = in.bl = in.bh = u32x4{0u, 0u, 0u, 0u};
    if (16u * lane < need_a) in.ap = reinterpret_cast<const u32x4 *>(ws.stage_aux + tile * kAux)[lane];
    if (16u * lane < need_v) in.vp = sv4[lane];
    // only blocks that start before the last exponent (a whole destination
    // block never takes bytes from a source block past it)
    if (m >= kValPre) {
        if (16u * (63u + lane) < m) in.bl = sv4[63 + lane];
        if (16u * (64u + lane) < m) in.bh = sv4[64 + lane];
    }
}

// What a tile's own wave loads before it knows its prefix: the tile's
// prefix in its group, and entry `lane` of its staged list and exponents or
// (place_load_blocks) the first KiB of each staged part and more.
__device__ __forceinline__ void place_own_loads(const EncWs &ws, const EncParams &p, uint64_t tile, uint32_t m,
                                                PlaceIn &in, uint32_t &tp)
{
    const uint32_t lane = threadIdx.x & 63;
    tp = ws.tpre[tile];
    if (m <= 64u * kDirectR) {
        in.dp = p.posw ? reinterpret_cast<const uint16_t *>(ws.stage_aux + tile * kAux)[lane] : 0u;
        in.dv = ws.stage_val[tile * kEncTile + lane];
    } else {
        place_load_blocks(ws, p, tile, m, in);
    }
}

// One wave, nt <= kLightT consecutive tiles of one group:
// every tile's count, prefix and first 64 staged entries in one load round;
// a tile with at most 64 escapes is stored from those (one with more is
// placed by its own wave); the chunk offsets of all the tiles go out
// together, 64 per store.
__device__ __forceinline__ void place_run(const EncWs &ws, uint8_t *__restrict__ out, const EncParams &p,
                                              uint64_t tile0, uint32_t nt, uint32_t before_w, uint64_t M)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t m_l = lane < nt ? ws.counts[tile0 + lane] : 0u;
    const uint32_t P_l = before_w + (lane < nt ? ws.tpre[tile0 + lane] : 0u);
    uint32_t e[kLightT];                    // entry `lane` of tile j: exponent << 16 | position
#pragma unroll
    for (int j = 0; j < kLightT; j++) {
        const uint64_t t = tile0 + ((uint32_t)j < nt ? (uint32_t)j : 0u);
        const uint32_t ps = p.posw ? reinterpret_cast<const uint16_t *>(ws.stage_aux + t * kAux)[lane] : 0u;
        e[j] = (uint32_t)ws.stage_val[t * kEncTile + lane] << 16 | ps;
    }
    // the chunks that start in these tiles, lane-strided: the first 256 of
    // their in-tile prefixes come with the same round
    const bool small_c = p.Cmask + 1 < (uint32_t)kEncTile;
    uint64_t c0 = 0, cn = 0;
    uint32_t cp[4] = {0u, 0u, 0u, 0u};
    if (small_c) {
        c0 = (tile0 * kEncTile) >> p.logC;
        cn = ((uint64_t)nt * kEncTile) >> p.logC;
        if (c0 + cn > p.nch) cn = p.nch - c0;
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (lane + 64u * r < cn) cp[r] = ws.chunk_pre[c0 + lane + 64u * r];
    }
    const uint64_t off_val = p.off_pos + (p.posw ? align256(2 * M) : 0);
    uint16_t *dpos = reinterpret_cast<uint16_t *>(out + p.off_pos);
    uint8_t *dval = out + off_val;
#pragma unroll
    for (int j = 0; j < kLightT; j++) {
        // lanes past nt hold m = 0
        const uint32_t m = (uint32_t)__builtin_amdgcn_readlane(m_l, j);
        const uint32_t P = (uint32_t)__builtin_amdgcn_readlane(P_l, j);
        if (m <= 64u && lane < m) {
            if (p.posw) st_place((uint16_t)e[j], dpos + P + lane);
            st_place((uint8_t)(e[j] >> 16), dval + P + lane);
        }
    }
    uint32_t *offs = reinterpret_cast<uint32_t *>(out + p.off_offs);
    if (small_c) {
        // chunk c's tile is c >> (13 - logC) (2^13 words per tile); its
        // prefix is read from that tile's lane with every lane active
        static_assert(kEncTile == 1 << 13, "chunks per tile as a shift");
        const uint32_t sh = 13u - p.logC;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const uint64_t c = lane + 64u * r;
            if (64u * r >= cn) break;
            const uint32_t jt = (uint32_t)(c >> sh);
            const uint32_t Pj = (uint32_t)__shfl((int)P_l, (int)(jt < nt ? jt : 0u), 64);
            if (c < cn) offs[c0 + c] = Pj + cp[r];
        }
        for (uint64_t b = 256; b < cn; b += 64) {
            const uint64_t c = b + lane;
            const uint32_t jt = (uint32_t)(c >> sh);
            const uint32_t Pj = (uint32_t)__shfl((int)P_l, (int)(jt < nt ? jt : 0u), 64);
            if (c < cn) offs[c0 + c] = Pj + ws.chunk_pre[c0 + c];
        }
    } else if (lane < nt) {
        const uint64_t t0 = (tile0 + lane) * kEncTile;
        if ((t0 & p.Cmask) == 0) offs[t0 >> p.logC] = P_l;
    }
}

// Sum of the group sums before group g (lane-strided over the first 256 in
// gs, the rest loaded), as a wave total.
__device__ __forceinline__ uint32_t groups_before(const EncWs &ws, const EncParams &p, const uint32_t gs[4],
                                                  uint64_t g)
{
    const int lane = threadIdx.x & 63;
    uint32_t before = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
        if ((uint64_t)lane + 64 * i < g) before += gs[i];
    for (uint64_t q = (uint64_t)lane + 256; q < g; q += 64) before += ws.gsum[q];
    return (uint32_t)__builtin_amdgcn_readlane(wave_inclusive_sum(before), 63);
}

// The group sums, the first 256 of them 4 per lane in gs, and their total M.
__device__ __forceinline__ uint64_t place_sums(const EncWs &ws, const EncParams &p, uint32_t gs[4])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint64_t q = (uint64_t)lane + 64 * i;
        gs[i] = q < p.ngroups ? ws.gsum[q] : 0u;
    }
    uint32_t all = gs[0] + gs[1] + gs[2] + gs[3];
    for (uint64_t q = (uint64_t)lane + 256; q < p.ngroups; q += 64) all += ws.gsum[q];
    // readlane returns a signed int: through uint32_t, so that an M of 2^31
    // or more is not sign-extended
    return (uint32_t)__builtin_amdgcn_readlane(wave_inclusive_sum(all), 63);
}

// A tile with more than 64 escapes, from its own wave.
__device__ __forceinline__ void place_own(const EncWs &ws, uint8_t *__restrict__ out, const EncParams &p,
                                          uint64_t tile, uint32_t m, uint32_t P, uint64_t M, const PlaceIn &in,
                                          uint16_t *buf, uint32_t *bm)
{
    if (m <= 64u * kDirectR)
        place_direct(ws, out, p, tile, m, P, M, in);
    else
        place_tile(ws, out, p, tile, m, P, M, in, buf, bm);
}

__global__ __launch_bounds__(kPlaceThreads) void k_place_escapes(EncWs ws, uint8_t *__restrict__ out, EncParams p,
                                                                 HeaderParams hp)
{
    // one buffer of positions per wave: a pass, plus the carried partial block
    __shared__ __attribute__((aligned(16))) uint16_t s_pos[kPlaceThreads / 64][kPassVals + 16];
    __shared__ __attribute__((aligned(16))) uint32_t s_bm[kPlaceThreads / 64][kAux / 4];
    // wave-uniform values are moved to scalar registers (readfirstlane)
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t wave = (uint64_t)blockIdx.x * (kPlaceThreads / 64) + wv;
    // Wave w places the tiles of run w (kLightT tiles) that have at most 64
    // escapes and all their chunk offsets, and tile w if it has more. A wave
    // past the runs reads its tile's count alone and, with a tile to place,
    // issues that tile's loads together with the group sums'.
    if (wave * kLightT >= p.ntiles) {
        const uint32_t m = wave < p.ntiles ? ws.counts[wave] : 0u;
        if (m <= 64u) return;
        PlaceIn in;
        uint32_t tp;
        place_own_loads(ws, p, wave, m, in, tp);
        uint32_t gs[4];
        const uint64_t M = place_sums(ws, p, gs);
        place_own(ws, out, p, wave, m, groups_before(ws, p, gs, wave >> p.gshift) + tp, M, in, s_pos[wv], s_bm[wv]);
        return;
    }
    // ---- a run: the group sums (L2-resident) and the count of tile `wave`
    uint32_t gs[4];
    const uint32_t m_own = ws.counts[wave];
    const uint64_t M = place_sums(ws, p, gs);
    {
        const uint64_t tile0 = wave * kLightT;
        const uint32_t nt = (uint32_t)((p.ntiles - tile0 < (uint64_t)kLightT) ? p.ntiles - tile0 : (uint64_t)kLightT);
        place_run(ws, out, p, tile0, nt, groups_before(ws, p, gs, tile0 >> p.gshift), M);
    }
    if (m_own > 64u) {
        PlaceIn in;
        uint32_t tp;
        place_own_loads(ws, p, wave, m_own, in, tp);
        place_own(ws, out, p, wave, m_own, groups_before(ws, p, gs, wave >> p.gshift) + tp, M, in, s_pos[wv],
                  s_bm[wv]);
    }
    if (wave != 0) return;
    const uint64_t off_val = p.off_pos + (p.posw ? align256(2 * M) : 0);
    uint32_t *offs = reinterpret_cast<uint32_t *>(out + p.off_offs);
    // header: template + M + total_bytes
    const uint64_t total = off_val + M;
    uint32_t w = reinterpret_cast<const uint32_t *>(hp.tmpl)[lane];
    if (lane == 6) w = (uint32_t)M;
    if (lane == 7) w = (uint32_t)(M >> 32);
    if (lane == 8) w = (uint32_t)total;
    if (lane == 9) w = (uint32_t)(total >> 32);
    if (p.ddec && lane >= 10 && lane < 14) w = reinterpret_cast<const uint32_t *>(p.ddec)[lane - 10];
    reinterpret_cast<uint32_t *>(out)[lane] = w;
    if (lane == 0) offs[p.nch] = (uint32_t)M;
    // zero padding after each section (each gap is under 256 bytes)
    for (int i = lane; i < 256; i += 64) {
        const uint64_t sm_end = kHeader + p.sm_bytes;
        if (sm_end + i < p.off_codes) out[sm_end + i] = 0;
        for (uint32_t b = 0; b < p.nplanes; b++) {
            const uint64_t codes_end = p.off_codes + b * p.plane + p.code_bytes;
            if (codes_end + i < p.off_codes + (b + 1) * p.plane) out[codes_end + i] = 0;
        }
        const uint64_t offs_end = p.off_offs + 4 * (p.nch + 1);
        if (offs_end + i < p.off_pos) out[offs_end + i] = 0;
        const uint64_t pos_end = p.off_pos + p.posw * M;
        if (pos_end + i < off_val) out[pos_end + i] = 0;
    }
}

// ============================================================== decode ====
// View of one input stream inside a kernel.
struct StreamIn {
    const uint8_t *base;
    uint64_t bytes;       // readable bytes at base
};

// A tile's patch, for the tile's words [t0, t0 + TILE) and NT threads, is
// prepared in two steps, so that its dependent loads take two rounds and
// overlap the tile's dense loads:
//   patch_begin, before the dense loads: the stream's M and the tile's chunk
//     offsets (one per thread);
//   patch_fetch, after the dense loads are issued: the tile's escape range
//     and its first FB * NT escapes, held in registers;
// then patch_scatter applies it to an LDS copy of the tile's exponents (more
// escapes are loaded there, 4 * NT per round, only for tiles with over
// FB * NT of them). Every thread of the workgroup calls all of them. Values
// read from the stream are clamped so that a corrupt stream cannot drive an
// access out of bounds.
struct PatchHead {
    uint64_t M;
    uint32_t lo, hi;      // offsets at the tile's first chunk and past its last one
    uint32_t mine;        // offs[c0 + tid], for tid <= nc (chunks no larger than the tile)
};

template <int FB>
struct PatchFetch {
    uint32_t E0, cnt;     // the tile's escapes are [E0, E0 + cnt)
    uint32_t ps[FB], vv[FB];
    bool live;            // the same in every thread
};

template <int TILE>
__device__ __forceinline__ uint64_t tile_chunks(uint64_t t0, const DecParams &p)
{
    const uint64_t tile_end = (t0 + TILE < p.n) ? t0 + TILE : p.n;
    return ((tile_end - 1) >> p.logC) - (t0 >> p.logC) + 1;
}

template <int TILE, int NT>
__device__ __forceinline__ PatchHead patch_begin(const StreamIn &s, uint64_t t0, const DecParams &p)
{
    static_assert(TILE / 64 + 1 <= NT, "one chunk offset per thread");
    const int tid = threadIdx.x;
    const uint32_t *offs = reinterpret_cast<const uint32_t *>(s.base + p.off_offs) + (t0 >> p.logC);
    PatchHead h;
    h.M = *reinterpret_cast<const uint64_t *>(s.base + 24);
    if (p.C <= (uint32_t)TILE) {
        const uint32_t nc = (uint32_t)tile_chunks<TILE>(t0, p);
        h.lo = offs[0];
        h.hi = offs[nc];
        h.mine = (uint32_t)tid <= nc ? offs[tid] : 0u;
    } else {
        h.lo = offs[0];
        h.hi = offs[1];
        h.mine = 0u;
    }
    return h;
}

template <int TILE, int NT, int FB>
__device__ __forceinline__ PatchFetch<FB> patch_fetch(const StreamIn &s, uint64_t t0, const DecParams &p,
                                                      const PatchHead &h)
{
    const int tid = threadIdx.x;
    PatchFetch<FB> f;
    f.E0 = f.cnt = 0;
    // an M that does not fit the buffer disables the patch
    const uint64_t M = h.M;
    if (M > p.n || p.off_pos + align256(2 * M) + M > s.bytes) {
        f.live = false;
        return f;
    }
    const uint16_t *pos = reinterpret_cast<const uint16_t *>(s.base + p.off_pos);
    const uint8_t *val = s.base + p.off_pos + align256(2 * M);
    uint32_t lo = h.lo, hi = h.hi;                 // M < 2^32 here
    if (hi > (uint32_t)M) hi = (uint32_t)M;
    if (lo > hi) lo = hi;
    if (p.C <= (uint32_t)TILE) {
        f.E0 = lo;
        f.cnt = hi - lo;
    } else {
        // one chunk spans several tiles: find the escapes whose position
        // falls in this tile by an NT-way search over the ascending positions
        const uint32_t rel0 = (uint32_t)(t0 & (uint64_t)(p.C - 1));
        uint32_t res[2];
        for (int side = 0; side < 2; side++) {
            const uint32_t target = rel0 + (side ? (uint32_t)TILE : 0u);
            uint32_t a = lo, b = hi;                // answer in [a, b]
            while (b - a > (uint32_t)NT) {
                const uint32_t step = (b - a + NT - 1) / NT;
                const uint64_t j = a + (uint64_t)tid * step;
                const int below = (j < b) && (pos[j] < target);
                const int cnt = __syncthreads_count(below);
                const uint32_t na = (cnt > 0) ? a + (uint32_t)(cnt - 1) * step + 1 : a;
                uint64_t nb = a + (uint64_t)cnt * step;
                if (nb > b) nb = b;
                a = na;
                b = (uint32_t)nb;
            }
            const uint32_t j = a + tid;
            const int below = (j < b) && (pos[j] < target);
            res[side] = a + (uint32_t)__syncthreads_count(below);
        }
        f.E0 = res[0];
        f.cnt = res[1] - res[0];
    }
    f.live = f.cnt > 0;
#pragma unroll
    for (int u = 0; u < FB; u++) {
        const uint32_t d = (uint32_t)(u * NT + tid);
        f.ps[u] = (d < f.cnt) ? pos[f.E0 + d] : 0xFFFFFFFFu;
        f.vv[u] = (d < f.cnt) ? val[f.E0 + d] : 0u;
    }
    return f;
}

// The exponent form of the patch (BF16 and FP8 tiles): each thread writes the
// exponents it decoded (one byte per word) into an LDS copy of the tile,
// every escape then overwrites its word's byte in place, and each thread
// reads its bytes back before the merge. In order:
//   the threads' exponent bytes and patch_put_offs, a barrier,
//   patch_scatter, a barrier, the threads' reads.
// Only for tiles with escapes (PatchFetch::live, the same in every thread).
template <int TILE>
struct alignas(16) ExpTile {
    uint8_t ex[TILE];
    uint32_t offs[TILE / 64 + 1];
};

template <int TILE, int FB>
__device__ __forceinline__ void patch_put_offs(uint64_t t0, const DecParams &p, const PatchHead &h,
                                               const PatchFetch<FB> &f, ExpTile<TILE> &sh)
{
    const uint32_t tid = threadIdx.x;
    if (p.C > (uint32_t)TILE) return;
    const uint32_t nc = (uint32_t)tile_chunks<TILE>(t0, p), E1 = f.E0 + f.cnt;
    if (tid <= nc) sh.offs[tid] = h.mine > E1 ? E1 : h.mine;
}

// Escape j (position ps, exponent v) overwrites its word's exponent byte.
// Its chunk in the tile is the number of chunk offsets 1..nc-1 at or below
// j: counted against the offsets held in scalar registers (S, unused entries
// ~0) when the tile has at most kLinChunks chunks, else found by a binary
// search over the offsets in LDS.
constexpr int kLinChunks = 8;
template <int TILE>
__device__ __forceinline__ void patch_mark_ex(ExpTile<TILE> &sh, uint64_t t0, uint32_t rem, const DecParams &p,
                                              uint32_t nc, const uint32_t S[kLinChunks - 1], uint32_t j,
                                              uint32_t ps, uint32_t v)
{
    uint32_t li;
    if (p.C <= (uint32_t)TILE) {
        uint32_t a = 0;
        if (nc <= (uint32_t)kLinChunks) {
#pragma unroll
            for (int q = 0; q < kLinChunks - 1; q++) a += (j >= S[q]) ? 1u : 0u;
        } else {
            uint32_t b = nc;                // offs[a] <= j < offs[b]
            while (b - a > 1) {
                const uint32_t mid = (a + b) >> 1;
                if (sh.offs[mid] <= j) a = mid; else b = mid;
            }
        }
        li = (a << p.logC) + ps;
    } else {
        li = ps - (uint32_t)(t0 & (uint64_t)(p.C - 1));   // wraps for a position before the tile
    }
    if (ps < p.C && li < rem) sh.ex[li] = (uint8_t)v;
}

template <int TILE, int NT, int FB>
__device__ void patch_scatter(const StreamIn &s, uint64_t t0, const DecParams &p, const PatchHead &h,
                              const PatchFetch<FB> &f, ExpTile<TILE> &sh)
{
    const int tid = threadIdx.x;
    const uint32_t rem = (uint32_t)((p.n - t0 < (uint64_t)TILE) ? p.n - t0 : (uint64_t)TILE);
    const uint32_t nc = (p.C <= (uint32_t)TILE) ? (uint32_t)tile_chunks<TILE>(t0, p) : 0u;
    // offsets 1..nc-1 to scalar registers: two 16-byte LDS reads of the
    // same words in every lane (entries past nc are not used)
    static_assert(TILE / 64 + 1 >= kLinChunks, "the first kLinChunks offsets fit the table");
    uint32_t S[kLinChunks - 1];
    {
        const u32x4 o0 = *reinterpret_cast<const u32x4 *>(&sh.offs[0]);
        const u32x4 o1 = *reinterpret_cast<const u32x4 *>(&sh.offs[4]);
        const uint32_t o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
        for (int q = 0; q < kLinChunks - 1; q++)
            S[q] = (uint32_t)(q + 1) < nc && nc <= (uint32_t)kLinChunks
                       ? __builtin_amdgcn_readfirstlane(o[q + 1]) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < FB; u++) {
        const uint32_t d = (uint32_t)(u * NT + tid);
        if (d < f.cnt) patch_mark_ex<TILE>(sh, t0, rem, p, nc, S, f.E0 + d, f.ps[u], f.vv[u]);
    }
    if (f.cnt > (uint32_t)(FB * NT)) {
        const uint64_t M = h.M;
        const uint16_t *pos = reinterpret_cast<const uint16_t *>(s.base + p.off_pos) + f.E0;
        const uint8_t *val = s.base + p.off_pos + align256(2 * M) + f.E0;
        for (uint32_t db = FB * NT; db < f.cnt; db += 4 * NT) {
            uint32_t ps[4], vv[4];
            // issue the loads of 4 escapes per thread before using any of them
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint32_t d = db + (uint32_t)(u * NT + tid);
                ps[u] = (d < f.cnt) ? pos[d] : 0xFFFFFFFFu;
                vv[u] = (d < f.cnt) ? val[d] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const uint32_t d = db + (uint32_t)(u * NT + tid);
                if (d < f.cnt) patch_mark_ex<TILE>(sh, t0, rem, p, nc, S, f.E0 + d, ps[u], vv[u]);
            }
        }
    }
}

// A thread's exponent bytes of the group at tile word li0 (a multiple of 8)
// to and from the LDS tile.
template <int TILE>
__device__ __forceinline__ void ex_put8(ExpTile<TILE> &sh, uint32_t li0, const uint32_t e[2])
{
    *reinterpret_cast<u32x2 *>(&sh.ex[li0]) = u32x2{e[0], e[1]};
}
template <int TILE>
__device__ __forceinline__ void ex_get8(const ExpTile<TILE> &sh, uint32_t li0, uint32_t e[2])
{
    const u32x2 v = *reinterpret_cast<const u32x2 *>(&sh.ex[li0]);
    e[0] = v.x;
    e[1] = v.y;
}

template <bool kPatch>
__global__ __launch_bounds__(kDecThreads) void k_decode_tile(StreamIn s, uint16_t *__restrict__ y, DecParams p)
{
    __shared__ ExpTile<kDecTile> sh;
    const int tid = threadIdx.x;
    const uint64_t t0 = (uint64_t)blockIdx.x * kDecTile;
    // words of this tile (scalar), and the tile's bases: lanes index them
    // with 32-bit offsets
    const uint32_t rem = (uint32_t)((p.n - t0 < (uint64_t)kDecTile) ? p.n - t0 : (uint64_t)kDecTile);
    const uint8_t *smt = s.base + kHeader + t0;
    const uint8_t *cdt = s.base + p.off_codes + t0 / 2;
    uint16_t *yt = y + t0;
    uint32_t dec[4] = {p.dec[0], p.dec[1], p.dec[2], p.dec[3]};
    // groups of 8 words: group k covers tile words k*kDecThreads*8 + tid*8,
    // so every load and store instruction covers a contiguous span of the wave
    constexpr int kG = kDecGroups * 2;
    PatchHead ph;
    if (kPatch) ph = patch_begin<kDecTile, kDecThreads>(s, t0, p);
    u32x2 sm[kG];
    uint32_t cd[kG];
#pragma unroll
    for (int k = 0; k < kG; k++) {
        const uint32_t lo = (uint32_t)(k * (kDecThreads * 8) + tid * 8);
        if (lo < rem) {
            // sections are padded to 256 bytes, so a tail group's full loads stay inside them
            sm[k] = ld_stream(reinterpret_cast<const u32x2 *>(smt + lo));
            cd[k] = ld_stream(reinterpret_cast<const uint32_t *>(cdt + lo / 2));
        }
    }
    PatchFetch<kDecFetch> pf;
    if (kPatch) pf = patch_fetch<kDecTile, kDecThreads, kDecFetch>(s, t0, p, ph);
    uint32_t ex[kG][2];
#pragma unroll
    for (int k = 0; k < kG; k++) {
        const uint32_t lo = (uint32_t)(k * (kDecThreads * 8) + tid * 8);
        if (lo < rem) decode8_e(cd[k], dec, ex[k]);
    }
    if (kPatch && pf.live) {
#pragma unroll
        for (int k = 0; k < kG; k++) {
            const uint32_t lo = (uint32_t)(k * (kDecThreads * 8) + tid * 8);
            if (lo < rem) ex_put8(sh, lo, ex[k]);
        }
        patch_put_offs(t0, p, ph, pf, sh);
        __syncthreads();
        patch_scatter<kDecTile, kDecThreads, kDecFetch>(s, t0, p, ph, pf, sh);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kG; k++) {
            const uint32_t lo = (uint32_t)(k * (kDecThreads * 8) + tid * 8);
            if (lo < rem) ex_get8(sh, lo, ex[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < kG; k++) {
        const uint32_t lo = (uint32_t)(k * (kDecThreads * 8) + tid * 8);
        uint32_t out[4];
        if (lo < rem) merge8(sm[k].x, sm[k].y, ex[k], out);
        if (lo + 8 <= rem) {
            u32x4 v = {out[0], out[1], out[2], out[3]};
            st_stream(v, reinterpret_cast<u32x4 *>(yt + lo));
        } else if (lo < rem) {
            for (uint32_t j = 0; j < 8 && lo + j < rem; j++)
                yt[lo + j] = (uint16_t)(out[j >> 1] >> (16 * (j & 1)));
        }
    }
}

// Two-kernel variant, step 2: for every escape, overwrite the exponent field
// of the decoded word in place. One wave per chunk.
__global__ __launch_bounds__(kThreads) void k_patch(StreamIn s, uint16_t *__restrict__ y, DecParams p)
{
    const uint64_t M = *reinterpret_cast<const uint64_t *>(s.base + 24);
    if (M > p.n || p.off_pos + align256(2 * M) + M > s.bytes) return;
    const uint32_t *offs = reinterpret_cast<const uint32_t *>(s.base + p.off_offs);
    const uint16_t *pos = reinterpret_cast<const uint16_t *>(s.base + p.off_pos);
    const uint8_t *val = s.base + p.off_pos + align256(2 * M);
    const int lane = threadIdx.x & 63;
    const uint64_t waves = (uint64_t)gridDim.x * (kThreads / 64);
    for (uint64_t c = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); c < p.nch; c += waves) {
        uint64_t j0 = offs[c], j1 = offs[c + 1];
        if (j1 > M) j1 = M;
        for (uint64_t j = j0 + lane; j < j1; j += 64) {
            const uint32_t ps = pos[j];
            const uint64_t i = (c << p.logC) + ps;
            if (ps < p.C && i < p.n) {
                const uint32_t w = y[i];
                y[i] = (uint16_t)((w & 0x807Fu) | ((uint32_t)val[j] << 7));
            }
        }
    }
}

// ============================================================== reduce ====
// LDS: the exponent tiles (used while decoding) and the escape list (used
// while encoding) are never live at the same time.
struct ExpTile2 {
    ExpTile<kEncTile> a, b;
};
union ReduceLds {
    ExpTile2 ex;
    EscBuf esc;
};

// One tile of the pairwise reduce: both inputs decoded and patched, summed
// in binary32, rounded to BF16 and encoded. Built for 5 waves per SIMD (at
// most 96 registers, which the compiler meets without spilling).
__global__ __launch_bounds__(kEncThreads, 5) void k_reduce_tile(StreamIn sa, StreamIn sb, uint8_t *__restrict__ out,
                                                                EncWs ws, EncParams ep, DecParams dp)
{
    __shared__ EncShared esh;
    __shared__ ReduceLds lds;
    const int tid = threadIdx.x;
    const uint64_t tile = blockIdx.x;
    const uint64_t t0 = tile * kEncTile;
    uint32_t dec[4] = {dp.dec[0], dp.dec[1], dp.dec[2], dp.dec[3]};
    const uint32_t rem = enc_tile_words(t0, ep);
    const PatchHead ha = patch_begin<kEncTile, kEncThreads>(sa, t0, dp);
    const PatchHead hb = patch_begin<kEncTile, kEncThreads>(sb, t0, dp);
    const uint8_t *smta = sa.base + kHeader + t0, *cdta = sa.base + dp.off_codes + t0 / 2;
    const uint8_t *smtb = sb.base + kHeader + t0, *cdtb = sb.base + dp.off_codes + t0 / 2;
    u32x2 sma[kEncGroups], smb[kEncGroups];
    uint32_t cda[kEncGroups], cdb[kEncGroups];
#pragma unroll
    for (int k = 0; k < kEncGroups; k++) {
        const uint32_t lo = (uint32_t)(k * (kEncThreads * 8) + tid * 8);
        if (lo < rem) {
            sma[k] = ld_stream(reinterpret_cast<const u32x2 *>(smta + lo));
            cda[k] = ld_stream(reinterpret_cast<const uint32_t *>(cdta + lo / 2));
            smb[k] = ld_stream(reinterpret_cast<const u32x2 *>(smtb + lo));
            cdb[k] = ld_stream(reinterpret_cast<const uint32_t *>(cdtb + lo / 2));
        }
    }
    const PatchFetch<kRedFetch> fa = patch_fetch<kEncTile, kEncThreads, kRedFetch>(sa, t0, dp, ha);
    const PatchFetch<kRedFetch> fb = patch_fetch<kEncTile, kEncThreads, kRedFetch>(sb, t0, dp, hb);
    // exponents of both inputs; groups past the end decode to the word 0
    uint32_t ea[kEncGroups][2], eb[kEncGroups][2];
#pragma unroll
    for (int k = 0; k < kEncGroups; k++) {
        const uint32_t lo = (uint32_t)(k * (kEncThreads * 8) + tid * 8);
        if (lo < rem) {
            decode8_e(cda[k], dec, ea[k]);
            decode8_e(cdb[k], dec, eb[k]);
        } else {
            sma[k] = smb[k] = u32x2{0u, 0u};
            ea[k][0] = ea[k][1] = eb[k][0] = eb[k][1] = 0u;
        }
    }
    // the code table goes to LDS after the data loads are in flight (one copy
    // for the workgroup: the barriers below publish it)
    load_shared_lut(esh, ep.lut);
    // both inputs' escapes patched in one pass over two exponent tiles
    if (fa.live || fb.live) {
#pragma unroll
        for (int k = 0; k < kEncGroups; k++) {
            const uint32_t lo = (uint32_t)(k * (kEncThreads * 8) + tid * 8);
            if (fa.live) ex_put8(lds.ex.a, lo, ea[k]);
            if (fb.live) ex_put8(lds.ex.b, lo, eb[k]);
        }
        if (fa.live) patch_put_offs(t0, dp, ha, fa, lds.ex.a);
        if (fb.live) patch_put_offs(t0, dp, hb, fb, lds.ex.b);
        __syncthreads();
        if (fa.live) patch_scatter<kEncTile, kEncThreads, kRedFetch>(sa, t0, dp, ha, fa, lds.ex.a);
        if (fb.live) patch_scatter<kEncTile, kEncThreads, kRedFetch>(sb, t0, dp, hb, fb, lds.ex.b);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kEncGroups; k++) {
            const uint32_t lo = (uint32_t)(k * (kEncThreads * 8) + tid * 8);
            if (fa.live) ex_get8(lds.ex.a, lo, ea[k]);
            if (fb.live) ex_get8(lds.ex.b, lo, eb[k]);
        }
    } else {
        __syncthreads();                       // publishes the code table
    }
    uint32_t r[kEncGroups][4];
#pragma unroll
    for (int k = 0; k < kEncGroups; k++) {
        float fa[8], fb[8];
        floats8(sma[k].x, sma[k].y, ea[k], fa);
        floats8(smb[k].x, smb[k].y, eb[k], fb);
        bool nan = false;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            bool n;
            r[k][q] = bf16x2_rne_fast(fa[2 * q] + fb[2 * q], fa[2 * q + 1] + fb[2 * q + 1], n);
            nan = nan || n;
        }
        if (__ballot(nan) != 0ull) {         // a NaN sum in the wave: the full rule for the group
            floats8(sma[k].x, sma[k].y, ea[k], fa);
            floats8(smb[k].x, smb[k].y, eb[k], fb);
#pragma unroll
            for (int q = 0; q < 4; q++) r[k][q] = bf16x2_rne(fa[2 * q] + fb[2 * q], fa[2 * q + 1] + fb[2 * q + 1]);
        }
    }
    // encode_dense_rank writes the escape list only after its first barrier,
    // which every thread reaches after its last read of the patch map
    uint32_t cstart[kEncGroups];
    const uint32_t m = encode_dense_rank<kCodeNib>(r, t0, rem, out, ep, esh, lds.esc, cstart,
                                                   ws.stage_aux + tile * kAux);
    stage_escapes(m, cstart, t0, tile, ws, ep, lds.esc);
}

// k-input reduce: the inputs of one call, passed by value.
struct StreamSet {
    StreamIn in[UZIP_MAX_K];
    uint32_t k;
};

// Dense loads of one input's part of a tile: per group, 8 sign-mantissa
// bytes and 4 code bytes.
template <int NT, int NG>
struct DenseIn {
    u32x2 sm[NG];
    uint32_t cd[NG];
};

template <int NT, int NG>
__device__ __forceinline__ void load_dense(const StreamIn &s, uint64_t t0, uint32_t rem, const DecParams &p,
                                           DenseIn<NT, NG> &d)
{
    const int tid = threadIdx.x;
    const uint8_t *smt = s.base + kHeader + t0, *cdt = s.base + p.off_codes + t0 / 2;
#pragma unroll
    for (int k = 0; k < NG; k++) {
        const uint32_t lo = (uint32_t)(k * (NT * 8) + tid * 8);
        if (lo < rem) {
            d.sm[k] = ld_stream(reinterpret_cast<const u32x2 *>(smt + lo));
            d.cd[k] = ld_stream(reinterpret_cast<const uint32_t *>(cdt + lo / 2));
        } else {
            d.sm[k] = u32x2{0u, 0u};
            d.cd[k] = 0u;
        }
    }
}

constexpr int kRkThreads = kEncThreads;
constexpr int kRkGroups = kEncTile / (kRkThreads * 8);
static_assert(kRkThreads * kRkGroups * 8 == kEncTile && kRkGroups * (kRkThreads / 64) <= 16, "k-input reduce tile shape");

// One tile of the k-input reduce, kRkThreads threads per tile, each keeping
// binary32 sums of its kRkGroups groups of 8 words. The inputs are taken two
// at a time: both are loaded and decoded, their escapes are patched through
// the two LDS exponent tiles between one pair of barriers (half the barriers
// of one input at a time), and they are added to the sums in input order.
// The sums start at -0.0 (-0.0 + x is x for every binary32 x but a NaN,
// which stays a NaN: the first add sets them exactly). They are rounded once
// to BF16 and encoded like k_reduce_tile.
__global__ __launch_bounds__(kRkThreads) void k_reduce_k_tile(StreamSet ss, uint8_t *__restrict__ out,
                                                              EncWs ws, EncParams ep, DecParams dp)
{
    __shared__ EncSharedT<kRkThreads, kRkGroups> esh;
    __shared__ ReduceLds lds;
    const int tid = threadIdx.x;
    const uint64_t tile = blockIdx.x;
    const uint64_t t0 = tile * kEncTile;
    const uint32_t rem = enc_tile_words(t0, ep);
    uint32_t dec[4] = {dp.dec[0], dp.dec[1], dp.dec[2], dp.dec[3]};
    float acc[kRkGroups][8];
#pragma unroll
    for (int k = 0; k < kRkGroups; k++)
#pragma unroll
        for (int q = 0; q < 8; q++) acc[k][q] = -0.0f;
    bool synced = false;                                // a barrier has published the code table
    for (uint32_t i = 0; i < ss.k; i += 2) {
        const bool two = i + 1 < ss.k;                  // the same in every thread
        const StreamIn s0 = ss.in[i];
        const StreamIn s1 = ss.in[two ? i + 1 : i];
        const PatchHead h0 = patch_begin<kEncTile, kRkThreads>(s0, t0, dp);
        PatchHead h1 = h0;
        DenseIn<kRkThreads, kRkGroups> d0, d1;
        load_dense(s0, t0, rem, dp, d0);
        if (two) {
            h1 = patch_begin<kEncTile, kRkThreads>(s1, t0, dp);
            load_dense(s1, t0, rem, dp, d1);
        }
        if (i == 0) load_shared_lut(esh, ep.lut);   // after the first data loads are in flight
        const PatchFetch<kRedFetch> f0 = patch_fetch<kEncTile, kRkThreads, kRedFetch>(s0, t0, dp, h0);
        PatchFetch<kRedFetch> f1 = f0;
        f1.live = false;
        if (two) f1 = patch_fetch<kEncTile, kRkThreads, kRedFetch>(s1, t0, dp, h1);
        uint32_t e0[kRkGroups][2], e1[kRkGroups][2];
#pragma unroll
        for (int k = 0; k < kRkGroups; k++) {
            decode8_e(d0.cd[k], dec, e0[k]);
            if (two) decode8_e(d1.cd[k], dec, e1[k]);
        }
        if (f0.live || f1.live) {
            // each thread rewrites only its own bytes here, which no thread
            // reads after the previous pair's second barrier but itself
#pragma unroll
            for (int k = 0; k < kRkGroups; k++) {
                const uint32_t lo = (uint32_t)(k * (kRkThreads * 8) + tid * 8);
                if (f0.live) ex_put8(lds.ex.a, lo, e0[k]);
                if (f1.live) ex_put8(lds.ex.b, lo, e1[k]);
            }
            if (f0.live) patch_put_offs(t0, dp, h0, f0, lds.ex.a);
            if (f1.live) patch_put_offs(t0, dp, h1, f1, lds.ex.b);
            __syncthreads();
            if (f0.live) patch_scatter<kEncTile, kRkThreads, kRedFetch>(s0, t0, dp, h0, f0, lds.ex.a);
            if (f1.live) patch_scatter<kEncTile, kRkThreads, kRedFetch>(s1, t0, dp, h1, f1, lds.ex.b);
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kRkGroups; k++) {
                const uint32_t lo = (uint32_t)(k * (kRkThreads * 8) + tid * 8);
                if (f0.live) ex_get8(lds.ex.a, lo, e0[k]);
                if (f1.live) ex_get8(lds.ex.b, lo, e1[k]);
            }
            synced = true;
        }
        // inputs i, then i + 1: the sums keep the input order
#pragma unroll
        for (int k = 0; k < kRkGroups; k++) {
            float f[8];
            floats8(d0.sm[k].x, d0.sm[k].y, e0[k], f);
#pragma unroll
            for (int j = 0; j < 8; j++) acc[k][j] += f[j];
        }
        if (two) {
#pragma unroll
            for (int k = 0; k < kRkGroups; k++) {
                float f[8];
                floats8(d1.sm[k].x, d1.sm[k].y, e1[k], f);
#pragma unroll
                for (int j = 0; j < 8; j++) acc[k][j] += f[j];
            }
        }
    }
    uint32_t r[kRkGroups][4];
#pragma unroll
    for (int k = 0; k < kRkGroups; k++) {
        const uint32_t lo = (uint32_t)(k * (kRkThreads * 8) + tid * 8);
        bool nan = false;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            bool n;
            r[k][q] = bf16x2_rne_fast(acc[k][2 * q], acc[k][2 * q + 1], n);
            nan = nan || n;
        }
        if (__ballot(nan) != 0ull) {         // a NaN sum in the wave: the full rule for the group
#pragma unroll
            for (int q = 0; q < 4; q++) r[k][q] = bf16x2_rne(acc[k][2 * q], acc[k][2 * q + 1]);
        }
#pragma unroll
        for (int q = 0; q < 4; q++)
            if (lo >= rem) r[k][q] = 0u;
    }
    if (!synced) __syncthreads();
    uint32_t cstart[kRkGroups];
    const uint32_t m = encode_dense_rank<kCodeNib, kRkThreads, kRkGroups>(r, t0, rem, out, ep, esh, lds.esc, cstart,
                                                   ws.stage_aux + tile * kAux);
    stage_escapes<kRkGroups, 8, kRkThreads>(m, cstart, t0, tile, ws, ep, lds.esc);
}

// ============================================================ FP8 E5M2 ====
// The E5M2 variant ("SplitZip: Ultra Fast Lossless KV Compression for
// Disaggregated LLM Serving", section 4.2 / appendix C): the 5-bit exponent
// of each byte, e = (x >> 2) & 0x1f, takes a 4-bit Top-16 code; the other
// three bits, a = sign << 2 | mantissa, are packed 3 bits per value (value i
// at bits 3i..3i+2 of the section, least significant bit first). Escapes,
// offsets, placement and container are the BF16 ones.
constexpr int k8Vals = 32;                 // values per thread: 32 B of input
static_assert(kEncThreads * k8Vals == kEncTile, "the FP8 encode tile is the BF16 one (staging slots)");
constexpr int k8DecThreads = 128;
constexpr int k8DecTile = k8DecThreads * k8Vals;

// Three bits (sign, mantissa) of each byte of w, one per byte.
__device__ __forceinline__ uint32_t signmant8x4(uint32_t w)
{
    return bfi(0x03030303u, w, w >> 5) & 0x07070707u;
}

// Rebuild 4 E5M2 bytes from their 3 kept bits (a) and exponents (e), one per byte.
__device__ __forceinline__ uint32_t merge8x4(uint32_t a, uint32_t e)
{
    return ((a & 0x04040404u) << 5) | ((e & 0x1F1F1F1Fu) << 2) | (a & 0x03030303u);
}

__global__ __launch_bounds__(kEncThreads) void k8_encode_tile(const uint8_t *__restrict__ x,
                                                              uint8_t *__restrict__ out, EncWs ws, EncParams p)
{
    __shared__ uint32_t wtot[kEncThreads / 64];
    __shared__ EscBuf eb;
    __shared__ uint32_t s_lut[8];          // the 32 code-table bytes
    __shared__ __attribute__((aligned(16))) uint8_t s_exb[kEncThreads * k8Vals];   // each lane's exponents
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t tile = blockIdx.x;
    const uint64_t t0 = tile * kEncTile;
    const uint32_t rem = enc_tile_words(t0, p);
    const uint32_t lo = (uint32_t)tid * k8Vals;               // this thread's first value in the tile
    uint32_t w[8];
    if (lo + k8Vals <= rem) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + t0 + lo);
        const u32x4 v0 = ld_stream(src), v1 = ld_stream(src + 1);
        w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w;
        w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
    } else {
#pragma unroll
        for (int q = 0; q < 8; q++) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const uint32_t i = lo + 4 * q + b;
                if (i < rem) v |= (uint32_t)x[t0 + i] << (8 * b);
            }
            w[q] = v;
        }
    }
    // the table goes to LDS while the input loads are in flight
    if (tid < 8) s_lut[tid] = reinterpret_cast<const uint32_t *>(p.lut)[tid];
    __syncthreads();
    const uint8_t *tb = reinterpret_cast<const uint8_t *>(s_lut);
    uint32_t L[8], E[8], A[8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
        E[q] = (w[q] >> 2) & 0x1F1F1F1Fu;
        L[q] = (uint32_t)tb[(w[q] >> 2) & 0x1Fu] | ((uint32_t)tb[(w[q] >> 10) & 0x1Fu] << 8) |
               ((uint32_t)tb[(w[q] >> 18) & 0x1Fu] << 16) | ((uint32_t)tb[(w[q] >> 26) & 0x1Fu] << 24);
        A[q] = signmant8x4(w[q]);
    }
    if (lo + k8Vals > rem) {                     // tail: values past n are not escapes and take code 0
#pragma unroll
        for (int q = 0; q < 8; q++)
#pragma unroll
            for (int b = 0; b < 4; b++)
                if (lo + 4 * q + b >= rem) L[q] &= ~(0xFFu << (8 * b));
    }
    Codes8 c8[4];
#pragma unroll
    for (int q = 0; q < 4; q++) c8[q] = codes_flags8(L[2 * q], L[2 * q + 1]);
    if (lo < rem) {
        u32x4 cw;
        cw.x = c8[0].codes;
        cw.y = c8[1].codes;
        cw.z = c8[2].codes;
        cw.w = c8[3].codes;
        st_stream(cw, reinterpret_cast<u32x4 *>(out + p.off_codes + t0 / 2 + lo / 2));
        uint32_t c[8];
#pragma unroll
        for (int q = 0; q < 8; q++) c[q] = pack12(A[q]);
        const uint32_t sw[3] = {c[0] | (c[1] << 12) | (c[2] << 24),
                                (c[2] >> 8) | (c[3] << 4) | (c[4] << 16) | (c[5] << 28),
                                (c[5] >> 4) | (c[6] << 8) | (c[7] << 20)};
        uint8_t *smb = out + kHeader + (t0 + lo) / 8 * 3;
        if (lo + k8Vals <= rem) {
            uint32_t *smw = reinterpret_cast<uint32_t *>(smb);
            st_stream(sw[0], smw);
            st_stream(sw[1], smw + 1);
            st_stream(sw[2], smw + 2);
        } else {
            // the 12 bytes may run past the section (its end is a multiple of
            // 256, not of 12) into the codes that tile 0 writes: store only the
            // bytes that hold valid values
            const uint32_t nb = (3 * (rem - lo) + 7) / 8;
            for (uint32_t b = 0; b < nb; b++) smb[b] = (uint8_t)(sw[b >> 2] >> (8 * (b & 3)));
        }
    }
    // escapes: the lane's count, its rank in the tile (values are in lane
    // order), the list in LDS
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) cnt += __builtin_popcount(c8[q].flags);
    uint32_t pre = 0, wt = 0;
    if (__ballot(cnt != 0) != 0ull) {
        const uint32_t inc = wave_inclusive_sum(cnt);
        pre = inc - cnt;
        wt = __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0) wtot[wave] = wt;
    __syncthreads();
    uint32_t base = 0, m = 0;
#pragma unroll
    for (int v = 0; v < kEncThreads / 64; v++) {
        if (v < wave) base += wtot[v];
        m += wtot[v];
    }
    uint32_t rank = base + pre;
    const uint32_t g0m = ((uint32_t)(t0 & p.Cmask) + lo) & p.Cmask;   // a multiple of 32, below C
    uint32_t cstart[1];
    cstart[0] = (lo < rem && g0m == 0) ? rank : ~0u;
    // positions listed for a tile with at most kPosListMax escapes, else the
    // tile's escape bitmap: this lane's 32 values are its bytes 4 tid..4 tid + 3
    const bool lst = m <= (uint32_t)kPosListMax;
    // the lane's escape flags, bit j for value j
    uint32_t fm = flags_byte(c8[0].flags) | (flags_byte(c8[1].flags) << 8) | (flags_byte(c8[2].flags) << 16) |
                  (flags_byte(c8[3].flags) << 24);
    if (!lst) reinterpret_cast<uint32_t *>(ws.stage_aux + tile * kAux)[tid] = fm;
    // one loop over the lane's 32 values (as often as the wave's busiest
    // lane has escapes), each exponent read back from the lane's own 32
    // exponent bytes in LDS
    if (fm) {
        u32x4 *mine = reinterpret_cast<u32x4 *>(&s_exb[tid * k8Vals]);
        mine[0] = u32x4{E[0], E[1], E[2], E[3]};
        mine[1] = u32x4{E[4], E[5], E[6], E[7]};
    }
    while (fm) {
        const uint32_t j = __builtin_ctz(fm);
        if (lst) eb.pos[rank] = (uint16_t)(g0m + j);
        eb.val[rank] = s_exb[tid * k8Vals + j];
        rank++;
        fm &= fm - 1;
    }
    stage_escapes<1, k8Vals>(m, cstart, t0, tile, ws, p, eb);
}

template <bool kPatch>
__global__ __launch_bounds__(k8DecThreads) void k8_decode_tile(StreamIn s, uint8_t *__restrict__ y, DecParams p)
{
    __shared__ ExpTile<k8DecTile> sh;
    __shared__ u32x4 xp[k8DecThreads / 64][128];     // one wave's 2 KiB of output, for contiguous stores
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t t0 = (uint64_t)blockIdx.x * k8DecTile;
    const uint32_t rem = (uint32_t)((p.n - t0 < (uint64_t)k8DecTile) ? p.n - t0 : (uint64_t)k8DecTile);
    const uint32_t lo = (uint32_t)tid * k8Vals;
    uint32_t dec[4] = {p.dec[0], p.dec[1], p.dec[2], p.dec[3]};
    PatchHead ph;
    if (kPatch) ph = patch_begin<k8DecTile, k8DecThreads>(s, t0, p);
    uint32_t sm[3] = {0u, 0u, 0u};
    u32x4 cd = {0u, 0u, 0u, 0u};
    if (lo < rem) {
        // sections are padded to 256 bytes, so a tail group's full loads stay inside them
        const uint32_t *smw = reinterpret_cast<const uint32_t *>(s.base + kHeader + (t0 + lo) / 8 * 3);
        sm[0] = ld_stream(smw);
        sm[1] = ld_stream(smw + 1);
        sm[2] = ld_stream(smw + 2);
        cd = ld_stream(reinterpret_cast<const u32x4 *>(s.base + p.off_codes + t0 / 2 + lo / 2));
    }
    PatchFetch<kDecFetch> pf;
    if (kPatch) pf = patch_fetch<k8DecTile, k8DecThreads, kDecFetch>(s, t0, p, ph);
    const uint32_t c[8] = {sm[0] & 0xFFFu, (sm[0] >> 12) & 0xFFFu, (sm[0] >> 24) | ((sm[1] & 0xFu) << 8),
                           (sm[1] >> 4) & 0xFFFu, (sm[1] >> 16) & 0xFFFu, (sm[1] >> 28) | ((sm[2] & 0xFFu) << 4),
                           (sm[2] >> 8) & 0xFFFu, sm[2] >> 20};
    const uint32_t cw[4] = {cd.x, cd.y, cd.z, cd.w};
    uint32_t e[8];
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const uint32_t lo4 = cw[h] & 0x0F0F0F0Fu;             // codes of values 8h + 0, 2, 4, 6
        const uint32_t hi4 = (cw[h] >> 4) & 0x0F0F0F0Fu;      // 8h + 1, 3, 5, 7
        e[2 * h] = dec4(dec, perm(hi4, lo4, 0x05010400u));
        e[2 * h + 1] = dec4(dec, perm(hi4, lo4, 0x07030602u));
    }
    if (kPatch && pf.live) {
        // this thread's 32 exponent bytes to the LDS tile, where each escape
        // overwrites its own, and back
        u32x4 *ex4 = reinterpret_cast<u32x4 *>(&sh.ex[lo]);
        ex4[0] = u32x4{e[0], e[1], e[2], e[3]};
        ex4[1] = u32x4{e[4], e[5], e[6], e[7]};
        patch_put_offs(t0, p, ph, pf, sh);
        __syncthreads();
        patch_scatter<k8DecTile, k8DecThreads, kDecFetch>(s, t0, p, ph, pf, sh);
        __syncthreads();
        const u32x4 r0 = ex4[0], r1 = ex4[1];
        e[0] = r0.x; e[1] = r0.y; e[2] = r0.z; e[3] = r0.w;
        e[4] = r1.x; e[5] = r1.y; e[6] = r1.z; e[7] = r1.w;
    }
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; q++) out[q] = merge8x4(unpack12(c[q]), e[q]);
    uint8_t *yt = y + t0;
    const uint32_t wlo = (uint32_t)wave * 64u * k8Vals;          // the wave's first value in the tile
    if (wlo + 64u * k8Vals <= rem) {
        // the wave's 2 KiB go through LDS so that each store instruction
        // covers 1 KiB without gaps: lane l writes its 32 bytes at 32 l,
        // then stores the 16 bytes at 16 l and at 1024 + 16 l
        xp[wave][2 * lane] = u32x4{out[0], out[1], out[2], out[3]};
        xp[wave][2 * lane + 1] = u32x4{out[4], out[5], out[6], out[7]};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        u32x4 *dst = reinterpret_cast<u32x4 *>(yt + wlo);
        st_stream(xp[wave][lane], dst + lane);
        st_stream(xp[wave][64 + lane], dst + 64 + lane);
    } else if (lo + k8Vals <= rem) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(yt + lo);
        st_stream(u32x4{out[0], out[1], out[2], out[3]}, dst);
        st_stream(u32x4{out[4], out[5], out[6], out[7]}, dst + 1);
    } else if (lo < rem) {
        for (uint32_t i = 0; i < k8Vals && lo + i < rem; i++) yt[lo + i] = (uint8_t)(out[i >> 2] >> (8 * (i & 3)));
    }
}

// ================================================= Top-15 + sentinel ====
// "SplitZip" section 3.4 / Table 6: code 15 marks an escape, whose exponent
// is the next stored one of its chunk; no positions are stored. Encoding is
// k_encode_tile with a code table that gives every exponent outside
// dec[0..14] code 15 and the escape flag, and placement without positions.
// Decoding needs each sentinel's rank among the sentinels of its chunk: a
// tile (whose chunks all start inside it: C <= tile) loads M, its chunk
// offsets and its dense bytes, then its contiguous run of stored exponents
// into LDS; the sentinels of each group of 8 words are ranked in position
// order (wave scans, wave totals in LDS), and each takes its exponent from
// LDS.
constexpr int kS15Threads = 128;
constexpr int kS15Groups = 4;              // groups of 8 words per thread
constexpr int kS15Tile = kS15Threads * kS15Groups * 8;

__global__ __launch_bounds__(kS15Threads) void k_s15_decode_tile(StreamIn s, uint16_t *__restrict__ y, DecParams p)
{
    __shared__ uint8_t svals[kS15Tile];
    __shared__ uint32_t wtot[kS15Groups][kS15Threads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t t0 = (uint64_t)blockIdx.x * kS15Tile;
    const uint32_t rem = (uint32_t)((p.n - t0 < (uint64_t)kS15Tile) ? p.n - t0 : (uint64_t)kS15Tile);
    // first loads: M, the tile's chunk offsets (C <= tile: the tile starts a chunk)
    const uint64_t M = *reinterpret_cast<const uint64_t *>(s.base + 24);
    const uint32_t *offs = reinterpret_cast<const uint32_t *>(s.base + p.off_offs) + (t0 >> p.logC);
    const uint32_t nc = (uint32_t)(((t0 + rem - 1) >> p.logC) - (t0 >> p.logC) + 1);
    const uint32_t o0 = offs[0], o1 = offs[nc];
    const uint8_t *smt = s.base + kHeader + t0;
    const uint8_t *cdt = s.base + p.off_codes + t0 / 2;
    uint32_t dec[4] = {p.dec[0], p.dec[1], p.dec[2], p.dec[3]};
    u32x2 sm[kS15Groups];
    uint32_t cd[kS15Groups];
#pragma unroll
    for (int k = 0; k < kS15Groups; k++) {
        const uint32_t lo = (uint32_t)(k * (kS15Threads * 8) + tid * 8);
        sm[k] = u32x2{0u, 0u};
        cd[k] = 0u;
        if (lo < rem) {
            sm[k] = ld_stream(reinterpret_cast<const u32x2 *>(smt + lo));
            cd[k] = ld_stream(reinterpret_cast<const uint32_t *>(cdt + lo / 2));
        }
    }
    // the tile's stored exponents: [E0, E1), clamped so that a corrupt stream
    // reads inside the buffer
    const bool okM = M <= p.n && p.off_pos + M <= s.bytes;
    uint32_t E1 = okM ? (o1 < (uint32_t)M ? o1 : (uint32_t)M) : 0u;
    uint32_t E0 = o0 < E1 ? o0 : E1;
    if (E1 - E0 > rem) E1 = E0 + rem;
    const uint32_t cnt = E1 - E0;
    const uint8_t *val = s.base + p.off_pos + E0;
    for (uint32_t j = tid; j < cnt; j += kS15Threads) svals[j] = val[j];
    // sentinels: nibbles equal to 15, one flag per word at bit 4i
    uint32_t f[kS15Groups], pre[kS15Groups];
#pragma unroll
    for (int k = 0; k < kS15Groups; k++) {
        const uint32_t lo = (uint32_t)(k * (kS15Threads * 8) + tid * 8);
        uint32_t t = cd[k] & (cd[k] >> 1) & (cd[k] >> 2) & (cd[k] >> 3) & 0x11111111u;
        if (lo + 8 > rem) t = lo < rem ? t & ((1u << (4 * (rem - lo))) - 1u) : 0u;
        f[k] = t;
        const uint32_t c = __builtin_popcount(t);
        uint32_t pr = 0, wt = 0;
        if (__ballot(c != 0) != 0ull) {
            const uint32_t inc = wave_inclusive_sum(c);
            pr = inc - c;
            wt = __builtin_amdgcn_readlane(inc, 63);
        }
        pre[k] = pr;
        if (lane == 0) wtot[k][wave] = wt;
    }
    uint32_t ex[kS15Groups][2];
#pragma unroll
    for (int k = 0; k < kS15Groups; k++) decode8_e(cd[k], dec, ex[k]);
    __syncthreads();
    uint32_t run = 0;
    uint32_t out[kS15Groups][4];
#pragma unroll
    for (int k = 0; k < kS15Groups; k++) {
        uint32_t base = run;
#pragma unroll
        for (int w = 0; w < kS15Threads / 64; w++) {
            if (w < wave) base += wtot[k][w];
            run += wtot[k][w];
        }
        if (__ballot(f[k] != 0) != 0ull) {
            // word i's stored exponent (if it is a sentinel) is at rank
            // r + (sentinels before it); every word reads one, in bounds
            // (at most the tile's word count), kept only for sentinels
            const uint32_t r = base + pre[k];
            uint32_t z = (f[k] | (f[k] >> 3)) & 0x03030303u;      // flag 4i -> bit i
            z = (z | (z >> 6)) & 0x000F000Fu;
            z = (z | (z >> 12)) & 0xFFu;
#pragma unroll
            for (int q = 0; q < 2; q++) {
                uint32_t pd = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int j = 4 * q + i;
                    const uint32_t rj = r + __builtin_popcount(f[k] & ((1u << (4 * j)) - 1u));
                    const uint32_t v = rj < cnt ? (uint32_t)svals[rj] : 0u;
                    pd |= v << (8 * i);
                }
                // sentinels with no stored exponent (a corrupt stream) keep
                // the looked-up one
                uint32_t zq = (z >> (4 * q)) & 0xFu;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (r + __builtin_popcount(f[k] & ((1u << (4 * (4 * q + i))) - 1u)) >= cnt) zq &= ~(1u << i);
                ex[k][q] = bfi(bytemask4(zq), pd, ex[k][q]);
            }
        }
        merge8(sm[k].x, sm[k].y, ex[k], out[k]);
    }
    uint16_t *yt = y + t0;
#pragma unroll
    for (int k = 0; k < kS15Groups; k++) {
        const uint32_t lo = (uint32_t)(k * (kS15Threads * 8) + tid * 8);
        if (lo + 8 <= rem) {
            st_stream(u32x4{out[k][0], out[k][1], out[k][2], out[k][3]}, reinterpret_cast<u32x4 *>(yt + lo));
        } else if (lo < rem) {
            for (uint32_t j = 0; j < 8 && lo + j < rem; j++)
                yt[lo + j] = (uint16_t)(out[k][j >> 1] >> (16 * (j & 1)));
        }
    }
}

// ============================================ Top-7 3-bit + zero-point ====
// "ZipCCL" exponent coding: codes 1..7 name the seven most frequent
// exponents (dec[0..6]); code 0 is a zero-point, whose exponent is the next
// stored one of its chunk. The codes sit in three bit planes. A tile (C <=
// tile: its chunks start inside it) loads M, its chunk offsets, 16
// sign-mantissa bytes and 16 bits of each plane per 16 words, and its run of
// stored exponents into LDS. A 256-entry LDS table spreads a plane byte (8
// words) over 8 bytes, one bit each; three lookups give 8 code bytes, and one
// byte permute of the 8-entry table [0, dec0..dec6] turns 4 codes into 4
// exponents. Zero-points (no bit set in any plane) are ranked like sentinels,
// with wave scans, and take their exponents from LDS before the merge.
constexpr int kZ7Threads = 128;
constexpr int kZ7Groups = 2;               // groups of 16 words per thread
constexpr int kZ7Tile = kZ7Threads * kZ7Groups * 16;

__global__ __launch_bounds__(kZ7Threads) void kz_decode_tile(StreamIn s, uint16_t *__restrict__ y, DecParams p)
{
    __shared__ uint32_t zv32[kZ7Tile / 4 + 1];     // the tile's stored exponents, from a 4-byte boundary
    __shared__ u32x2 spread[256];                   // byte j of spread[b] = bit j of b
    __shared__ uint32_t wtot[kZ7Groups][kZ7Threads / 64];
    __shared__ u32x4 xp[kZ7Threads / 64][128];      // one wave's 2 KiB of a group's output
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t t0 = (uint64_t)blockIdx.x * kZ7Tile;
    const uint32_t rem = (uint32_t)((p.n - t0 < (uint64_t)kZ7Tile) ? p.n - t0 : (uint64_t)kZ7Tile);
    // first loads: M, the tile's chunk offsets, the dense bytes
    const uint64_t M = *reinterpret_cast<const uint64_t *>(s.base + 24);
    const uint32_t *offs = reinterpret_cast<const uint32_t *>(s.base + p.off_offs) + (t0 >> p.logC);
    const uint32_t nc = (uint32_t)(((t0 + rem - 1) >> p.logC) - (t0 >> p.logC) + 1);
    const uint32_t o0 = offs[0], o1 = offs[nc];
    const uint8_t *smt = s.base + kHeader + t0;
    const uint8_t *plt = s.base + p.off_codes + t0 / 8;
    u32x4 sm[kZ7Groups];
    uint32_t pb[kZ7Groups][3];
#pragma unroll
    for (int k = 0; k < kZ7Groups; k++) {
        const uint32_t lo = (uint32_t)(k * (kZ7Threads * 16) + tid * 16);
        sm[k] = u32x4{0u, 0u, 0u, 0u};
        pb[k][0] = pb[k][1] = pb[k][2] = 0u;
        if (lo < rem) {
            sm[k] = ld_stream(reinterpret_cast<const u32x4 *>(smt + lo));
#pragma unroll
            for (int b = 0; b < 3; b++)
                pb[k][b] = ld_stream(reinterpret_cast<const uint16_t *>(plt + b * p.plane + lo / 8));
        }
    }
    for (int b = tid; b < 256; b += kZ7Threads) spread[b] = u32x2{spread4(b & 0xF), spread4(b >> 4)};
    // the tile's stored exponents: [E0, E1), clamped so that a corrupt stream
    // reads inside the buffer; whole dwords, then the last partial one
    const bool okM = M <= p.n && p.off_pos + M <= s.bytes;
    uint32_t E1 = okM ? (o1 < (uint32_t)M ? o1 : (uint32_t)M) : 0u;
    uint32_t E0 = o0 < E1 ? o0 : E1;
    if (E1 - E0 > rem) E1 = E0 + rem;
    const uint32_t a0 = E0 & ~3u;
    const uint8_t *val = s.base + p.off_pos;
    const uint32_t nfull = (E1 - a0) / 4;
    for (uint32_t w = tid; w < nfull; w += kZ7Threads) zv32[w] = *reinterpret_cast<const uint32_t *>(val + a0 + 4 * w);
    if (tid == kZ7Threads - 1 && ((E1 - a0) & 3u)) {
        uint32_t t = 0;
        for (uint32_t i = a0 + 4 * nfull; i < E1; i++) t |= (uint32_t)val[i] << (8 * (i - a0 - 4 * nfull));
        zv32[nfull] = t;
    }
    // zero-points: no bit in any plane, one flag per word
    uint32_t z[kZ7Groups], pre[kZ7Groups];
#pragma unroll
    for (int k = 0; k < kZ7Groups; k++) {
        const uint32_t lo = (uint32_t)(k * (kZ7Threads * 16) + tid * 16);
        uint32_t t = ~(pb[k][0] | pb[k][1] | pb[k][2]) & 0xFFFFu;
        if (lo + 16 > rem) t = lo < rem ? t & ((1u << (rem - lo)) - 1u) : 0u;
        z[k] = t;
        const uint32_t c = __builtin_popcount(t);
        uint32_t pr = 0, wt = 0;
        if (__ballot(c != 0) != 0ull) {
            const uint32_t inc = wave_inclusive_sum(c);
            pr = inc - c;
            wt = __builtin_amdgcn_readlane(inc, 63);
        }
        pre[k] = pr;
        if (lane == 0) wtot[k][wave] = wt;
    }
    __syncthreads();
    const uint32_t T0 = p.dec[0] << 8;                           // [0, dec0, dec1, dec2]
    const uint32_t T1 = (p.dec[0] >> 24) | (p.dec[1] << 8);      // [dec3 .. dec6]
    const uint8_t *zb = reinterpret_cast<const uint8_t *>(zv32);
    uint16_t *yt = y + t0;
    uint32_t run = 0;
#pragma unroll
    for (int k = 0; k < kZ7Groups; k++) {
        uint32_t base = run;
#pragma unroll
        for (int w = 0; w < kZ7Threads / 64; w++) {
            if (w < wave) base += wtot[k][w];
            run += wtot[k][w];
        }
        // exponents of words 4q..4q+3 in e[q]
        uint32_t e[4];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const u32x2 s0 = spread[(pb[k][0] >> (8 * h)) & 0xFFu];
            const u32x2 s1 = spread[(pb[k][1] >> (8 * h)) & 0xFFu];
            const u32x2 s2 = spread[(pb[k][2] >> (8 * h)) & 0xFFu];
            e[2 * h] = perm(T1, T0, s0.x | (s1.x << 1) | (s2.x << 2));
            e[2 * h + 1] = perm(T1, T0, s0.y | (s1.y << 1) | (s2.y << 2));
        }
        if (__ballot(z[k] != 0) != 0ull) {
            // word j's stored exponent (if it is a zero-point) is at rank
            // r + (zero-points before j); every word reads one, in bounds
            const uint32_t r = base + pre[k] + (E0 & 3u);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint32_t pd = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int j = 4 * q + i;
                    const uint32_t rj = r + __builtin_popcount(z[k] & ((1u << j) - 1u));
                    pd |= (uint32_t)zb[rj] << (8 * i);
                }
                const uint32_t mask = perm(0u, 0u, 0x0C0C0C0Cu + spread4((z[k] >> (4 * q)) & 0xFu));
                e[q] = bfi(mask, pd, e[q]);
            }
        }
        const uint32_t smq[4] = {sm[k].x, sm[k].y, sm[k].z, sm[k].w};
        uint32_t out[8];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            out[2 * q] = merge2(perm(e[q], smq[q], 0x05010400u));
            out[2 * q + 1] = merge2(perm(e[q], smq[q], 0x07030602u));
        }
        const uint32_t lo = (uint32_t)(k * (kZ7Threads * 16) + tid * 16);
        const uint32_t wlo = (uint32_t)(k * (kZ7Threads * 16) + wave * 1024);   // the wave's first word
        if (wlo + 1024 <= rem) {
            // through LDS, so that each store instruction covers 1 KiB
            // without gaps: lane l writes its 32 bytes at 32 l, then stores
            // the 16 bytes at 16 l and at 1024 + 16 l of the wave's span
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            xp[wave][2 * lane] = u32x4{out[0], out[1], out[2], out[3]};
            xp[wave][2 * lane + 1] = u32x4{out[4], out[5], out[6], out[7]};
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            u32x4 *dst = reinterpret_cast<u32x4 *>(yt + wlo);
            st_stream(xp[wave][lane], dst + lane);
            st_stream(xp[wave][64 + lane], dst + 64 + lane);
        } else if (lo + 16 <= rem) {
            st_stream(u32x4{out[0], out[1], out[2], out[3]}, reinterpret_cast<u32x4 *>(yt + lo));
            st_stream(u32x4{out[4], out[5], out[6], out[7]}, reinterpret_cast<u32x4 *>(yt + lo + 8));
        } else if (lo < rem) {
            for (uint32_t j = 0; j < 16 && lo + j < rem; j++)
                yt[lo + j] = (uint16_t)(out[j >> 1] >> (16 * (j & 1)));
        }
    }
}

// ================================================ Top-8 3-bit, positions ====
// "SplitZip" section 4.3 / Table 3: codes 0..7 name dec[0..7], packed 3
// bits per value; escapes as in the Top-16 stream. A 128-thread tile of
// 4,096 words; each lane takes 2 groups of 16 words (group k at tile word
// 2048 k + 16 lane): 16 sign-mantissa bytes and the group's 6 code bytes,
// from two aligned dwords and a byte shift. unpack12 spreads 4 codes over 4
// bytes, which select from the 8-entry table [dec0..dec7] in one byte
// permute. Escapes patch the exponent bytes through the LDS exponent tile
// (as in k_decode_tile), and each wave's output goes through LDS so that
// every store instruction covers 1 KiB.
constexpr int kT8Threads = 128;
constexpr int kT8Groups = 2;
constexpr int kT8Tile = kT8Threads * kT8Groups * 16;
static_assert(kT8Tile == kDecTile, "the patch takes the decode tile's shape");

__global__ __launch_bounds__(kT8Threads) void kt8_decode_tile(StreamIn s, uint16_t *__restrict__ y, DecParams p)
{
    __shared__ ExpTile<kT8Tile> sh;
    __shared__ u32x4 xp[kT8Threads / 64][128];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t t0 = (uint64_t)blockIdx.x * kT8Tile;
    const uint32_t rem = (uint32_t)((p.n - t0 < (uint64_t)kT8Tile) ? p.n - t0 : (uint64_t)kT8Tile);
    const PatchHead ph = patch_begin<kT8Tile, kT8Threads>(s, t0, p);
    const uint8_t *smt = s.base + kHeader + t0;
    const uint8_t *cdt = s.base + p.off_codes + t0 / 8 * 3;      // 4-byte aligned (t0 is a multiple of 32)
    u32x4 sm[kT8Groups];
    uint32_t c0[kT8Groups], c1[kT8Groups], csh[kT8Groups];
#pragma unroll
    for (int k = 0; k < kT8Groups; k++) {
        const uint32_t lo = (uint32_t)(k * (kT8Threads * 16) + tid * 16);
        sm[k] = u32x4{0u, 0u, 0u, 0u};
        c0[k] = c1[k] = 0u;
        const uint32_t b = lo / 8 * 3;                      // the group's first code byte: 6 per lane
        csh[k] = b & 3u;                                    // 0 or 2
        if (lo < rem) {
            // the sections are padded to 256 bytes and followed by more of
            // the stream, so the 16- and 8-byte loads stay inside it
            sm[k] = ld_stream(reinterpret_cast<const u32x4 *>(smt + lo));
            const uint32_t *cw = reinterpret_cast<const uint32_t *>(cdt + (b & ~3u));
            c0[k] = ld_stream(cw);
            c1[k] = ld_stream(cw + 1);
        }
    }
    const PatchFetch<kDecFetch> pf = patch_fetch<kT8Tile, kT8Threads, kDecFetch>(s, t0, p, ph);
    const uint32_t T0 = p.dec[0], T1 = p.dec[1];                  // dec[0..3], dec[4..7]
    uint32_t ex[kT8Groups][4];
#pragma unroll
    for (int k = 0; k < kT8Groups; k++) {
        // the 48 code bits of the group's 16 words: lo32 | hi16 << 32
        const uint32_t lo32 = __builtin_amdgcn_alignbyte(c1[k], c0[k], csh[k]);
        const uint32_t hi16 = (c1[k] >> (8 * csh[k])) & 0xFFFFu;
        ex[k][0] = perm(T1, T0, unpack12(lo32 & 0xFFFu));
        ex[k][1] = perm(T1, T0, unpack12((lo32 >> 12) & 0xFFFu));
        ex[k][2] = perm(T1, T0, unpack12(((lo32 >> 24) | (hi16 << 8)) & 0xFFFu));
        ex[k][3] = perm(T1, T0, unpack12((hi16 >> 4) & 0xFFFu));
    }
    if (pf.live) {
#pragma unroll
        for (int k = 0; k < kT8Groups; k++) {
            const uint32_t lo = (uint32_t)(k * (kT8Threads * 16) + tid * 16);
            if (lo < rem) *reinterpret_cast<u32x4 *>(&sh.ex[lo]) = u32x4{ex[k][0], ex[k][1], ex[k][2], ex[k][3]};
        }
        patch_put_offs(t0, p, ph, pf, sh);
        __syncthreads();
        patch_scatter<kT8Tile, kT8Threads, kDecFetch>(s, t0, p, ph, pf, sh);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kT8Groups; k++) {
            const uint32_t lo = (uint32_t)(k * (kT8Threads * 16) + tid * 16);
            if (lo < rem) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(&sh.ex[lo]);
                ex[k][0] = v.x; ex[k][1] = v.y; ex[k][2] = v.z; ex[k][3] = v.w;
            }
        }
    }
    uint16_t *yt = y + t0;
#pragma unroll
    for (int k = 0; k < kT8Groups; k++) {
        const uint32_t smq[4] = {sm[k].x, sm[k].y, sm[k].z, sm[k].w};
        uint32_t out[8];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            out[2 * q] = merge2(perm(ex[k][q], smq[q], 0x05010400u));
            out[2 * q + 1] = merge2(perm(ex[k][q], smq[q], 0x07030602u));
        }
        const uint32_t lo = (uint32_t)(k * (kT8Threads * 16) + tid * 16);
        const uint32_t wlo = (uint32_t)(k * (kT8Threads * 16) + wave * 1024);
        if (wlo + 1024 <= rem) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            xp[wave][2 * lane] = u32x4{out[0], out[1], out[2], out[3]};
            xp[wave][2 * lane + 1] = u32x4{out[4], out[5], out[6], out[7]};
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            u32x4 *dst = reinterpret_cast<u32x4 *>(yt + wlo);
            st_stream(xp[wave][lane], dst + lane);
            st_stream(xp[wave][64 + lane], dst + 64 + lane);
        } else if (lo + 16 <= rem) {
            st_stream(u32x4{out[0], out[1], out[2], out[3]}, reinterpret_cast<u32x4 *>(yt + lo));
            st_stream(u32x4{out[4], out[5], out[6], out[7]}, reinterpret_cast<u32x4 *>(yt + lo + 8));
        } else if (lo < rem) {
            for (uint32_t j = 0; j < 16 && lo + j < rem; j++)
                yt[lo + j] = (uint16_t)(out[j >> 1] >> (16 * (j & 1)));
        }
    }
}

// ================================================================ host ====
thread_local char g_hip_err[160];

int hip_fail(hipError_t e, const char *what)
{
    snprintf(g_hip_err, sizeof g_hip_err, "HIP error in %s: %s", what, hipGetErrorString(e));
    return UZIP_EHIP;
}

#define UZIP_LAUNCH_CHECK(what)                       \
    do {                                              \
        hipError_t e_ = hipGetLastError();            \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_nc(uint64_t n, uint32_t C)
{
    if (n == 0 || n >= (1ull << 32)) return false;
    if (C < 64 || C > 65536 || (C & (C - 1)) != 0) return false;
    return true;
}

// The codebook's three tables must agree with dec[].
int check_codebook(const uzip_codebook_t *cb)
{
    if (!cb || cb->version != UZIP_VERSION) return UZIP_EINVAL;
    uint8_t seen[256] = {0};
    for (int k = 0; k < 16; k++) {
        if (seen[cb->dec[k]]) return UZIP_EINVAL;
        seen[cb->dec[k]] = 1;
    }
    for (int e = 0; e < 256; e++) {
        if (cb->member[e] != seen[e]) return UZIP_EINVAL;
        if (!seen[e] && cb->enc[e] != 0) return UZIP_EINVAL;
    }
    for (int k = 0; k < 16; k++)
        if (cb->enc[cb->dec[k]] != k) return UZIP_EINVAL;
    return UZIP_OK;
}

// A codebook for FP8 E5M2 streams: consistent, and every exponent below 32.
int check_codebook8(const uzip_codebook_t *cb)
{
    const int rc = check_codebook(cb);
    if (rc) return rc;
    for (int k = 0; k < 16; k++)
        if (cb->dec[k] > 31) return UZIP_EINVAL;
    return UZIP_OK;
}

EncParams make_enc_params(const Layout &L, const uzip_codebook_t *cb)
{
    EncParams p;
    for (int e = 0; e < 256; e++) p.lut[e] = 0x80;
    for (int k = 0; k < 16; k++) p.lut[cb->dec[k]] = (uint8_t)k;
    p.n = L.n;
    p.nch = L.nch;
    p.ntiles = (L.n + kEncTile - 1) / kEncTile;
    p.gshift = group_shift(p.ntiles);
    p.ngroups = (p.ntiles + (1ull << p.gshift) - 1) >> p.gshift;
    p.Cmask = L.C - 1;
    p.logC = L.logC;
    p.off_codes = L.off_codes;
    p.off_offs = L.off_offs;
    p.off_pos = L.off_pos;
    p.dlut = nullptr;
    p.ddec = nullptr;
    p.sm_bytes = sm_bytes_of(L.n, L.fmt == kFmtFP8);
    p.code_bytes = L.code_bytes;
    p.plane = L.plane;
    p.nplanes = L.nplanes;
    p.posw = has_pos(L.fmt) ? 2 : 0;
    return p;
}

DecParams make_dec_params(const Layout &L, const uzip_codebook_t *cb)
{
    DecParams p;
    memcpy(p.dec, cb->dec, 16);
    p.n = L.n;
    p.nch = L.nch;
    p.C = L.C;
    p.logC = L.logC;
    p.off_codes = L.off_codes;
    p.off_offs = L.off_offs;
    p.off_pos = L.off_pos;
    p.plane = L.plane;
    return p;
}

HeaderParams make_header_params(const Layout &L, const uzip_codebook_t *cb)
{
    HeaderParams h;
    memset(h.tmpl, 0, sizeof h.tmpl);
    h.tmpl[0] = 0x55; h.tmpl[1] = 0x5A; h.tmpl[2] = 0x42; h.tmpl[3] = 0x31;
    const uint16_t ver = 1;
    memcpy(h.tmpl + 4, &ver, 2);
    h.tmpl[6] = L.fmt;                        // format: 0 BF16, 1 FP8 E5M2, 2 Top-15 + sentinel, 3 Top-7 + zero-point
    memcpy(h.tmpl + 8, &L.C, 4);
    memcpy(h.tmpl + 16, &L.n, 8);
    memcpy(h.tmpl + 40, cb->dec, 16);
    return h;
}

EncWs make_ws(void *d_ws, uint64_t n, uint32_t C)
{
    const WsLayout w = ws_layout(n, C);
    uint8_t *b = static_cast<uint8_t *>(d_ws);
    EncWs ws;
    ws.hist = reinterpret_cast<unsigned long long *>(b + w.hist);
    ws.lut = b + w.lut;
    ws.dec = b + w.dec;
    ws.counts = reinterpret_cast<uint32_t *>(b + w.counts);
    ws.gsum = reinterpret_cast<uint32_t *>(b + w.gsum);
    ws.tpre = reinterpret_cast<uint32_t *>(b + w.tpre);
    ws.chunk_pre = reinterpret_cast<uint32_t *>(b + w.chunk_pre);
    ws.stage_aux = b + w.stage_aux;
    ws.stage_val = b + w.stage_val;
    return ws;
}

struct Events {
    const uzip_opts_t *o;
    hipStream_t s;
    int record(uint32_t i) const
    {
        if (!o || !o->events || i >= o->n_events) return UZIP_OK;
        hipError_t e = hipEventRecord(o->events[i], s);
        return e == hipSuccess ? UZIP_OK : hip_fail(e, "hipEventRecord");
    }
};

// Scan + placement shared by encode and reduce (kernels 2 and 3 of the call).
int finish_encode(const Layout &L, const uzip_codebook_t *cb, const EncParams &ep, const EncWs &ws,
                  uint8_t *out, const Events &ev, hipStream_t s, uint32_t ev0 = 2)
{
    const HeaderParams hp = make_header_params(L, cb);
    k_group_sums<<<(unsigned)ep.ngroups, kThreads, 0, s>>>(ws, ep);
    UZIP_LAUNCH_CHECK("k_group_sums");
    int rc = ev.record(ev0);
    if (rc) return rc;
    k_place_escapes<<<(unsigned)((ep.ntiles + kPlaceThreads / 64 - 1) / (kPlaceThreads / 64)), kPlaceThreads, 0, s>>>(
        ws, out, ep, hp);
    UZIP_LAUNCH_CHECK("k_place_escapes");
    return ev.record(ev0 + 1);
}

// Histogram launch: kHistUnroll 16-byte groups per thread and round, at
// most 2048 workgroups.
// eb: element bytes (2 BF16, 1 FP8 E5M2); block and sample are multiples of
// 16 / eb values.
void launch_hist(const void *d_x, uint64_t n, uint64_t block, uint64_t sample, uint64_t *d_hist,
                 hipStream_t s, int eb = 2)
{
    const uint64_t vg = 16 / eb;
    // a block longer than x is x: keeps the kernel's group numbers in 32 bits
    const uint64_t nr = (n + vg - 1) / vg * vg;
    if (block > nr) block = nr;
    if (sample > block) sample = block;
    const uint64_t groups = ((n + block - 1) / block) * (sample / vg);
    const uint64_t wgs = (groups + kThreads * kHistUnroll - 1) / (kThreads * kHistUnroll);
    const unsigned grid = (unsigned)(wgs < 2048 ? (wgs ? wgs : 1) : 2048);
    const uint8_t *x = static_cast<const uint8_t *>(d_x);
    unsigned long long *h = reinterpret_cast<unsigned long long *>(d_hist);
    if (eb == 2) k_hist<2><<<grid, kThreads, 0, s>>>(x, n, block, sample, h);
    else k_hist<1><<<grid, kThreads, 0, s>>>(x, n, block, sample, h);
}

// Workspace of uzip_encode_noalloc: one fixed array per GPU, in the code
// object's device memory, that every call on that GPU shares. In host code
// `scratch` names a host-side stand-in, not device memory: kernels get the
// device address that hipGetSymbolAddress returns for the current device
// (each device holds its own copy at its own address), looked up once per
// device and cached.
constexpr uint64_t kScratchBytes = UZIP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return UZIP_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned16(p)) return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return UZIP_OK;
}

// Host-side structural check (same rules as the header comment of
// uzip_validate_host).
uint16_t rd16(const uint8_t *p) { uint16_t v; memcpy(&v, p, 2); return v; }
uint32_t rd32(const uint8_t *p) { uint32_t v; memcpy(&v, p, 4); return v; }
uint64_t rd64(const uint8_t *p) { uint64_t v; memcpy(&v, p, 8); return v; }

}  // namespace

// ============================================================== C-ABI =====
extern "C" {

uint64_t uzip_max_bytes(uint64_t n, uint32_t chunk)
{
    if (!valid_nc(n, chunk)) return 0;
    return total_of(make_layout(n, chunk), n);
}

uint64_t uzip_workspace_bytes(uint64_t n, uint32_t chunk)
{
    if (!valid_nc(n, chunk)) return 0;
    return ws_layout(n, chunk).total;
}

int uzip_codebook_from_dec(const uint8_t dec[16], uzip_codebook_t *cb)
{
    if (!dec || !cb) return UZIP_EINVAL;
    uzip_codebook_t c;
    memset(&c, 0, sizeof c);
    c.version = UZIP_VERSION;
    for (int k = 0; k < 16; k++) {
        if (c.member[dec[k]]) return UZIP_EINVAL;          // entries must be distinct
        c.dec[k] = dec[k];
        c.member[dec[k]] = 1;
        c.enc[dec[k]] = (uint8_t)k;
    }
    *cb = c;
    return UZIP_OK;
}

int uzip_codebook_from_hist(const uint64_t hist[256], uzip_codebook_t *cb)
{
    if (!hist || !cb) return UZIP_EINVAL;
    // rank all 256 exponents: count descending, exponent ascending (stable
    // insertion sort over an index array already in ascending order)
    int order[256];
    for (int e = 0; e < 256; e++) order[e] = e;
    for (int i = 1; i < 256; i++) {
        int v = order[i], j = i - 1;
        while (j >= 0 && hist[order[j]] < hist[v]) {
            order[j + 1] = order[j];
            j--;
        }
        order[j + 1] = v;
    }
    memset(cb, 0, sizeof *cb);
    cb->version = UZIP_VERSION;
    uint64_t total = 0;
    for (int e = 0; e < 256; e++) {
        cb->hist[e] = hist[e];
        total += hist[e];
    }
    cb->n_cal = total;
    for (int k = 0; k < 16; k++) {
        const int e = order[k];
        cb->dec[k] = (uint8_t)e;
        cb->enc[e] = (uint8_t)k;
        cb->member[e] = 1;
    }
    return UZIP_OK;
}

int uzip_parse_header(const void *h_header, uint64_t *n, uint32_t *chunk, uint64_t *m,
                      uint64_t *total_bytes, uint8_t dec[16])
{
    if (!h_header) return UZIP_EINVAL;
    const uint8_t *h = static_cast<const uint8_t *>(h_header);
    if (!(h[0] == 0x55 && h[1] == 0x5A && h[2] == 0x42 && h[3] == 0x31)) return UZIP_ECORRUPT;
    if (rd16(h + 4) != 1) return UZIP_ECORRUPT;
    if (n) *n = rd64(h + 16);
    if (chunk) *chunk = rd32(h + 8);
    if (m) *m = rd64(h + 24);
    if (total_bytes) *total_bytes = rd64(h + 32);
    if (dec) memcpy(dec, h + 40, 16);
    return UZIP_OK;
}

int uzip_validate_host(const void *h_stream, uint64_t bytes, const uzip_codebook_t *cb)
{
    if (!h_stream || !cb) return UZIP_EINVAL;
    const uint8_t *s = static_cast<const uint8_t *>(h_stream);
    if (bytes < kHeader) return UZIP_ECORRUPT;
    uint64_t n, m, total;
    uint32_t C;
    uint8_t dec[16];
    if (uzip_parse_header(s, &n, &C, &m, &total, dec) != UZIP_OK) return UZIP_ECORRUPT;
    const uint16_t fmt = rd16(s + 6);       // 0 BF16, 1 FP8 E5M2, 2 Top-15 + sentinel, 3 Top-7 + zero-point, 4 Top-8
    if (fmt > 4 || rd32(s + 12) != 0) return UZIP_ECORRUPT;
    const bool fp8 = fmt == kFmtFP8, s15 = fmt == kFmtS15, z7 = fmt == kFmtZ7, t8 = fmt == kFmtT8;
    for (uint64_t i = 56; i < kHeader; i++)
        if (s[i]) return UZIP_ECORRUPT;
    if (!valid_nc(n, C) || m > n) return UZIP_ECORRUPT;
    if (s15 && C > (uint32_t)kS15Tile) return UZIP_ECORRUPT;
    if (z7 && C > (uint32_t)kZ7Tile) return UZIP_ECORRUPT;
    const Layout L = make_layout(n, C, (uint8_t)fmt);
    const uint64_t off_val = off_val_of(L, m);
    if (total != off_val + m || bytes < total) return UZIP_ECORRUPT;
    if (memcmp(dec, cb->dec, 16) != 0) return UZIP_ECODEBOOK;
    bool in_book[256] = {false}, seen[256] = {false};
    for (int k = 0; k < 16; k++) {
        if (seen[dec[k]] || (fp8 && dec[k] > 31)) return UZIP_ECORRUPT;
        seen[dec[k]] = true;
        in_book[dec[k]] = z7 ? k < 7 : t8 ? k < 8 : (!s15 || k < 15);   // Top-15: dec[0..14], Top-7: dec[0..6], Top-8: dec[0..7]
    }
    auto zero = [&](uint64_t a, uint64_t b) {
        for (uint64_t i = a; i < b; i++)
            if (s[i]) return false;
        return true;
    };
    const uint64_t smb = sm_bytes_of(n, fp8);
    if (!zero(kHeader + smb, L.off_codes)) return UZIP_ECORRUPT;
    if (fp8 && (3 * n) % 8 && (s[kHeader + smb - 1] >> ((3 * n) % 8))) return UZIP_ECORRUPT;   // unused bits
    if (!z7 && !t8 && (n & 1) && (s[L.off_codes + n / 2] >> 4)) return UZIP_ECORRUPT;
    if (t8 && (3 * n) % 8 && (s[L.off_codes + (3 * n) / 8] >> ((3 * n) % 8))) return UZIP_ECORRUPT;   // bits past 3n
    for (uint32_t b = 0; b < L.nplanes; b++) {
        const uint64_t pl = L.off_codes + b * L.plane;
        if (z7 && (n & 7) && (s[pl + n / 8] >> (n & 7))) return UZIP_ECORRUPT;     // plane bits past n
        if (!zero(pl + L.code_bytes, pl + L.plane)) return UZIP_ECORRUPT;
    }
    if (!zero(L.off_offs + 4 * (L.nch + 1), L.off_pos)) return UZIP_ECORRUPT;
    if (has_pos(L.fmt) && !zero(L.off_pos + 2 * m, off_val)) return UZIP_ECORRUPT;
    const uint8_t *offs = s + L.off_offs;
    if (rd32(offs) != 0 || rd32(offs + 4 * L.nch) != m) return UZIP_ECORRUPT;
    if (z7) {
        // each chunk: as many stored exponents as zero-points (code 0), all outside dec[0..6]
        for (uint64_t c = 0; c < L.nch; c++) {
            const uint64_t j0 = rd32(offs + 4 * c), j1 = rd32(offs + 4 * (c + 1));
            const uint64_t lo = c * C, hi = (lo + C < n) ? lo + C : n;
            uint64_t zeros = 0;
            for (uint64_t i = lo; i < hi; i++) {
                uint32_t code = 0;
                for (uint32_t b = 0; b < 3; b++) code |= ((s[L.off_codes + b * L.plane + i / 8] >> (i & 7)) & 1u) << b;
                zeros += code == 0;
            }
            if (j1 < j0 || j1 > m || j1 - j0 != zeros) return UZIP_ECORRUPT;
            for (uint64_t j = j0; j < j1; j++)
                if (in_book[s[off_val + j]]) return UZIP_ECORRUPT;
        }
        return UZIP_OK;
    }
    if (s15) {
        // each chunk: as many stored exponents as sentinels (code 15), all outside dec[0..14]
        for (uint64_t c = 0; c < L.nch; c++) {
            const uint64_t j0 = rd32(offs + 4 * c), j1 = rd32(offs + 4 * (c + 1));
            const uint64_t lo = c * C, hi = (lo + C < n) ? lo + C : n;
            uint64_t sentinels = 0;
            for (uint64_t i = lo; i < hi; i++) {
                const uint8_t b = s[L.off_codes + i / 2];
                sentinels += (((i & 1) ? (b >> 4) : (b & 0xF)) == 15);
            }
            if (j1 < j0 || j1 > m || j1 - j0 != sentinels) return UZIP_ECORRUPT;
            for (uint64_t j = j0; j < j1; j++)
                if (in_book[s[off_val + j]]) return UZIP_ECORRUPT;
        }
        return UZIP_OK;
    }
    for (uint64_t c = 0; c < L.nch; c++) {
        const uint64_t j0 = rd32(offs + 4 * c), j1 = rd32(offs + 4 * (c + 1));
        const uint64_t len = (c + 1) * C <= n ? C : n - c * C;
        if (j1 < j0 || j1 > m || j1 - j0 > len) return UZIP_ECORRUPT;
        uint32_t prev = 0;
        for (uint64_t j = j0; j < j1; j++) {
            const uint32_t p = rd16(s + L.off_pos + 2 * j);
            if (p >= len || (j > j0 && p <= prev)) return UZIP_ECORRUPT;
            prev = p;
            if (in_book[s[off_val + j]] || (fp8 && s[off_val + j] > 31)) return UZIP_ECORRUPT;
            const uint64_t i = c * C + p;
            if (t8) {
                uint32_t code = 0;
                for (uint32_t k = 0; k < 3; k++)
                    code |= ((s[L.off_codes + (3 * i + k) / 8] >> ((3 * i + k) % 8)) & 1u) << k;
                if (code != 0) return UZIP_ECORRUPT;
                continue;
            }
            const uint8_t b = s[L.off_codes + i / 2];
            if (((i & 1) ? (b >> 4) : (b & 0xF)) != 0) return UZIP_ECORRUPT;
        }
    }
    return UZIP_OK;
}

const char *uzip_strerror(int code)
{
    switch (code) {
    case UZIP_OK: return "ok";
    case UZIP_EINVAL: return "invalid argument (null or misaligned pointer, bad n, chunk or codebook)";
    case UZIP_ENOSPC: return "output capacity or workspace too small";
    case UZIP_ECORRUPT: return "stream is malformed";
    case UZIP_ECODEBOOK: return "stream was encoded with a different codebook";
    case UZIP_EHIP: return g_hip_err[0] ? g_hip_err : "HIP runtime error";
    case UZIP_ESCRATCH: return "input too large for uzip_encode_noalloc: its workspace exceeds the fixed "
                               "UZIP_NOALLOC_SCRATCH_BYTES scratch (use uzip_encode with a workspace)";
    default: return "unknown error";
    }
}

int uzip_histogram_sampled(const uint16_t *d_x, uint64_t n, uint64_t block, uint64_t sample, uint64_t *d_hist,
                           hipStream_t s)
{
    if (!d_x || !d_hist || !aligned16(d_x) || ((uintptr_t)d_hist & 7u)) return UZIP_EINVAL;
    if (n == 0 || n >= (1ull << 32)) return UZIP_EINVAL;
    if (block == 0) block = sample = (n + 7) & ~7ull;      // the whole of x
    if (sample == 0 || sample > block || (block & 7) || (sample & 7)) return UZIP_EINVAL;
    launch_hist(d_x, n, block, sample, d_hist, s);
    UZIP_LAUNCH_CHECK("k_hist");
    return UZIP_OK;
}

int uzip_histogram(const uint16_t *d_x, uint64_t n, uint64_t *d_hist, hipStream_t s)
{
    return uzip_histogram_sampled(d_x, n, 0, 0, d_hist, s);
}

int uzip_calibrate(const uint16_t *d_x, uint64_t n, uint64_t *d_hist_ws, uzip_codebook_t *cb, hipStream_t s)
{
    if (!cb || !d_hist_ws) return UZIP_EINVAL;
    hipError_t e = hipMemsetAsync(d_hist_ws, 0, 256 * sizeof(uint64_t), s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
    int rc = uzip_histogram(d_x, n, d_hist_ws, s);
    if (rc) return rc;
    uint64_t h[256];
    e = hipMemcpyAsync(h, d_hist_ws, sizeof h, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return uzip_codebook_from_hist(h, cb);
}

int uzip_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                   const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_x || !d_out || !d_ws || !aligned16(d_x) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    if (out_cap < uzip_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk);
    const EncParams ep = make_enc_params(L, cb);
    const EncWs ws = make_ws(d_ws, n, chunk);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    k_encode_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(d_x, static_cast<uint8_t *>(d_out), ws, ep);
    UZIP_LAUNCH_CHECK("k_encode_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_encode_online_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, uint64_t block, uint64_t sample,
                          uzip_codebook_t *d_cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                          const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_x || !d_out || !d_ws || !aligned16(d_x) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (d_cb && ((uintptr_t)d_cb & 7u)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    if (block == 0) block = sample = (n + 7) & ~7ull;
    if (sample == 0 || sample > block || (block & 7) || (sample & 7)) return UZIP_EINVAL;
    if (out_cap < uzip_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk);
    uzip_codebook_t none;                  // the tables come from the device
    memset(&none, 0, sizeof none);
    EncParams ep = make_enc_params(L, &none);
    const EncWs ws = make_ws(d_ws, n, chunk);
    ep.dlut = ws.lut;
    ep.ddec = ws.dec;
    const Events ev{opts, s};
    int rc;
    if ((rc = ev.record(0))) return rc;
    k_zero_hist<<<1, 256, 0, s>>>(ws.hist);
    UZIP_LAUNCH_CHECK("k_zero_hist");
    launch_hist(d_x, n, block, sample, reinterpret_cast<uint64_t *>(ws.hist), s);
    UZIP_LAUNCH_CHECK("k_hist");
    k_top16<<<1, 256, 0, s>>>(ws.hist, ws.lut, ws.dec, d_cb);
    UZIP_LAUNCH_CHECK("k_top16");
    if ((rc = ev.record(1))) return rc;
    k_encode_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(d_x, static_cast<uint8_t *>(d_out), ws, ep);
    UZIP_LAUNCH_CHECK("k_encode_tile");
    if ((rc = ev.record(2))) return rc;
    return finish_encode(L, &none, ep, ws, static_cast<uint8_t *>(d_out), ev, s, 3);
}

int uzip_encode_online(const uint16_t *d_x, uint64_t n, uint32_t chunk, uint64_t block, uint64_t sample,
                       uzip_codebook_t *d_cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       hipStream_t s)
{
    return uzip_encode_online_ex(d_x, n, chunk, block, sample, d_cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

uint64_t uzip_s15_max_bytes(uint64_t n, uint32_t chunk)
{
    if (!valid_nc(n, chunk) || chunk > (uint32_t)kS15Tile) return 0;
    return total_of(make_layout(n, chunk, kFmtS15), n);
}

int uzip_s15_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_x || !d_out || !d_ws || !aligned16(d_x) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk) || chunk > (uint32_t)kS15Tile) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    if (out_cap < uzip_s15_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk, kFmtS15);
    EncParams ep = make_enc_params(L, cb);
    ep.lut[cb->dec[15]] = 0x80;                 // the 16th exponent is an escape here
    for (int e = 0; e < 256; e++)
        if (ep.lut[e] & 0x80) ep.lut[e] = 0x80 | 15;   // escapes take the sentinel code
    const EncWs ws = make_ws(d_ws, n, chunk);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    k_encode_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(d_x, static_cast<uint8_t *>(d_out), ws, ep);
    UZIP_LAUNCH_CHECK("k_encode_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_s15_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s)
{
    return uzip_s15_encode_ex(d_x, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

int uzip_s15_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_in || !d_y || !aligned16(d_in) || !aligned16(d_y)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk) || chunk > (uint32_t)kS15Tile) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    const Layout L = make_layout(n, chunk, kFmtS15);
    if (in_bytes < total_of(L, 0)) return UZIP_EINVAL;
    const DecParams dp = make_dec_params(L, cb);
    const StreamIn si{static_cast<const uint8_t *>(d_in), in_bytes};
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    const uint64_t tiles = (n + kS15Tile - 1) / kS15Tile;
    k_s15_decode_tile<<<(unsigned)tiles, kS15Threads, 0, s>>>(si, d_y, dp);
    UZIP_LAUNCH_CHECK("k_s15_decode_tile");
    return ev.record(1);
}

int uzip_s15_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    uint16_t *d_y, hipStream_t s)
{
    return uzip_s15_decode_ex(d_in, in_bytes, n, chunk, cb, d_y, nullptr, s);
}

uint64_t uzip_t8_max_bytes(uint64_t n, uint32_t chunk)
{
    if (!valid_nc(n, chunk)) return 0;
    return total_of(make_layout(n, chunk, kFmtT8), n);
}

int uzip_t8_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                      void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                      const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_x || !d_out || !d_ws || !aligned16(d_x) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    if (out_cap < uzip_t8_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk, kFmtT8);
    EncParams ep = make_enc_params(L, cb);
    for (int e = 0; e < 256; e++) ep.lut[e] = 0x80;       // escape: dummy code 0
    for (int k = 0; k < 8; k++) ep.lut[cb->dec[k]] = (uint8_t)k;
    const EncWs ws = make_ws(d_ws, n, chunk);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    kt8_encode_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(d_x, static_cast<uint8_t *>(d_out), ws, ep);
    UZIP_LAUNCH_CHECK("kt8_encode_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_t8_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s)
{
    return uzip_t8_encode_ex(d_x, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

int uzip_t8_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                      uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_in || !d_y || !aligned16(d_in) || !aligned16(d_y)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    const Layout L = make_layout(n, chunk, kFmtT8);
    if (in_bytes < total_of(L, 0)) return UZIP_EINVAL;
    const DecParams dp = make_dec_params(L, cb);
    const StreamIn si{static_cast<const uint8_t *>(d_in), in_bytes};
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    const uint64_t tiles = (n + kT8Tile - 1) / kT8Tile;
    kt8_decode_tile<<<(unsigned)tiles, kT8Threads, 0, s>>>(si, d_y, dp);
    UZIP_LAUNCH_CHECK("kt8_decode_tile");
    return ev.record(1);
}

int uzip_t8_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   uint16_t *d_y, hipStream_t s)
{
    return uzip_t8_decode_ex(d_in, in_bytes, n, chunk, cb, d_y, nullptr, s);
}

uint64_t uzip_z7_max_bytes(uint64_t n, uint32_t chunk)
{
    if (!valid_nc(n, chunk) || chunk > (uint32_t)kZ7Tile) return 0;
    return total_of(make_layout(n, chunk, kFmtZ7), n);
}

int uzip_z7_encode_ex(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                      void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                      const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_x || !d_out || !d_ws || !aligned16(d_x) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk) || chunk > (uint32_t)kZ7Tile) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    if (out_cap < uzip_z7_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk, kFmtZ7);
    EncParams ep = make_enc_params(L, cb);
    for (int e = 0; e < 256; e++) ep.lut[e] = 0x80;       // zero-point: code 0, escape flag
    for (int k = 0; k < 7; k++) ep.lut[cb->dec[k]] = (uint8_t)(k + 1);
    const EncWs ws = make_ws(d_ws, n, chunk);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    kz_encode_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(d_x, static_cast<uint8_t *>(d_out), ws, ep);
    UZIP_LAUNCH_CHECK("kz_encode_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_z7_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s)
{
    return uzip_z7_encode_ex(d_x, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

int uzip_z7_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                      uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_in || !d_y || !aligned16(d_in) || !aligned16(d_y)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk) || chunk > (uint32_t)kZ7Tile) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    const Layout L = make_layout(n, chunk, kFmtZ7);
    if (in_bytes < total_of(L, 0)) return UZIP_EINVAL;
    const DecParams dp = make_dec_params(L, cb);
    const StreamIn si{static_cast<const uint8_t *>(d_in), in_bytes};
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    const uint64_t tiles = (n + kZ7Tile - 1) / kZ7Tile;
    kz_decode_tile<<<(unsigned)tiles, kZ7Threads, 0, s>>>(si, d_y, dp);
    UZIP_LAUNCH_CHECK("kz_decode_tile");
    return ev.record(1);
}

int uzip_z7_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                   uint16_t *d_y, hipStream_t s)
{
    return uzip_z7_decode_ex(d_in, in_bytes, n, chunk, cb, d_y, nullptr, s);
}

uint64_t uzip_fp8_max_bytes(uint64_t n, uint32_t chunk)
{
    if (!valid_nc(n, chunk)) return 0;
    return total_of(make_layout(n, chunk, kFmtFP8), n);
}

int uzip_fp8_histogram(const uint8_t *d_x, uint64_t n, uint64_t *d_hist, hipStream_t s)
{
    if (!d_x || !d_hist || !aligned16(d_x) || ((uintptr_t)d_hist & 7u)) return UZIP_EINVAL;
    if (n == 0 || n >= (1ull << 32)) return UZIP_EINVAL;
    const uint64_t all = (n + 15) & ~15ull;
    launch_hist(d_x, n, all, all, d_hist, s, 1);
    UZIP_LAUNCH_CHECK("k_hist");
    return UZIP_OK;
}

int uzip_fp8_calibrate(const uint8_t *d_x, uint64_t n, uint64_t *d_hist_ws, uzip_codebook_t *cb, hipStream_t s)
{
    if (!cb || !d_hist_ws) return UZIP_EINVAL;
    hipError_t e = hipMemsetAsync(d_hist_ws, 0, 256 * sizeof(uint64_t), s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
    int rc = uzip_fp8_histogram(d_x, n, d_hist_ws, s);
    if (rc) return rc;
    uint64_t h[256];
    e = hipMemcpyAsync(h, d_hist_ws, sizeof h, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return uzip_codebook_from_hist(h, cb);
}

int uzip_fp8_encode_ex(const uint8_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_x || !d_out || !d_ws || !aligned16(d_x) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook8(cb);
    if (rc) return rc;
    if (out_cap < uzip_fp8_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk, kFmtFP8);
    const EncParams ep = make_enc_params(L, cb);
    const EncWs ws = make_ws(d_ws, n, chunk);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    k8_encode_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(d_x, static_cast<uint8_t *>(d_out), ws, ep);
    UZIP_LAUNCH_CHECK("k8_encode_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_fp8_encode(const uint8_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s)
{
    return uzip_fp8_encode_ex(d_x, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

int uzip_fp8_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       uint8_t *d_y, const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_in || !d_y || !aligned16(d_in) || !aligned16(d_y)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook8(cb);
    if (rc) return rc;
    const Layout L = make_layout(n, chunk, kFmtFP8);
    if (in_bytes < total_of(L, 0)) return UZIP_EINVAL;   // smaller than any stream of n values
    const DecParams dp = make_dec_params(L, cb);
    const StreamIn si{static_cast<const uint8_t *>(d_in), in_bytes};
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    const uint64_t tiles = (n + k8DecTile - 1) / k8DecTile;
    k8_decode_tile<true><<<(unsigned)tiles, k8DecThreads, 0, s>>>(si, d_y, dp);
    UZIP_LAUNCH_CHECK("k8_decode_tile");
    return ev.record(1);
}

int uzip_fp8_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    uint8_t *d_y, hipStream_t s)
{
    return uzip_fp8_decode_ex(d_in, in_bytes, n, chunk, cb, d_y, nullptr, s);
}

int uzip_encode(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s)
{
    return uzip_encode_ex(d_x, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

int uzip_encode_noalloc(const uint16_t *d_x, uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                        void *d_out, uint64_t out_cap, hipStream_t s)
{
    // the size check comes before any HIP call, so an input that is too
    // large is rejected without touching the device
    if (valid_nc(n, chunk) && uzip_workspace_bytes(n, chunk) > kScratchBytes) return UZIP_ESCRATCH;
    void *ws = nullptr;
    const int rc = scratch_for_current_device(&ws);
    if (rc) return rc;
    return uzip_encode_ex(d_x, n, chunk, cb, d_out, out_cap, ws, kScratchBytes, nullptr, s);
}

int uzip_stream_bytes(const void *d_stream, uint64_t *total_bytes, uint64_t *m, hipStream_t s)
{
    if (!d_stream) return UZIP_EINVAL;
    uint8_t h[kHeader];
    hipError_t e = hipMemcpyAsync(h, d_stream, kHeader, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    return uzip_parse_header(h, nullptr, nullptr, m, total_bytes, nullptr);
}

int uzip_decode_ex(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                   const uzip_codebook_t *cb, uint16_t *d_y, const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_in || !d_y || !aligned16(d_in) || !aligned16(d_y)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    const Layout L = make_layout(n, chunk);
    if (in_bytes < total_of(L, 0)) return UZIP_EINVAL;   // smaller than any stream of n values
    const DecParams dp = make_dec_params(L, cb);
    const StreamIn si{static_cast<const uint8_t *>(d_in), in_bytes};
    const unsigned grid = (unsigned)((n + kDecTile - 1) / kDecTile);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    if (opts && (opts->flags & UZIP_F_SEPARATE_PATCH)) {
        k_decode_tile<false><<<grid, kDecThreads, 0, s>>>(si, d_y, dp);
        UZIP_LAUNCH_CHECK("k_decode_tile<dense>");
        if ((rc = ev.record(1))) return rc;
        uint64_t wgs = (L.nch + (kThreads / 64) - 1) / (kThreads / 64);
        k_patch<<<(unsigned)(wgs < 8192 ? wgs : 8192), kThreads, 0, s>>>(si, d_y, dp);
        UZIP_LAUNCH_CHECK("k_patch");
        return ev.record(2);
    }
    k_decode_tile<true><<<grid, kDecThreads, 0, s>>>(si, d_y, dp);
    UZIP_LAUNCH_CHECK("k_decode_tile");
    return ev.record(1);
}

int uzip_decode(const void *d_in, uint64_t in_bytes, uint64_t n, uint32_t chunk,
                const uzip_codebook_t *cb, uint16_t *d_y, hipStream_t s)
{
    return uzip_decode_ex(d_in, in_bytes, n, chunk, cb, d_y, nullptr, s);
}

int uzip_reduce_add_ex(const void *d_a, uint64_t a_bytes, const void *d_b, uint64_t b_bytes,
                       uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                       void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                       const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_a || !d_b || !d_out || !d_ws) return UZIP_EINVAL;
    if (!aligned16(d_a) || !aligned16(d_b) || !aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    if (out_cap < uzip_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk);
    if (a_bytes < total_of(L, 0) || b_bytes < total_of(L, 0)) return UZIP_EINVAL;
    const EncParams ep = make_enc_params(L, cb);
    const DecParams dp = make_dec_params(L, cb);
    const EncWs ws = make_ws(d_ws, n, chunk);
    const StreamIn sa{static_cast<const uint8_t *>(d_a), a_bytes};
    const StreamIn sb{static_cast<const uint8_t *>(d_b), b_bytes};
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    k_reduce_tile<<<(unsigned)ep.ntiles, kEncThreads, 0, s>>>(sa, sb, static_cast<uint8_t *>(d_out), ws, ep, dp);
    UZIP_LAUNCH_CHECK("k_reduce_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_reduce_add(const void *d_a, uint64_t a_bytes, const void *d_b, uint64_t b_bytes,
                    uint64_t n, uint32_t chunk, const uzip_codebook_t *cb,
                    void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes, hipStream_t s)
{
    return uzip_reduce_add_ex(d_a, a_bytes, d_b, b_bytes, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes,
                              nullptr, s);
}

int uzip_reduce_k_ex(const void *const *d_in, const uint64_t *in_bytes, uint32_t k, uint64_t n, uint32_t chunk,
                     const uzip_codebook_t *cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                     const uzip_opts_t *opts, hipStream_t s)
{
    if (!d_in || !in_bytes || !d_out || !d_ws || k == 0 || k > UZIP_MAX_K) return UZIP_EINVAL;
    if (!aligned16(d_out) || !aligned16(d_ws)) return UZIP_EINVAL;
    if (!valid_nc(n, chunk)) return UZIP_EINVAL;
    int rc = check_codebook(cb);
    if (rc) return rc;
    if (out_cap < uzip_max_bytes(n, chunk) || ws_bytes < uzip_workspace_bytes(n, chunk)) return UZIP_ENOSPC;
    const Layout L = make_layout(n, chunk);
    StreamSet ss{};
    ss.k = k;
    for (uint32_t i = 0; i < k; i++) {
        if (!d_in[i] || !aligned16(d_in[i]) || in_bytes[i] < total_of(L, 0)) return UZIP_EINVAL;
        ss.in[i] = StreamIn{static_cast<const uint8_t *>(d_in[i]), in_bytes[i]};
    }
    const EncParams ep = make_enc_params(L, cb);
    const DecParams dp = make_dec_params(L, cb);
    const EncWs ws = make_ws(d_ws, n, chunk);
    const Events ev{opts, s};
    if ((rc = ev.record(0))) return rc;
    k_reduce_k_tile<<<(unsigned)ep.ntiles, kRkThreads, 0, s>>>(ss, static_cast<uint8_t *>(d_out), ws, ep, dp);
    UZIP_LAUNCH_CHECK("k_reduce_k_tile");
    if ((rc = ev.record(1))) return rc;
    return finish_encode(L, cb, ep, ws, static_cast<uint8_t *>(d_out), ev, s);
}

int uzip_reduce_k(const void *const *d_in, const uint64_t *in_bytes, uint32_t k, uint64_t n, uint32_t chunk,
                  const uzip_codebook_t *cb, void *d_out, uint64_t out_cap, void *d_ws, uint64_t ws_bytes,
                  hipStream_t s)
{
    return uzip_reduce_k_ex(d_in, in_bytes, k, n, chunk, cb, d_out, out_cap, d_ws, ws_bytes, nullptr, s);
}

int uzip_validate(const void *d_stream, uint64_t bytes, const uzip_codebook_t *cb, hipStream_t s)
{
    if (!d_stream || !cb || bytes < kHeader) return d_stream && cb ? UZIP_ECORRUPT : UZIP_EINVAL;
    uint8_t *h = static_cast<uint8_t *>(malloc(bytes));
    if (!h) return UZIP_ENOSPC;
    hipError_t e = hipMemcpyAsync(h, d_stream, bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        free(h);
        return hip_fail(e, "hipMemcpyAsync");
    }
    int rc = uzip_validate_host(h, bytes, cb);
    free(h);
    return rc;
}

}  // extern "C"
