/*
 * fp4_oracle.c -- plain, slow CPU oracle for FP4 (E2M1) block-scaled
 * quantisation and matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; it shares no source, header, table or constant
 * generator with the HIP path.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it.
 *
 * Every number format below is written out from its definition, with scalar
 * loops and, for the matrix product, FP64 accumulation.  Compile with
 * -O2 -fno-fast-math -ffp-contract=off so that every FP32 operation written
 * here rounds exactly once, as IEEE-754 binary32 round-to-nearest-even.
 *
 * Sources (the pages this oracle follows):
 *   [P1] "Rubin架构FP4 GEMM深度解析" (yfxerp.com/news/178243):
 *        §3.1 E2M1 with one mantissa bit, block scaling, E8M0 power-of-two
 *        scales, GEMM result times the product of the two scales;
 *        §4.2 epilogue C = (A_fp4 * B_fp4) * (scaleA * scaleB);
 *        §3.4 weights and activations may take different precisions
 *        (activations kept in FP8 while weights go to FP4);
 *        §5.2 two FP4 values per byte, order must be fixed explicitly.
 *   [P2] NVFP4 video transcript (prism.simon-ai.net/article/7890):
 *        MXFP4 = 32-value blocks with a power-of-two scale (a scale of 70
 *        must become 64 or 128); NVFP4 = 16-value blocks, E4M3 block scale,
 *        plus one FP32 tensor scale for the global range.
 *   [P4] Ultralytics glossary "FP4" (ultralytics.com/ru/glossary/fp4),
 *        "How FP4 works": the E2M1 value set {0, ±0.5, ±1, ±1.5, ±2, ±3,
 *        ±4, ±6}; the block scale maps the block's largest magnitude to 6;
 *        the worked example rounds |x|/scale to the nearest grid value and
 *        dequantises as grid * sign * scale.
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes): round-to-nearest-even onto the grid; MXFP4 exponent = the
 * smallest e with amax <= 6 * 2^e ("ceil"), with the OCP-style
 * floor(log2 amax) - 2 rule as a second mode; E4M3 = bias 7, max 448, no
 * infinities, rounding to nearest-even with saturation; NVFP4 tensor scale
 * s_t = amax_t / (6 * 448); low nibble holds the even-K element.  MXFP8
 * (the FP8 operand of a mixed product, [P1] §3.1 names MXFP8 beside MXFP4):
 * E4M3 elements, one byte each, under 32-block E8M0 scales chosen by the
 * MXFP4 rules with 448 in place of 6.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <float.h>

#define OR_FMT_MXFP4 0
#define OR_FMT_NVFP4 1
#define OR_FMT_MXFP4_OCP 2
#define OR_FMT_MXFP8 3
#define OR_FMT_MXFP8_OCP 4
#define IS_MX8(fmt) ((fmt) == OR_FMT_MXFP8 || (fmt) == OR_FMT_MXFP8_OCP)

#define OR_DT_F32 0
#define OR_DT_BF16 1

/* ------------------------------------------------------------------ */
/* E2M1 ([P4] "How FP4 works": the eight non-negative values; [P1] §3.1:
 * 1 sign bit, 2 exponent bits, 1 mantissa bit, bias 1).               */
/* ------------------------------------------------------------------ */

/* Magnitude of each 3-bit code, written from the format: exponent field
 * E = code>>1, mantissa bit M = code&1; E == 0 is subnormal (M * 0.5),
 * otherwise (1 + M/2) * 2^(E-1). */
double oracle_e2m1_value(int code)
{
    int mag = code & 7;
    int E = mag >> 1, M = mag & 1;
    double v = (E == 0) ? 0.5 * M : (1.0 + 0.5 * M) * ldexp(1.0, E - 1);
    return (code & 8) ? -v : v;
}

/* Nearest grid magnitude to y >= 0, ties to the even code (the grid's
 * round-to-nearest-even); values beyond 6 land on 6 because 6 is then the
 * nearest grid point.  Plain argmin over the eight candidates. */
int oracle_e2m1_encode_mag(float y)
{
    if (y >= 6.0f)
        return 7; /* at or past the top of the grid 6 is the nearest value */
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs((double)y - oracle_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* The page's worked example ([P4]): nearest grid point by argmin, the
 * first (lower) candidate winning a tie, as torch.argmin does. */
static int e2m1_encode_mag_first(float y)
{
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs((double)y - oracle_e2m1_value(c));
        if (d < bestd) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* E8M0 ([P1] §3.1, §4.2: a pure power-of-two exponent byte).  Bias 127;
 * byte 255 would be NaN and is never produced.                        */
/* ------------------------------------------------------------------ */
double oracle_e8m0_value(int byte) { return ldexp(1.0, byte - 127); }

/* Default rule: the smallest e in [-127, 127] with amax <= 6 * 2^e, i.e.
 * the power of two that maps the block maximum closest to 6 from below
 * without clipping ([P4]: largest magnitude mapped to 6; [P2]: the scale
 * must be a power of two).  Found by counting upward, exactly in FP64. */
int oracle_mx_exponent(float amax)
{
    int e = -127;
    while (e < 127 && (double)amax > 6.0 * ldexp(1.0, e))
        ++e;
    return e;
}

/* Second rule (the OCP MX choice the pages name in [P1] §3.1):
 * e = floor(log2 amax) - 2, where 2 is E2M1's largest exponent, clamped to
 * the E8M0 range; elements above 6 then saturate to 6. */
int oracle_mx_exponent_ocp(float amax)
{
    if (amax == 0.0f)
        return -127;
    int ex;
    (void)frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------ */
/* E4M3 ([P2]: NVFP4 block scale with 4 exponent and 3 mantissa bits).
 * Reading: OCP FP8 E4M3 -- bias 7, subnormals, no infinity, only
 * S.1111.111 is NaN, so the largest finite value is 448.             */
/* ------------------------------------------------------------------ */
double oracle_e4m3_value(int byte)
{
    int E = (byte >> 3) & 15, M = byte & 7;
    double v = (E == 0) ? M * ldexp(1.0, -9) : (1.0 + M / 8.0) * ldexp(1.0, E - 7);
    return (byte & 0x80) ? -v : v;
}

/* Nearest finite non-negative E4M3 value to r >= 0, ties to the even code;
 * anything above 448 saturates to 448 (the nearest finite value). */
int oracle_e4m3_encode(float r)
{
    if (r >= 448.0f)
        return 0x7E; /* at or past the largest finite value, 448 is nearest */
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 127; ++c) { /* 0x7F is NaN */
        double d = fabs((double)r - oracle_e4m3_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* MXFP8 scale ([P1] §3.1: MX formats share one power-of-two E8M0 scale per
 * block; §3.4: FP8 activations beside FP4 weights).  The MXFP4 rules with
 * E4M3's largest value 448 (= 1.75 * 2^8) in place of 6:
 *   default: the smallest e in [-127, 127] with amax <= 448 * 2^e, found
 *            by counting upward, exactly in FP64 (no element clips);
 *   OCP:     e = floor(log2 amax) - 8, 8 being E4M3's largest exponent,
 *            clamped; scaled elements above 448 then saturate to 448.   */
/* ------------------------------------------------------------------ */
int oracle_mx8_exponent(float amax)
{
    int e = -127;
    while (e < 127 && (double)amax > 448.0 * ldexp(1.0, e))
        ++e;
    return e;
}

int oracle_mx8_exponent_ocp(float amax)
{
    if (amax == 0.0f)
        return -127;
    int ex;
    (void)frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
    int e = (ex - 1) - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------ */
/* BF16 <-> FP32: BF16 keeps the top 16 bits of an FP32; rounding to it is
 * round-to-nearest-even on the dropped 16 bits (finite inputs).        */
/* ------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t oracle_f32_to_bf16(float f)
{
    /* Among the two BF16 neighbours (truncation and truncation + 1 ulp),
     * take the nearer; on a tie take the one with an even last bit. */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lo = u & 0xFFFF0000u;
    uint32_t hi = lo + 0x10000u;
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    /* Past the largest BF16 the upper neighbour is infinity, which rounding
     * treats as the next power of two, 2^128. */
    double vhi = isinf(fhi) ? copysign(ldexp(1.0, 128), fhi) : (double)fhi;
    double dlo = fabs((double)f - (double)flo);
    double dhi = fabs((double)f - vhi);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* ------------------------------------------------------------------ */
/* Scale-buffer layout (the library's documented byte order).  Scales
 * live in tiles of 32 rows x 256 K values, stored row-tile major; inside
 * a tile, row i and 32-value K chunk c (c = 0..7) belong to "lane"
 * 32*(c%2) + i and "sub-step" c/2.
 *   MXFP4 (32-blocks): 256-byte tiles; lane L holds 4 bytes at 4L, byte
 *     s = the sub-step's block (block q = chunk q).
 *   NVFP4 (16-blocks): 512-byte tiles; lane L holds 8 bytes at 8L, bytes
 *     2s and 2s+1 = the sub-step chunk's two blocks (block q is in chunk
 *     q/2, half q%2).
 * Padding rows and blocks hold 0.                                      */
/* ------------------------------------------------------------------ */
static int64_t block_size(int fmt) { return fmt == OR_FMT_NVFP4 ? 16 : 32; }
static int64_t tile_bytes(int fmt) { return fmt == OR_FMT_NVFP4 ? 512 : 256; }

int64_t oracle_scale_bytes(int fmt, int64_t rows, int64_t K)
{
    int64_t KT = (K + 255) / 256;
    return ((rows + 31) / 32) * KT * tile_bytes(fmt);
}

int64_t oracle_scale_offset(int fmt, int64_t rows, int64_t K, int64_t r, int64_t b)
{
    (void)rows;
    int64_t KT = (K + 255) / 256;
    int64_t k0 = b * block_size(fmt);          /* first K value of the block */
    int64_t tile = (r / 32) * KT + k0 / 256;
    int64_t i = r % 32, c = (k0 % 256) / 32;    /* row and chunk in the tile */
    int64_t lane = 32 * (c % 2) + i, s = c / 2;
    if (fmt == OR_FMT_NVFP4)
        return tile * 512 + lane * 8 + 2 * s + (b % 2);
    return tile * 256 + lane * 4 + s;
}

/* ------------------------------------------------------------------ */
/* Quantisation.                                                        */
/* ------------------------------------------------------------------ */
static float load_elem(const void* x, int dt, int64_t idx)
{
    if (dt == OR_DT_BF16)
        return oracle_bf16_to_f32(((const uint16_t*)x)[idx]);
    return ((const float*)x)[idx];
}

/* NVFP4 tensor scale ([P2]: one FP32 scale for the global range).
 * Reading: s_t = amax_t / (6 * 448) in FP32, so the block holding the
 * tensor's largest magnitude gets the largest E4M3 scale; an all-zero
 * tensor takes s_t = 1; s_t is kept at or above the smallest normal
 * FP32 so the block-scale division stays finite. */
float oracle_nvfp4_tensor_scale(float amax_t)
{
    if (amax_t == 0.0f)
        return 1.0f;
    float s = amax_t / 2688.0f;
    if (s < FLT_MIN)
        s = FLT_MIN;
    return s;
}

float oracle_tensor_amax(const void* x, int dt, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_elem(x, dt, i));
        if (a > m) m = a;
    }
    return m;
}

/* ------------------------------------------------------------------ */
/* Stochastic rounding ([P2], the training recipe's fourth part: a value
 * between two representable points goes up with probability equal to its
 * distance from the lower point -- 0.3 becomes 1 with probability 30% and
 * 0 otherwise -- so the expectation is kept).
 * Random words come from Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011), a counter-
 * based generator: ten rounds, each two 64 x 64 -> 128-bit products of
 * counter words with the multipliers below, mixed with the key; the key is
 * advanced by the two Weyl constants between rounds.                     */
/* ------------------------------------------------------------------ */
void oracle_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out)
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* The 32-bit random word of element i (row-major flat index of the
 * quantised matrix) under `seed`: Philox4x64-10 with key (seed, 0) and
 * counter (i / 8, 0, 0, 0); word (i mod 8) / 2 of the output, its low 32
 * bits for even i, high 32 bits for odd i.  (Reading: the pages name no
 * generator; a counter-based one makes the result a function of the seed
 * and the element alone.) */
uint32_t oracle_sr_word(uint64_t seed, uint64_t i)
{
    uint64_t ctr[4] = {i >> 3, 0, 0, 0}, key[2] = {seed, 0}, out[4];
    oracle_philox4x64_10(ctr, key, out);
    uint64_t w = out[(i & 7) >> 1];
    return (uint32_t)((i & 1) ? (w >> 32) : w);
}

/* E2M1 magnitude code of y >= 0 rounded stochastically with word r: lo =
 * the largest grid value <= y (y >= 6 saturates to code 7), hi the next
 * one; round up iff u * (hi - lo) < y - lo with u = (r >> 8) * 2^-24.
 * Every quantity is exact in FP32 (hi - lo is a power of two; y - lo is
 * exact because lo >= hi / 2 or lo = 0), so the decision is too, and
 * P(up) = ceil((y - lo) / (hi - lo) * 2^24) / 2^24. */
int oracle_e2m1_sr_mag(float y, uint32_t r)
{
    int lo = 0;
    while (lo < 7 && (float)oracle_e2m1_value(lo + 1) <= y)
        ++lo;
    if (lo == 7)
        return 7;
    float glo = (float)oracle_e2m1_value(lo), ghi = (float)oracle_e2m1_value(lo + 1);
    float u = (float)(r >> 8) * 0x1p-24f;
    return (u * (ghi - glo) < y - glo) ? lo + 1 : lo;
}

/* Quantise one block of `bs` values.  Writes 4-bit codes (one per byte, in
 * codes_out[0..bs)) and returns the scale byte.  `rule` is the format;
 * s_t is the NVFP4 tensor scale (ignored for MXFP4).  sr: round the
 * elements stochastically (element k's word: oracle_sr_word(seed, base + k));
 * the scales are chosen exactly as without it. */
static int quantize_block(const float* v, int bs, int rule, float s_t, uint8_t* codes_out, int sr, uint64_t seed,
                          int64_t base, float amax_in)
{
    float amax = 0.0f;
    for (int k = 0; k < bs; ++k)
        if (fabsf(v[k]) > amax) amax = fabsf(v[k]);
    if (amax_in >= 0.0f)
        amax = amax_in;   /* 2-D scaling: the 16 x 16 patch's maximum */

    int sbyte;
    if (rule == OR_FMT_NVFP4) {
        /* r = (amax_b / 6) / s_t, two FP32 divisions; block scale = E4M3 of
         * r; effective divisor d = E4M3(r) * s_t in FP32. */
        float r = (amax / 6.0f) / s_t;
        sbyte = oracle_e4m3_encode(r);
        float d = (float)oracle_e4m3_value(sbyte) * s_t;
        for (int k = 0; k < bs; ++k) {
            int sign = signbit(v[k]) ? 8 : 0;
            float y = (sbyte == 0) ? 0.0f : fabsf(v[k]) / d;
            int mag = sr ? oracle_e2m1_sr_mag(y, oracle_sr_word(seed, (uint64_t)(base + k)))
                         : oracle_e2m1_encode_mag(y);
            codes_out[k] = (uint8_t)(sign | mag);
        }
    } else if (IS_MX8(rule)) {
        /* MXFP8: y = |x| * 2^-e (exact), E4M3 byte nearest to y with ties
         * to even, saturating at 448; bit 7 = the input's sign bit. */
        int e = (rule == OR_FMT_MXFP8_OCP) ? oracle_mx8_exponent_ocp(amax) : oracle_mx8_exponent(amax);
        sbyte = e + 127;
        for (int k = 0; k < bs; ++k) {
            int sign = signbit(v[k]) ? 0x80 : 0;
            float y = ldexpf(fabsf(v[k]), -e);
            codes_out[k] = (uint8_t)(sign | oracle_e4m3_encode(y));
        }
    } else {
        int e = (rule == OR_FMT_MXFP4_OCP) ? oracle_mx_exponent_ocp(amax) : oracle_mx_exponent(amax);
        sbyte = e + 127;
        for (int k = 0; k < bs; ++k) {
            int sign = signbit(v[k]) ? 8 : 0;
            float y = ldexpf(fabsf(v[k]), -e);
            int mag = sr ? oracle_e2m1_sr_mag(y, oracle_sr_word(seed, (uint64_t)(base + k)))
                         : oracle_e2m1_encode_mag(y);
            codes_out[k] = (uint8_t)(sign | mag);
        }
    }
    return sbyte;
}

/* Quantise a rows x K matrix (K contiguous).
 *   codes:  rows x K/2 bytes, element 2i in bits 0-3 of byte i, 2i+1 in
 *           bits 4-7 ([P1] §5.2 leaves the order open; this is the reading);
 *           MXFP8: rows x K bytes, one E4M3 byte per element.
 *   scales: the tiled layout above (oracle_scale_bytes bytes), or, when
 *           scales_canon is non-NULL, additionally rows x K/bs canonical.
 *   tensor_scale: NVFP4 only.  If ts_given, *tensor_scale is read;
 *           otherwise it is computed from the whole operand and written.
 * Returns 0, or -1 on a shape the formats do not define. */
/* 2-D block scaling ([P2], the training recipe's second part: a weight
 * matrix is used as W in the forward pass and as W^T in the backward pass,
 * so NVFP4 scales are shared by 16 x 16 patches instead of 1 x 16 blocks;
 * W and W^T then quantise alike).  Reading: the patch of rows 16p..16p+15
 * (those inside the matrix) and columns 16b..16b+15 takes the E4M3 scale of
 * its largest magnitude, and every row of it uses that scale; rows past the
 * matrix keep scale byte 0 as in the 1-D layout.                          */
static int quantize_matrix(const void* x, int dt, int fmt, int64_t rows, int64_t K, uint8_t* codes,
                           uint8_t* scales, uint8_t* scales_canon, float* tensor_scale, int ts_given, int sr,
                           uint64_t seed, int twod)
{
    int bs = (int)block_size(fmt);
    if (rows < 0 || K < 0 || K % bs != 0)
        return -1;
    if (twod && fmt != OR_FMT_NVFP4)
        return -1;
    if (sr && IS_MX8(fmt))
        return -1;   /* stochastic rounding is defined for the E2M1 grid only */
    float s_t = 1.0f;
    if (fmt == OR_FMT_NVFP4) {
        if (ts_given) {
            s_t = *tensor_scale;
        } else {
            s_t = oracle_nvfp4_tensor_scale(oracle_tensor_amax(x, dt, rows * K));
            *tensor_scale = s_t;
        }
    }
    memset(scales, 0, (size_t)oracle_scale_bytes(fmt, rows, K));
    int64_t KB = K / bs;
    float v[32];
    uint8_t c[32];
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            for (int k = 0; k < bs; ++k)
                v[k] = load_elem(x, dt, r * K + b * bs + k);
            float pm = -1.0f;
            if (twod) {
                pm = 0.0f;
                int64_t r0 = r - r % 16, r1 = r0 + 16 < rows ? r0 + 16 : rows;
                for (int64_t rr = r0; rr < r1; ++rr)
                    for (int k = 0; k < bs; ++k) {
                        float a = fabsf(load_elem(x, dt, rr * K + b * bs + k));
                        if (a > pm) pm = a;
                    }
            }
            int sb = quantize_block(v, bs, fmt, s_t, c, sr, seed, r * K + b * bs, pm);
            scales[oracle_scale_offset(fmt, rows, K, r, b)] = (uint8_t)sb;
            if (scales_canon)
                scales_canon[r * KB + b] = (uint8_t)sb;
            if (IS_MX8(fmt)) {
                for (int k = 0; k < bs; ++k)
                    codes[r * K + b * bs + k] = c[k];   /* one byte per element */
            } else {
                for (int k = 0; k < bs; k += 2)
                    codes[(r * K + b * bs + k) / 2] = (uint8_t)(c[k] | (c[k + 1] << 4));
            }
        }
    }
    return 0;
}

int oracle_quantize(const void* x, int dt, int fmt, int64_t rows, int64_t K, uint8_t* codes,
                    uint8_t* scales, uint8_t* scales_canon, float* tensor_scale, int ts_given)
{
    return quantize_matrix(x, dt, fmt, rows, K, codes, scales, scales_canon, tensor_scale, ts_given, 0, 0, 0);
}

/* As oracle_quantize, with the elements rounded stochastically under `seed`
 * (scales unchanged). */
int oracle_quantize_sr(const void* x, int dt, int fmt, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales, uint8_t* scales_canon, float* tensor_scale, int ts_given, uint64_t seed)
{
    return quantize_matrix(x, dt, fmt, rows, K, codes, scales, scales_canon, tensor_scale, ts_given, 1, seed, 0);
}

/* Both options: sr (stochastic rounding under seed) and twod (NVFP4 16 x 16
 * patch scales). */
int oracle_quantize_ex(const void* x, int dt, int fmt, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                       uint8_t* scales_canon, float* tensor_scale, int ts_given, int sr, uint64_t seed, int twod)
{
    return quantize_matrix(x, dt, fmt, rows, K, codes, scales, scales_canon, tensor_scale, ts_given, sr, seed, twod);
}

/* ------------------------------------------------------------------ */
/* Random Hadamard transform ([P2], the training recipe's third part: the
 * values of a block are mixed so that an outlier no longer sets the block
 * scale alone; the vector's magnitude is unchanged and dot products
 * survive because the transform is orthogonal).  Reading: on every
 * 16-value block along K (the NVFP4 block), y = (1/4) H16 D x, with D the
 * diagonal of signs s_k = -1 if the top bit of oracle_sr_word(seed, k) is
 * set, else +1 (k = column, so two matrices transformed with one seed keep
 * their products along K), and H16 the 16-point Walsh-Hadamard matrix
 * applied as butterflies of distance 1, 2, 4, 8 (a + b, a - b) in FP32,
 * in that order; the 1/4 is exact.  Output FP32.                        */
/* ------------------------------------------------------------------ */
void oracle_rht16(const void* x, int dt, int64_t rows, int64_t K, uint64_t seed, float* y)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K / 16; ++b) {
            float v[16];
            for (int k = 0; k < 16; ++k) {
                int64_t col = b * 16 + k;
                float s = (oracle_sr_word(seed, (uint64_t)col) >> 31) ? -1.0f : 1.0f;
                v[k] = load_elem(x, dt, r * K + col) * s;
            }
            for (int h = 1; h < 16; h *= 2)
                for (int i = 0; i < 16; i += 2 * h)
                    for (int m = i; m < i + h; ++m) {
                        float a = v[m], c = v[m + h];
                        v[m] = a + c;
                        v[m + h] = a - c;
                    }
            for (int k = 0; k < 16; ++k)
                y[r * K + b * 16 + k] = v[k] * 0.25f;
        }
}

/* Exact value of element (r, k) of a quantised matrix, without the tensor
 * scale: E2M1(code) * block scale ([P4]: grid * sign * scale); MXFP8:
 * E4M3(byte) * 2^(scale byte - 127). */
static double elem_value(const uint8_t* codes, const uint8_t* scales, int fmt, int64_t rows, int64_t K,
                         int64_t r, int64_t k)
{
    int bs = (int)block_size(fmt);
    int sb = scales[oracle_scale_offset(fmt, rows, K, r, k / bs)];
    if (IS_MX8(fmt))
        return oracle_e4m3_value(codes[r * K + k]) * oracle_e8m0_value(sb);
    uint8_t byte = codes[(r * K + k) / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 15);
    double s = (fmt == OR_FMT_NVFP4) ? oracle_e4m3_value(sb) : oracle_e8m0_value(sb);
    return oracle_e2m1_value(code) * s;
}

/* Dequantise to FP32 or BF16.  MXFP4: E2M1 * 2^(byte-127), exact (MXFP8
 * likewise, for the scale bytes the quantiser produces).  NVFP4:
 * (E2M1 * E4M3) * s_t -- the first product is exact, the second is one
 * FP32 rounding.  BF16 output is the round-to-nearest-even of that FP32. */
void oracle_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int fmt,
                       void* out, int out_dt, int64_t rows, int64_t K)
{
    double s_t = (fmt == OR_FMT_NVFP4) ? (double)*tensor_scale : 1.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            /* p * s_t is exact in FP64 (<= 6 + 24 significant bits); the cast
             * to float is then the single FP32 rounding. */
            float f = (float)(elem_value(codes, scales, fmt, rows, K, r, k) * s_t);
            if (out_dt == OR_DT_BF16)
                ((uint16_t*)out)[r * K + k] = oracle_f32_to_bf16(f);
            else
                ((float*)out)[r * K + k] = f;
        }
}

/* ------------------------------------------------------------------ */
/* Matrix multiply ([P1] §1.1: FP4 inputs, FP32 accumulation; §3.1 and
 * §4.2: result times the product of the scales).  The oracle is the exact
 * definition evaluated in FP64:
 *   C[m,n] = (sum_k A^[m,k] * B^[n,k]) * tsA * tsB
 *   T[m,n] = (sum_k |A^[m,k] * B^[n,k]|) * |tsA * tsB|
 * with A^, B^ the dequantised values without tensor scales.  A is M x K,
 * B is N x K (one row per output column).  T bounds accumulation error:
 * a result is accepted when |C - Cref| <= 1e-5 * T.                     */
/* ------------------------------------------------------------------ */
/* Mixed operands ([P1] §3.4: A and B in different formats, e.g. FP8
 * activations times FP4 weights): A in format fmtA, B in fmtB. */
void oracle_gemm_mixed(const uint8_t* A, const uint8_t* sA, int fmtA, const uint8_t* B, const uint8_t* sB,
                       int fmtB, double tsA, double tsB, int64_t M, int64_t N, int64_t K, double* C, double* T)
{
    double ts = tsA * tsB;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = elem_value(A, sA, fmtA, M, K, m, k) * elem_value(B, sB, fmtB, N, K, n, k);
                acc += p;
                mag += fabs(p);
            }
            C[m * N + n] = acc * ts;
            if (T) T[m * N + n] = mag * fabs(ts);
        }
}

void oracle_gemm(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, double tsA,
                 double tsB, int64_t M, int64_t N, int64_t K, int fmt, double* C, double* T)
{
    oracle_gemm_mixed(A, sA, fmt, B, sB, fmt, tsA, tsB, M, N, K, C, T);
}

/* ------------------------------------------------------------------ */
/* Epilogue ([P1] §3.2: the FP32 result is multiplied by the scales, the
 * bias is added, the activation applied, and the value converted to FP4
 * if wanted; §4.2: C = (A_fp4 * B_fp4) * (scaleA * scaleB) + bias).  From
 * the scaled product Cref (FP64, as oracle_gemm returns it):
 *   v = Cref[m,n] + bias[n]   (bias NULL: no addition, so -0 stays -0),
 *       summed in FP64 and rounded once to FP32;
 *   act 1 (ReLU, the pages leave the function unnamed): v > 0 ? v : +0,
 *       so -0 becomes +0.
 * An FP4 output is then oracle_quantize of v (rows M, K = N).           */
/* ------------------------------------------------------------------ */
void oracle_epilogue(const double* C, const float* bias, int act, int64_t M, int64_t N, float* out)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = C[m * N + n];
            if (bias) v += (double)bias[n];
            float f = (float)v;
            if (act == 1) f = f > 0.0f ? f : 0.0f;
            out[m * N + n] = f;
        }
}

/* Only the listed output elements (rows[i], cols[i]); for sampled checks at
 * sizes where the full product would take too long on the CPU. */
void oracle_gemm_mixed_sampled(const uint8_t* A, const uint8_t* sA, int fmtA, const uint8_t* B,
                               const uint8_t* sB, int fmtB, double tsA, double tsB, int64_t M, int64_t N,
                               int64_t K, const int64_t* rows, const int64_t* cols, int64_t count, double* C,
                               double* T)
{
    double ts = tsA * tsB;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = elem_value(A, sA, fmtA, M, K, rows[i], k) * elem_value(B, sB, fmtB, N, K, cols[i], k);
            acc += p;
            mag += fabs(p);
        }
        C[i] = acc * ts;
        if (T) T[i] = mag * fabs(ts);
    }
}

void oracle_gemm_sampled(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, double tsA,
                         double tsB, int64_t M, int64_t N, int64_t K, int fmt, const int64_t* rows,
                         const int64_t* cols, int64_t count, double* C, double* T)
{
    oracle_gemm_mixed_sampled(A, sA, fmt, B, sB, fmt, tsA, tsB, M, N, K, rows, cols, count, C, T);
}

/* Grouped product for mixture-of-experts layers ([P4], "Inference and
 * training in FP4": MXFP4 expert weights).  Output row r belongs to the
 * expert e with group_off[e] <= r < group_off[e+1]; it multiplies token
 * row row_idx[r] of A (T_rows x K) by expert e's weights B_e (N x K,
 * stored one expert after another, codes N*K/2 bytes and scales
 * oracle_scale_bytes(fmt, N, K) bytes apart).  Only the listed
 * (out_rows[i], cols[i]) are evaluated. */
void oracle_gemm_grouped_sampled(const uint8_t* A, const uint8_t* sA, int64_t T_rows, const int32_t* row_idx,
                                 const int32_t* group_off, int32_t E, const uint8_t* B, const uint8_t* sB,
                                 double tsA, double tsB, int64_t N, int64_t K, int fmt,
                                 const int64_t* out_rows, const int64_t* cols, int64_t count, double* C,
                                 double* T)
{
    double ts = tsA * tsB;
    int64_t cb = N * K / 2, sbytes = oracle_scale_bytes(fmt, N, K);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i) {
        int64_t r = out_rows[i];
        int32_t e = 0;
        while (e < E && !(group_off[e] <= r && r < group_off[e + 1]))
            ++e;
        double acc = 0.0, mag = 0.0;
        if (e < E) {
            const uint8_t* Be = B + e * cb;
            const uint8_t* sBe = sB + e * sbytes;
            for (int64_t k = 0; k < K; ++k) {
                double p = elem_value(A, sA, fmt, T_rows, K, row_idx[r], k) *
                           elem_value(Be, sBe, fmt, N, K, cols[i], k);
                acc += p;
                mag += fabs(p);
            }
        }
        C[i] = acc * ts;
        if (T) T[i] = mag * fabs(ts);
    }
}

/* ------------------------------------------------------------------ */
/* Mean absolute quantisation error of a vector at a given block size
 * ([P4], worked example: whole tensor, then 32- and 16-value blocks).
 *   mode 0 ("page"): scale = amax/6 in FP32, no scale encoding, nearest
 *           grid point with the first candidate winning a tie,
 *           dequantised = grid * sign * scale in FP32 -- the page's recipe.
 *   mode 1: MXFP4 default exponent rule at this block size.
 *   mode 2: MXFP4 OCP exponent rule at this block size.
 *   mode 3: NVFP4 two-level scaling at this block size.
 * The mean is taken in FP64.                                            */
/* ------------------------------------------------------------------ */
double oracle_block_mae(const float* x, int64_t n, int64_t bs, int mode)
{
    double sum = 0.0;
    float s_t = 1.0f;
    if (mode == 3)
        s_t = oracle_nvfp4_tensor_scale(oracle_tensor_amax(x, OR_DT_F32, n));
    for (int64_t b0 = 0; b0 < n; b0 += bs) {
        float amax = 0.0f;
        for (int64_t k = 0; k < bs; ++k)
            if (fabsf(x[b0 + k]) > amax) amax = fabsf(x[b0 + k]);
        for (int64_t k = 0; k < bs; ++k) {
            float v = x[b0 + k];
            float sign = (v > 0.0f) ? 1.0f : (v < 0.0f ? -1.0f : 0.0f);
            float deq;
            if (mode == 0) {
                float scale = amax / 6.0f;
                int c = e2m1_encode_mag_first(fabsf(v) / scale);
                deq = (float)oracle_e2m1_value(c) * sign * scale;
            } else if (mode == 3) {
                float r = (amax / 6.0f) / s_t;
                int sb = oracle_e4m3_encode(r);
                float d = (float)oracle_e4m3_value(sb) * s_t;
                int c = (sb == 0) ? 0 : oracle_e2m1_encode_mag(fabsf(v) / d);
                deq = (float)((double)oracle_e2m1_value(c) * oracle_e4m3_value(sb) * (double)s_t) * sign;
            } else {
                int e = (mode == 2) ? oracle_mx_exponent_ocp(amax) : oracle_mx_exponent(amax);
                int c = oracle_e2m1_encode_mag(ldexpf(fabsf(v), -e));
                deq = (float)(oracle_e2m1_value(c) * ldexp(1.0, e)) * sign;
            }
            sum += fabs((double)deq - (double)v);
        }
    }
    return sum / (double)n;
}

/* ------------------------------------------------------------------ */
/* Batch helpers so the tests can sweep many inputs per call.          */
/* ------------------------------------------------------------------ */
void oracle_e2m1_encode_mag_batch(const float* y, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)oracle_e2m1_encode_mag(y[i]);
}

void oracle_e4m3_encode_batch(const float* r, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)oracle_e4m3_encode(r[i]);
}

void oracle_mx_exponent_batch(const float* amax, int64_t n, int ocp, int32_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ocp ? oracle_mx_exponent_ocp(amax[i]) : oracle_mx_exponent(amax[i]);
}

void oracle_f32_to_bf16_batch(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(f[i]);
}
