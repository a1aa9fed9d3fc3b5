// fp4_device.h -- device-side number-format helpers shared by the libfp4
// kernels (gfx950).  Internal header; not part of the C ABI.
//
// Formats (sources: Ultralytics glossary "FP4", "How FP4 works"; NVFP4 video
// transcript, prism.simon-ai.net; "Rubin FP4 GEMM deep dive", yfxerp.com §3.1):
//   E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa, values 0..6.
//   E8M0: power-of-two scale byte, 2^(byte - 127).
//   E4M3: bias 7, 3-bit mantissa, subnormals, largest finite 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFmtMX = 0, kFmtNV = 1, kFmtMXOcp = 2;
// MXFP8: E4M3 elements (one byte each) under 32-block E8M0 scales.
constexpr int kFmtMX8 = 3, kFmtMX8Ocp = 4;

// Input / output element types (the C ABI's fp4_dtype values).
constexpr int kDtF32 = 0, kDtBF16 = 1;

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ---- cross-lane moves by DPP (VALU, no LDS round trip).  Every lane of the
// wavefront must be active where they are used.
// The value of lane ^ 1 (quad_perm [1, 0, 3, 2]) and of lane ^ 2 ([2, 3, 0, 1]).
__device__ __forceinline__ float lane_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
// fmaxf over the wavefront, in every lane: rotations by 1, 2, 4 and 8 inside
// each row of 16 lanes (DPP row_ror), then the four rows' results.
__device__ __forceinline__ float wave_fmax(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
  const int x = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Magnitude code (0..7) of the E2M1 value nearest to y >= 0, ties to the even
// code, saturating at 6: count the rounding boundaries y has passed.  A
// boundary that is a tie is passed only when the code above it is even.
__device__ __forceinline__ uint32_t e2m1_mag(float y) {
  return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) + (uint32_t)(y >= 1.75f) +
         (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) + (uint32_t)(y > 5.0f);
}

// E8M0 byte of an MXFP4 block from its largest magnitude (finite, >= 0).
// Default rule: the smallest e with amax <= 6 * 2^e.  With amax = m * 2^E,
// m in [1, 2): e = E - 2 if m <= 1.5, else E - 1; zero and subnormal maxima
// clamp to e = -127 (byte 0).  In FP32 bits: byte = max(0, exp_field - 2 +
// (mantissa > 0x400000)).
// OCP rule: e = floor(log2 amax) - 2, i.e. byte = max(0, exp_field - 2).
template <int FMT>
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  uint32_t u = f2u(amax);
  int be = (int)(u >> 23);
  int b = be - 2;
  if (FMT == kFmtMX) b += ((u & 0x7FFFFFu) > 0x400000u) ? 1 : 0;
  return (uint32_t)(b < 0 ? 0 : b);
}

// E8M0 byte of an MXFP8 block: the MXFP4 rules with E4M3's largest value
// 448 = 1.75 * 2^8 in place of 6.  Default: the smallest e with
// amax <= 448 * 2^e, i.e. e = E - 8 if m <= 1.75, else E - 7 (amax = m * 2^E);
// in FP32 bits byte = max(0, exp_field - 8 + (mantissa > 0x600000)).  OCP:
// e = floor(log2 amax) - 8, byte = max(0, exp_field - 8).
template <int FMT>
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  uint32_t u = f2u(amax);
  int b = (int)(u >> 23) - 8;
  if (FMT == kFmtMX8) b += ((u & 0x7FFFFFu) > 0x600000u) ? 1 : 0;
  return (uint32_t)(b < 0 ? 0 : b);
}

// E4M3 codes of four values (bytes 0..3), each first limited to [-448, 448]
// (saturation; the conversion itself would give NaN above 448.5), then
// converted by the hardware, which rounds to nearest even and keeps the sign
// (-0 -> 0x80).
__device__ __forceinline__ uint32_t e4m3x4_sat(float a, float b, float c, float d) {
  const float lim = 448.0f;
  a = fminf(fmaxf(a, -lim), lim);
  b = fminf(fmaxf(b, -lim), lim);
  c = fminf(fmaxf(c, -lim), lim);
  d = fminf(fmaxf(d, -lim), lim);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// E4M3 byte nearest to r >= 0 (ties to even), saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float r) {
  if (!(r < 448.0f)) return 0x7Eu;                 // also catches +inf
  if (r < 0.015625f) {                              // below 2^-6: step 2^-9
    float m = __builtin_rintf(r * 512.0f);          // exact scaling, then RNE
    return (uint32_t)m;                             // 8 -> 0x08 == 2^-6
  }
  uint32_t u = f2u(r);
  uint32_t e = (u >> 23) - 127 + 7;                 // 1..15
  uint32_t keep = (u >> 20) & 7u;
  uint32_t rest = u & 0xFFFFFu;
  uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  uint32_t code = (e << 3) + keep + up;             // a carry bumps the exponent
  return code;
}

// Value of a non-negative E4M3 byte (<= 0x7E) as FP32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;       // m * 2^-9
  return u2f(((e + 120u) << 23) | (m << 20));       // (1 + m/8) * 2^(e-7)
}

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = f2u(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Byte offset of scale (row r, block b) in the tiled layout.  Tiles cover
// 32 rows x 256 K values and are stored row-tile major (KT tiles per row
// tile); inside a tile, row i and 32-value K chunk c (0..7) belong to lane
// 32*(c%2) + i of the 32x32 matrix-core operand, sub-step s = c/2:
//   MXFP4: 256-byte tiles, lane L's 4 bytes at 4L, byte s = chunk's block;
//   NVFP4: 512-byte tiles, lane L's 8 bytes at 8L, bytes 2s, 2s+1 = the
//          chunk's two 16-blocks.
template <int FMT>
__device__ __forceinline__ uint32_t scale_offset(uint32_t r, uint32_t b, uint32_t KT) {
  const uint32_t k0 = (FMT == kFmtNV) ? 16u * b : 32u * b;
  const uint32_t tile = (r >> 5) * KT + (k0 >> 8);
  const uint32_t i = r & 31u, c = (k0 & 255u) >> 5;
  const uint32_t lane = 32u * (c & 1u) + i, s = c >> 1;
  if (FMT == kFmtNV) return tile * 512u + lane * 8u + 2u * s + (b & 1u);
  return tile * 256u + lane * 4u + s;
}


// ---- NVFP4 operand decode to FP16 (exact: E2M1 x E4M3 needs <= 6 significant
// bits and lies in [2^-10, 2688]).

// E4M3 byte (0..0x7E) -> FP16 bits.  Normal values (byte >= 8) keep their
// 3 mantissa bits and rebias the exponent by 8; subnormals m * 2^-9 are normal
// FP16 numbers and are converted through FP32.
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t b) {
  if (b >= 8u) return (b << 7) + 0x2000u;
  const _Float16 h = (_Float16)((float)b * 0.001953125f);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Both halves of a packed FP16 pair set to the E4M3 scale `b`.
__device__ __forceinline__ v2h scale_pair(uint32_t b) {
  const uint32_t h = e4m3_to_f16_bits(b);
  return __builtin_bit_cast(v2h, h | (h << 16));
}

// Eight already-scaled values to eight E2M1 codes (element 2i in the low
// nibble of byte i).  The gfx950 converter rounds x/1.0 to the nearest E2M1
// value, ties to even, saturating at +-6, and keeps the sign (so -0 and
// negative values that round to zero give code 8).
__device__ __forceinline__ uint32_t pack8(const float y[8]) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[0], y[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], 1.0f, 3);
  return r;
}

// x / d rounded to nearest even, for the 16 elements of an NVFP4 block that
// share d (finite, > 0) and rd = 1.0f / d (correctly rounded).  For
// d >= 2^-100: q = RN(|x| * rd) is within a few ulps of |x| / d; each step
// q + RN(|x| - q * d) * rd (the remainder is exact in one FMA) is Markstein's
// correction, and the second one starts from a faithful q, so it returns the
// correctly rounded quotient (no underflow: the quotients that matter,
// >= 0.25, have |x| >= 2^-102).  Tiny d takes the plain division.  The sign
// is copied, so -0 stays -0.
constexpr float kNvDivFastMin = 7.888609052210118e-31f;  // 2^-100

// The d >= 2^-100 branch of nv_div alone (a caller with one d for many x
// takes the branch once).
__device__ __forceinline__ float nv_div_fast(float x, float d, float rd) {
  const float a = __builtin_fabsf(x);
  float q = a * rd;
  q = __builtin_fmaf(__builtin_fmaf(-q, d, a), rd, q);
  q = __builtin_fmaf(__builtin_fmaf(-q, d, a), rd, q);
  return __builtin_copysignf(q, x);
}

__device__ __forceinline__ float nv_div(float x, float d, float rd) {
  if (d >= kNvDivFastMin) return nv_div_fast(x, d, rd);
  return __builtin_copysignf(__builtin_fabsf(x) / d, x);
}

// Two E4M3 bytes (bits 0-15 of w, or 16-31 when HI) as two FP16 values: the
// gfx950 FP8 converter with a unit scale is exact for every finite byte,
// subnormals included.
template <bool HI>
__device__ __forceinline__ v2h e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

__device__ __forceinline__ v2h splat_lo(v2h p) { return __builtin_shufflevector(p, p, 0, 0); }
__device__ __forceinline__ v2h splat_hi(v2h p) { return __builtin_shufflevector(p, p, 1, 1); }

// Eight FP16 values = E2M1 codes of one dword (low nibble first) times s.
// The gfx950 converter gives each code's E2M1 value (scale operand 1.0); the
// packed multiply by the E4M3 scale is exact.
__device__ __forceinline__ v8h decode8(uint32_t w, v2h s) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ---- stochastic rounding (NVFP4 video transcript, the training recipe's
// fourth part: a value between two representable points goes up with
// probability equal to its distance from the lower one, so the expectation
// is kept).  Random words: Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), ten rounds of
// two 64 x 64 -> 128-bit products mixed with the key, the key advanced by
// two Weyl constants between rounds.
//
// The 128-bit product of two 64-bit words, schoolbook from four 32 x 32 -> 64
// partial products (each one v_mad_u64_u32, the carries folded into the
// addends: no sum below can exceed 2^64 - 1).  Computing the low half with a
// plain 64-bit multiply and the high half with __umul64hi repeats partial
// products, and the multiplies are what bound the stochastic quantiser.
__device__ __forceinline__ void mul_wide_u64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32), b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t t = (uint64_t)a0 * b1 + (p00 >> 32);
  const uint64_t u = (uint64_t)a1 * b0 + (uint32_t)t;
  lo = (u << 32) | (uint32_t)p00;
  hi = (uint64_t)a1 * b1 + ((t >> 32) + (u >> 32));
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mul_wide_u64(M0, c[0], hi0, lo0);
    mul_wide_u64(M1, c[2], hi1, lo1);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// The random words of elements i0 .. i0 + 7 (row-major flat index of the
// quantised matrix, i0 % 8 == 0) under `seed`: one Philox block with key
// (seed, 0) and counter (i0 / 8, 0, 0, 0); element i0 + j takes word j / 2,
// its low 32 bits for even j.
__device__ __forceinline__ void sr_words8(uint64_t seed, uint64_t i0, uint32_t (&r)[8]) {
  uint64_t c[4] = {i0 >> 3, 0ull, 0ull, 0ull};
  philox4x64_10(c, seed, 0ull);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = (uint32_t)c[j];
    r[2 * j + 1] = (uint32_t)(c[j] >> 32);
  }
}

// E2M1 grid value of magnitude code c (0..7).
__device__ __forceinline__ float e2m1_grid(uint32_t c) {
  return c < 2u ? 0.5f * (float)c : u2f(((c >> 1) + 126u) << 23) * (1.0f + 0.5f * (float)(c & 1u));
}

// Stochastically rounded E2M1 code of an already scaled value y (sign bit
// copied): lo = the largest grid value <= |y| (|y| >= 6 saturates to 6), hi
// the next one; up iff u * (hi - lo) < |y| - lo with u = (r >> 8) * 2^-24.
// Every term is exact in FP32 (hi - lo is a power of two, |y| - lo exact), so
// the decision is exact.
__device__ __forceinline__ uint32_t e2m1_sr_code(float y, uint32_t r) {
  const float a = fabsf(y);
  const uint32_t lo = (uint32_t)(a >= 0.5f) + (uint32_t)(a >= 1.0f) + (uint32_t)(a >= 1.5f) + (uint32_t)(a >= 2.0f) +
                      (uint32_t)(a >= 3.0f) + (uint32_t)(a >= 4.0f) + (uint32_t)(a >= 6.0f);
  const float glo = e2m1_grid(lo), ghi = e2m1_grid(lo < 7u ? lo + 1u : 7u);
  const float u = (float)(r >> 8) * 0x1p-24f;
  const uint32_t up = (lo < 7u && u * (ghi - glo) < a - glo) ? 1u : 0u;
  return (lo + up) | ((f2u(y) >> 28) & 8u);
}

// Eight scaled values to eight stochastically rounded codes (element 2i in
// the low nibble of byte i).
__device__ __forceinline__ uint32_t pack8_sr(const float y[8], const uint32_t (&r)[8]) {
  uint32_t w = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= e2m1_sr_code(y[k], r[k]) << (4 * k);
  return w;
}

}  // namespace fp4
