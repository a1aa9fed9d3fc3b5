// gemv_nv_dot.hip -- NVFP4 decode GEMV for one activation row (gfx950), on
// the vector ALU with exact block sums.
//
//   C[n] = tsA tsW sum_b sW[n,b] (sA[b] sum_{k in b} e2m1(A[k]) e2m1(W[n,k]))
//
// (NVFP4 video transcript: 16-value blocks, E4M3 block scale, one FP32 tensor
// scale; "Rubin FP4 GEMM deep dive" §1.2, §6.2: a decode step streams every
// weight once, so the kernel is shaped around that stream.)
//
// Why this kernel.  At one activation row the matrix core has nothing to
// amortise: what bounds the step is how fast the weights come out of HBM.
// The matrix-core GEMV gives each lane one weight row (the operand layout), so
// a load instruction touches 32 rows x 32 bytes; here a load instruction
// reads 1 KB of one weight row, whole 128-byte lines, and a workgroup of 4
// wavefronts reads 16 rows (64 KB at K = 8192): at 8192 x 8192, 512
// workgroups, two per compute unit.  Measured one-shot 32 MiB reads (weights
// rotated past the Infinity Cache): lane-per-row loads 8.5 us, 1 KB row
// pieces from 1024-thread workgroups 7.6 us, from 256-thread workgroups
// 6.9 us.  At two or more activation rows the vector work per weight grows
// with the row count and the matrix-core kernels win (measured at M = 2:
// 14.5 vs 12.5 us fused), so this kernel serves M = 1 only.
//
// Work split.  Thread t owns the 16-byte chunk t (32 values, blocks 2t and
// 2t + 1) of every one of the workgroup's 16 rows and the same chunk of the
// activation, which it decodes once into registers.  Per weight row it
// converts the 32 codes to FP16 E2M1 values (exact) and forms each block's
// dot product with the activation's FP16 values e2m1(A) * sA (exact: E2M1 x
// E4M3 needs at most 6 significant bits and lies in [2^-10, 2688]) by packed
// FP16 dot products accumulated in FP32, in two chains of four per block:
// every partial sum is a multiple of sA / 4 below 576 sA, so the block sum
// sA * sum e2m1 e2m1 comes out exact.  The two block sums times sW[n,b] are
// added with one rounding each.  The weight scale bytes are read as whole
// 16-byte pieces of the tiled layout (two runs of 8 bytes per row and tile)
// and handed to the threads through LDS: two-byte loads per thread and row
// cost 2.2 us of the 9 us step.  The 256 threads' sums of each row are then
// added in a fixed order (LDS, then rotations inside 16-lane rows): the result
// is deterministic, and the pre-quantised and the fused call stage the same
// FP16 values, so the two return the same bits.
//
// Load order.  A wave issues in order and stalls once the memory pipeline is
// full, so whatever follows the weight requests in program order starts only
// after the whole stream has been handed out.  Hence: the activation, the
// scale pieces and the first rows' codes; the activation staged; then the
// rest of the codes.
//
// Fused call: X (FP32 or BF16) arrives unquantised.  Every workgroup takes
// the tensor maximum over the whole of X (its threads' chunks cover it) and
// quantises its chunks exactly as fp4_quantize does (same scale byte, same
// codes: nv_div's arithmetic, its branch taken once per block).
#include <float.h>

#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));

constexpr uint32_t DG_THREADS = 256;   // 4 wavefronts
constexpr uint32_t DG_MAX_K = 8192;    // one 16-byte chunk per thread and row
// Weight rows whose codes are requested before the activation is staged
// (8192 x 8192, X quantised in the kernel: 2 rows 9.57 us, 4 rows 9.52 us,
// 6 rows 9.81 us, all 16 rows 11.6 us).
constexpr uint32_t DG_HEAD = 4;

// Four FP16 pairs: the E2M1 values of the eight codes of w (low nibble first).
__device__ __forceinline__ void e2m1_pairs(uint32_t w, v2h (&p)[4]) {
  p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
}

template <int MB, int RB, bool FUSED, int OUT, int XDT>
__global__ __launch_bounds__(DG_THREADS, 2) void gemv_dot_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ sW, const float* __restrict__ tsA, const float* __restrict__ tsW, void* __restrict__ C,
    uint32_t M, uint32_t N, uint32_t K, const void* __restrict__ X, float* __restrict__ ts_out, uint32_t flags) {
  constexpr uint32_t RB_ = (uint32_t)RB;
  static_assert(RB * MB == 16, "16 (row, activation row) sums per workgroup");
  constexpr uint32_t PSTRIDE = DG_THREADS + 16u;   // floats; rows 16 banks apart
  __shared__ float psum[RB * MB * PSTRIDE];
  // the workgroup's weight scale bytes: per 256-value tile, RB rows x 8 bytes
  // of each chunk parity (the two runs the rows occupy in the tiled layout)
  __shared__ __attribute__((aligned(16))) uint8_t wsl[(DG_MAX_K / 256u) * RB * 16u];
  __shared__ float wmax[4];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ldb = K / 2u;                 // bytes per row (K % 32 == 0)
  const uint32_t cpr = K / 32u;                // 16-byte chunks per row (<= 256)
  const uint32_t KT = (K + 255u) / 256u;       // scale tiles per 32-row tile row
  const uint32_t srow = KT * 512u;
  const uint32_t n0 = blockIdx.x * RB;
  const bool own = tid < cpr;                  // chunk tid exists
  const uint32_t c8 = tid & 7u;
  // Offset of chunk tid's two scale bytes for row i (0..31) of a 32-row tile row.
  auto soff = [&](uint32_t i) { return (tid >> 3) * 512u + (32u * (c8 & 1u) + i) * 8u + 2u * (c8 >> 1); };

  // ---- activation loads first
  constexpr uint32_t XEB = XDT == kDtBF16 ? 2u : 4u;
  constexpr int XL = FUSED ? (int)(32u * XEB / 16u) : 1;   // 16-byte loads per chunk
  v4i xl[MB][XL];
  uint32_t asb[MB];
  if (FUSED) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, M * K * XEB);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int l = 0; l < XL; ++l)
        xl[m][l] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(
                     rx, own && (uint32_t)m < M ? ((uint32_t)m * K + 32u * tid) * XEB + 16u * (uint32_t)l : 0x80000000u,
                     0, 0));
  } else {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, M * ldb);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sA, srow);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const bool ok = own && (uint32_t)m < M;
      xl[m][0] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? (uint32_t)m * ldb + 16u * tid : 0x80000000u, 0, 0));
      asb[m] = __builtin_amdgcn_raw_buffer_load_b16(rsa, ok ? soff((uint32_t)m) : 0x80000000u, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- every weight load of the workgroup: scale pairs, then codes (row
  // n0 + r; rows past N read out of range: zeros)
  const uint32_t rows = __builtin_amdgcn_readfirstlane(N - n0 < RB ? N - n0 : RB);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * ldb, rows * ldb);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(sW + (size_t)(n0 >> 5) * srow, srow);
  const uint32_t i0 = n0 & 31u;   // first row inside its 32-row scale tile
  // Scale bytes in 16-byte pieces q < KT * RB: tile q / RB, parity
  // j = (q % RB) / (RB / 2), piece u = q % (RB / 2) of the run of lanes
  // 32 j + i0 .. 32 j + i0 + RB - 1 (8 bytes each).
  constexpr uint32_t SP = (DG_MAX_K / 256u) * RB / DG_THREADS;   // pieces per thread (at most)
  v4i wsp[SP];
  const uint32_t npieces = KT * RB_;
  v4i wc[RB];
  auto load_scales = [&]() {
#pragma unroll
    for (uint32_t i = 0; i < SP; ++i) {
      const uint32_t q = tid + DG_THREADS * i, T = q / RB_, rem = q % RB_;
      const uint32_t off = T * 512u + (32u * (rem / (RB_ / 2u)) + i0) * 8u + 16u * (rem % (RB_ / 2u));
      wsp[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rsw, q < npieces ? off : 0x80000000u, 0, 0));
    }
  };
  auto load_codes = [&](uint32_t lo, uint32_t hi) {
#pragma unroll
    for (uint32_t r = lo; r < hi; ++r)
      wc[r] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, own ? r * ldb + 16u * tid : 0x80000000u, 0, 0));
  };
  // The scale pieces and the first DG_HEAD rows' codes; then wait for the
  // activation.  The rest of the stream is requested only once the
  // activation is staged: a wave issues in order and stalls on a full load
  // queue, so with every load requested first the activation's staging (the
  // fused quantisation: a few hundred vector instructions) would start only
  // after the whole stream had been handed out.
  load_scales();
  load_codes(0u, DG_HEAD);
#pragma unroll
  for (int m = 0; m < MB; ++m) {
#pragma unroll
    for (int l = 0; l < XL; ++l) asm volatile("" : : "v"(xl[m][l]));
    if (!FUSED) asm volatile("" : : "v"(asb[m]));
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- the activation chunk as FP16 pairs e2m1(A) * sA: act[m][4d + j] is
  // values 8d + 2j, 8d + 2j + 1 (d = dword of the 16 code bytes)
  v2h act[MB][16];
  float s_x = 1.0f;
  if (!FUSED) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const v2h s = scale_pair((asb[m] >> (8 * (d >> 1))) & 0xFFu);
        v2h p[4];
        e2m1_pairs((uint32_t)xl[m][0][d], p);
#pragma unroll
        for (int j = 0; j < 4; ++j) act[m][4 * d + j] = p[j] * s;
      }
    }
    s_x = *tsA;
  } else {
    // The chunk's values (unpacked once), block maxima (two blocks per row
    // chunk), then the tensor maximum.
    float xv[MB][32];
    float am[MB][2];
    float tmax = 0.0f;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        if (XDT == kDtBF16) {
          const uint32_t w = (uint32_t)xl[m][q >> 3][(q >> 1) & 3];
          xv[m][q] = (q & 1) ? u2f(w & 0xFFFF0000u) : u2f(w << 16);
        } else {
          xv[m][q] = u2f((uint32_t)xl[m][q >> 2][q & 3]);
        }
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(xv[m][16 * b + e]));
        am[m][b] = a;
        tmax = fmaxf(tmax, a);
      }
    }
    if (flags & 1u) {
      s_x = *tsA;
    } else {
      tmax = wave_fmax(tmax);
      if (lane == 0) wmax[wave] = tmax;
      __syncthreads();
      const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
      // Tensor scale: amax / (6 * 448), 1 for an all-zero X, at least FLT_MIN.
      if (amax > 0.0f) {
        s_x = amax / 2688.0f;
        if (s_x < FLT_MIN) s_x = FLT_MIN;
      }
      if (blockIdx.x == 0 && tid == 0 && ts_out) *ts_out = s_x;
    }
    // Quantise each block as the quantiser does (E4M3 scale byte of
    // (amax_b / 6) / s_x, codes of x / (e4m3(sb) s_x)), then decode.
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float y[16];
        const uint32_t sb = e4m3_encode((am[m][b] / 6.0f) / s_x);
#pragma unroll
        for (int e = 0; e < 16; ++e) y[e] = xv[m][16 * b + e];
        if (sb == 0u) {
#pragma unroll
          for (int e = 0; e < 16; ++e) y[e] = __builtin_copysignf(0.0f, y[e]);   // x / inf
        } else {
          const float dd = e4m3_value(sb) * s_x;
          const float rd = 1.0f / dd;
          // nv_div with its branch taken once per block
          if (dd >= kNvDivFastMin) {
#pragma unroll
            for (int e = 0; e < 16; ++e) y[e] = nv_div_fast(y[e], dd, rd);
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) y[e] = __builtin_copysignf(__builtin_fabsf(y[e]) / dd, y[e]);
          }
        }
        const v2h s = scale_pair(sb);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t code = pack8(y + 8 * h);
          v2h p[4];
          e2m1_pairs(code, p);
#pragma unroll
          for (int j = 0; j < 4; ++j) act[m][8 * b + 4 * h + j] = p[j] * s;
        }
      }
    // Rows past M and chunks past K are zero (their loads read zeros, but a
    // zero block's pairs are zero anyway; keep them exactly +0).
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (!(own && (uint32_t)m < M))
#pragma unroll
        for (int j = 0; j < 16; ++j) act[m][j] = v2h{};
  }
  // the rest of the weight stream, once the activation is staged
  __builtin_amdgcn_sched_barrier(0);
  load_codes(DG_HEAD, RB);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (uint32_t i = 0; i < SP; ++i) {
    const uint32_t q = tid + DG_THREADS * i;
    if (q < npieces) *reinterpret_cast<v4i*>(wsl + 16u * q) = wsp[i];
  }
  __syncthreads();
  // this thread's scale pair of row r: tile t / 8, parity j, pair s of the lane's 8 bytes
  const uint32_t sl0 = (tid >> 3) * 16u * RB_ + (c8 & 1u) * 8u * RB_ + 2u * (c8 >> 1);
  // ---- per weight row: exact block sums, times sW, two roundings per row
  float part[RB][MB];
#pragma unroll
  for (uint32_t r = 0; r < RB; ++r) {
    const uint32_t wsr = own ? (uint32_t)*reinterpret_cast<const uint16_t*>(wsl + sl0 + 8u * r) : 0u;
    const v2f sw = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wsr, 1.0f, false);
    v2h wp[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v2h p[4];
      e2m1_pairs((uint32_t)wc[r][d], p);
#pragma unroll
      for (int j = 0; j < 4; ++j) wp[4 * d + j] = p[j];
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      // four independent chains of four; a block's two partial sums and
      // their sum are exact (multiples of sA / 4 below 576 sA)
      float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) t[c] = __builtin_amdgcn_fdot2(wp[4 * c + j], act[m][4 * c + j], t[c], false);
      part[r][m] = __builtin_fmaf(t[2] + t[3], sw[1], (t[0] + t[1]) * sw[0]);
    }
  }

  // ---- row sums: every thread's RB x MB partial sums through LDS, each sum
  // of 256 added by 16 threads (16 values each, in thread order), then
  // across those 16 lanes by rotations inside a 16-lane row (DPP); lane 0 of
  // the row stores.  A fixed order: deterministic.
#pragma unroll
  for (uint32_t r = 0; r < RB_; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) psum[(r * MB + (uint32_t)m) * PSTRIDE + tid] = part[r][m];
  __syncthreads();
  {
    const uint32_t pr = tid >> 4, l = tid & 15u;   // pair (row, m) = pr, 16 pairs
    float v = 0.0f;
#pragma unroll
    for (uint32_t k = 0; k < 16u; ++k) v += psum[pr * PSTRIDE + l + 16u * k];
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    const uint32_t r = pr / MB, m = pr % MB, col = n0 + r;
    if (l == 0u && m < M && col < N) {
      v *= s_x * *tsW;
      if (OUT == 0)
        static_cast<float*>(C)[(size_t)m * N + col] = v;
      else
        static_cast<uint16_t*>(C)[(size_t)m * N + col] = f32_to_bf16(v);
    }
  }
}

template <int MB>
hipError_t dg_launch(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                     const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype, bool fused,
                     const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, hipStream_t stream) {
  constexpr int RB = 16 / MB;
  const dim3 grid((uint32_t)((N + RB - 1) / RB)), block(DG_THREADS);
  const uint32_t m = (uint32_t)M, n = (uint32_t)N, k = (uint32_t)K;
  if (!fused) {
    if (out_dtype == 0)
      gemv_dot_kernel<MB, RB, false, 0, kDtBF16><<<grid, block, 0, stream>>>(A, sA, B, sB, tsA, tsB, C, m, n, k, nullptr,
                                                                        nullptr, 0u);
    else
      gemv_dot_kernel<MB, RB, false, 1, kDtBF16><<<grid, block, 0, stream>>>(A, sA, B, sB, tsA, tsB, C, m, n, k, nullptr,
                                                                        nullptr, 0u);
    return hipGetLastError();
  }
  const float* ts_in = x_tensor_scale;
  float* ts_o = (flags & 1u) ? nullptr : x_tensor_scale;
#define DG_FUSED(OUTT, XT)                                                                                        \
  gemv_dot_kernel<MB, RB, true, OUTT, XT><<<grid, block, 0, stream>>>(nullptr, nullptr, B, sB, ts_in, tsB, C, m, n, k, X, \
                                                                 ts_o, flags)
  if (x_dtype == kDtBF16) {
    if (out_dtype == 0) DG_FUSED(0, kDtBF16);
    else DG_FUSED(1, kDtBF16);
  } else {
    if (out_dtype == 0) DG_FUSED(0, kDtF32);
    else DG_FUSED(1, kDtF32);
  }
#undef DG_FUSED
  return hipGetLastError();
}

}  // namespace

bool gemv_dot_applies(int64_t M, int64_t N, int64_t K) {
  return M == 1 && N >= 1 && K >= 0 && K <= (int64_t)DG_MAX_K && K % 32 == 0 && (N + 15) / 16 <= 0x7FFFFFFF;
}

hipError_t launch_gemv_dot(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                           const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                           hipStream_t stream) {
  return dg_launch<1>(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, false, nullptr, kDtBF16, nullptr, 0u, stream);
}

hipError_t launch_gemv_dot_fused(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* B,
                                 const uint8_t* sB, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                                 int out_dtype, hipStream_t stream) {
  return dg_launch<1>(nullptr, nullptr, B, sB, nullptr, tsB, C, M, N, K, out_dtype, true, X, x_dtype, x_tensor_scale,
                      flags, stream);
}

}  // namespace fp4
