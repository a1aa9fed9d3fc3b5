// gemm_mx.hip -- MXFP4 x MXFP4 GEMM on the gfx950 block-scaled FP4 matrix core.
//
// C[m,n] = (sum_k A[m,k] B[n,k]) * tsA * tsB with A, B in E2M1 codes plus one
// E8M0 scale per 32 K values ("Rubin FP4 GEMM deep dive", §3.1: the product is
// multiplied by the two scales; §3.2: global -> shared -> registers -> matrix
// core -> FP32 accumulators -> epilogue).  On gfx950 the E8M0 scales ride in
// the instruction itself (v_mfma_scale_f32_16x16x128_f8f6f4, one scale byte per
// lane per 32-value K chunk), so the FP32 accumulators already hold the scaled
// product and the epilogue only applies the optional tensor scales.
//
// Structure (one 256 x 256 output tile per workgroup of 4 wavefronts):
//   - K advances in steps of 128 values (64 bytes per row).  Per step the
//     workgroup streams A[256 x 64 B] and B[256 x 64 B] straight from global
//     memory into LDS with buffer_load ... lds (no VGRPs), double-buffered so
//     step s+1 is in flight while step s is multiplied.
//   - LDS is fragment-major: 16 rows x 128 K = one 1 KB matrix-core operand,
//     stored in the lane order the instruction consumes (lane 16j + i holds row
//     i, K chunk j), so every ds_read_b128 reads 1 KB contiguously and is free
//     of bank conflicts.
//   - Each wavefront owns a 128 x 128 sub-tile: 8 A and 8 B operands per step,
//     64 MFMAs, 256 FP32 accumulators per lane.
//   - Scales bypass LDS: the tiled scale layout stores, per 16-row tile, one
//     dword per lane covering four K steps, so each wavefront loads its 16
//     scale dwords directly every 512 K values and shifts the byte for the step.
//   - Out-of-range rows and K chunks read as zero through the buffer
//     descriptor's range check (rows) and an out-of-range offset (K tail).
//   - Workgroups are mapped to tiles so that tiles sharing A rows or B columns
//     run on the same XCD (blockIdx.x round-robins over the 8 XCDs) and, within
//     an XCD, in groups of 4 tile-rows for L2 reuse.
#include "fp4_device.h"
#include "fp4_launch.h"

namespace fp4 {

namespace {

constexpr int BM = 256, BN = 256;
constexpr int STEP_BYTES = 64;                // 128 FP4 values per row per step
constexpr int FRAG_BYTES = 1024;              // 16 rows x 64 bytes
constexpr int FRAGS_A = BM / 16, FRAGS_B = BN / 16;
constexpr int STAGE_BYTES = (FRAGS_A + FRAGS_B) * FRAG_BYTES;  // 32 KB
constexpr int GROUP_M = 4;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Issue the direct-to-LDS loads of one K step: this wave's 4 A and 4 B operands.
__device__ __forceinline__ void issue_step(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, uint8_t* stage,
                                           const uint32_t (&voff_a)[4], const uint32_t (&voff_b)[4], uint32_t wave,
                                           uint32_t kbyte, uint32_t kmask_ok) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t f = wave + 4u * t;
    const uint32_t va = kmask_ok ? voff_a[t] + kbyte : 0x80000000u;
    const uint32_t vb = kmask_ok ? voff_b[t] + kbyte : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(stage + f * FRAG_BYTES), 16, va, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(stage + (FRAGS_A + f) * FRAG_BYTES), 16, vb, 0, 0, 0);
  }
}

template <int OUT>
__global__ __launch_bounds__(256, 1) void gemm_mx_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB,
                                                        const float* __restrict__ tsA, const float* __restrict__ tsB,
                                                        void* __restrict__ C, uint32_t M, uint32_t N, uint32_t K,
                                                        uint32_t tilesM, uint32_t tilesN) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE_BYTES];

  // ---- tile mapping: XCD-contiguous chunks, grouped raster inside a chunk
  const uint32_t ntiles = tilesM * tilesN;
  uint32_t t = blockIdx.x;
  if ((ntiles & 7u) == 0u) t = (blockIdx.x & 7u) * (ntiles >> 3) + (blockIdx.x >> 3);
  const uint32_t group = GROUP_M * tilesN;
  const uint32_t g = t / group, first_m = g * GROUP_M;
  const uint32_t gm = (tilesM - first_m) < GROUP_M ? (tilesM - first_m) : GROUP_M;
  const uint32_t tm = first_m + (t % group) % gm;
  const uint32_t tn = (t % group) / gm;
  const uint32_t m0 = tm * BM, n0 = tn * BN;

  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint32_t wm = wave >> 1, wn = wave & 1u;
  const uint32_t ldb = K / 2u;  // bytes per row
  const uint32_t rowsA = (M - m0) < BM ? (M - m0) : BM;
  const uint32_t rowsB = (N - n0) < BN ? (N - n0) : BN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * ldb, rowsA * ldb);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * ldb, rowsB * ldb);

  // Per-lane source offsets of this wave's operands (relative to the tile base).
  uint32_t voff_a[4], voff_b[4];
  const uint32_t li = lane & 15u, lj = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t f = wave + 4u * q;
    voff_a[q] = (16u * f + li) * ldb + 16u * lj;
    voff_b[q] = voff_a[q];
  }

  const uint32_t nsteps = (K + 127u) / 128u;
  const uint32_t KT = (K / 32u + 15u) / 16u;     // scale tiles per row tile
  const uint32_t RTA = (M + 15u) / 16u, RTB = (N + 15u) / 16u;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  uint32_t sa[8], sb[8];
  if (nsteps > 0) issue_step(ra, rb, lds, voff_a, voff_b, wave, 0u, 16u * lj < ldb);

  for (uint32_t s = 0; s < nsteps; ++s) {
    if ((s & 3u) == 0u) {
      const uint32_t kt = s >> 2;
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const uint32_t rta = m0 / 16u + 8u * wm + f, rtb = n0 / 16u + 8u * wn + f;
        sa[f] = rta < RTA ? *reinterpret_cast<const uint32_t*>(sA + ((size_t)rta * KT + kt) * 256u + lane * 4u) : 0u;
        sb[f] = rtb < RTB ? *reinterpret_cast<const uint32_t*>(sB + ((size_t)rtb * KT + kt) * 256u + lane * 4u) : 0u;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (s + 1u < nsteps) {
      const uint32_t kb = (s + 1u) * STEP_BYTES;
      issue_step(ra, rb, lds + ((s + 1u) & 1u) * STAGE_BYTES, voff_a, voff_b, wave, kb, kb + 16u * lj < ldb);
    }
    const uint8_t* st = lds + (s & 1u) * STAGE_BYTES;
    uint4 af[8], bf[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      af[f] = *reinterpret_cast<const uint4*>(st + (8u * wm + f) * FRAG_BYTES + lane * 16u);
      bf[f] = *reinterpret_cast<const uint4*>(st + (FRAGS_A + 8u * wn + f) * FRAG_BYTES + lane * 16u);
    }
    const uint32_t sh = (s & 3u) * 8u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const v4i ai = {(int)af[i].x, (int)af[i].y, (int)af[i].z, (int)af[i].w};
      const v8i a8 = __builtin_shufflevector(ai, ai, 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v4i bj = {(int)bf[j].x, (int)bf[j].y, (int)bf[j].z, (int)bf[j].w};
        const v8i b8 = __builtin_shufflevector(bj, bj, 0, 1, 2, 3, -1, -1, -1, -1);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc[i][j], 4, 4, 0, (int)(sa[i] >> sh), 0,
                                                                      (int)(sb[j] >> sh));
      }
    }
  }

  // ---- epilogue: x tsA * tsB, FP32 or BF16 (round to nearest even)
  const float scale = (tsA ? *tsA : 1.0f) * (tsB ? *tsB : 1.0f);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t col = n0 + 128u * wn + 16u * j + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = m0 + 128u * wm + 16u * i + 4u * lj + r;
        if (row < M && col < N) {
          const float v = acc[i][j][r] * scale;
          if (OUT == 0)
            static_cast<float*>(C)[(size_t)row * N + col] = v;
          else
            static_cast<uint16_t*>(C)[(size_t)row * N + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                          int out_dtype, hipStream_t stream) {
  const uint32_t tilesM = (uint32_t)((M + BM - 1) / BM), tilesN = (uint32_t)((N + BN - 1) / BN);
  const dim3 grid(tilesM * tilesN);
  if (out_dtype == 0)
    gemm_mx_kernel<0><<<grid, dim3(256), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, (uint32_t)M, (uint32_t)N,
                                                      (uint32_t)K, tilesM, tilesN);
  else
    gemm_mx_kernel<1><<<grid, dim3(256), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, (uint32_t)M, (uint32_t)N,
                                                      (uint32_t)K, tilesM, tilesN);
  return hipGetLastError();
}

}  // namespace fp4
