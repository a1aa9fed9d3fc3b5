// gemm_mx.hip -- MXFP4 x MXFP4 GEMM on the gfx950 block-scaled FP4 matrix core.
//
// C[m,n] = (sum_k A[m,k] B[n,k]) * tsA * tsB with A, B in E2M1 codes plus one
// E8M0 scale per 32 K values ("Rubin FP4 GEMM deep dive", §3.1: the product is
// multiplied by the two scales; §3.2: global -> shared -> registers -> matrix
// core -> FP32 accumulators -> epilogue).  On gfx950 the E8M0 scales ride in
// the instruction itself (v_mfma_scale_f32_32x32x64_f8f6f4: one scale byte per
// lane per 32-value K chunk), so the FP32 accumulators already hold the scaled
// product and the epilogue only applies the optional tensor scales.
//
// Structure (one 256 x 256 output tile per workgroup of 8 wavefronts, two per
// SIMD, so one wave's LDS reads and barrier waits overlap the other's MFMAs):
//   - K advances in steps of 128 values (64 bytes per row).  Each step's A and
//     B tiles (256 rows x 64 B each) and the scale dwords they need are
//     streamed from global memory straight into LDS with buffer_load ... lds
//     (no VGPRs), through a ring of 3 stages: step s+2 is in flight while s is
//     multiplied.  Every wave issues the same 6 loads per step, so "stage s has
//     landed" is one s_waitcnt vmcnt(6) plus a barrier.
//   - LDS rows are 64 bytes; the four 16-byte chunks of row r are stored at
//     chunk ^ ((r >> 2) & 3), which makes the matrix-core operand reads
//     (lane = 32 * chunk + row) free of bank conflicts while each direct-to-LDS
//     load still reads whole 64-byte row segments.
//   - Each wavefront owns a 128 x 64 sub-tile: per 64-value K sub-step it reads
//     4 A and 2 B operands (ds_read_b128) and issues 8 MFMAs of 32x32x64; 128
//     FP32 accumulators per lane.  (The 32x32x64 form is the full-rate FP4
//     instruction on gfx950; 16x16x128 runs at half rate.)
//   - The scale layout (32-row x 8-block tiles, lane = 32 * chunk + row) is
//     the operand's lane order, so one dword per lane and 32-row block carries
//     the scales of four K sub-steps, picked by op_sel.
//   - Workgroups are mapped to tiles so that tiles sharing A rows or B columns
//     run on the same XCD (blockIdx.x round-robins over the 8 XCDs) and, within
//     an XCD, in groups of 4 tile-rows for L2 reuse.
#include "fp4_device.h"
#include "fp4_launch.h"

#include <type_traits>

namespace fp4 {

namespace {

constexpr uint32_t BM = 256, BN = 256;
constexpr uint32_t STEP_BYTES = 64;                 // 128 FP4 values per row per step
constexpr uint32_t REGION = 256 * STEP_BYTES;       // 16 KB: one operand's rows of a step
constexpr uint32_t SCALE_REGION = 8 * 256;          // 8 scale tiles (256 rows x 256 K)
constexpr uint32_t STAGE_BYTES = 2 * REGION + 2 * SCALE_REGION;  // 36 KB
constexpr uint32_t NSTAGE = 3;
constexpr uint32_t GROUP_M = 4;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// max(total - off, 0) for uniform values, kept in a scalar register (a
// saturating subtract would otherwise be selected as a vector instruction and
// turn the buffer descriptor into a per-lane value).
__device__ __forceinline__ uint32_t uniform_rem(uint32_t total, uint32_t off) {
  return __builtin_amdgcn_readfirstlane(total > off ? total - off : 0u);
}

// A uniform value the compiler may not strength-reduce into per-step vector
// registers.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return __builtin_amdgcn_readfirstlane(x);
}

template <int OUT>
__global__ __launch_bounds__(512, 1) void gemm_mx_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB,
                                                        const float* __restrict__ tsA, const float* __restrict__ tsB,
                                                        void* __restrict__ C, uint32_t M, uint32_t N, uint32_t K,
                                                        uint32_t tilesM, uint32_t tilesN) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE_BYTES];

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

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const uint32_t wm = wave >> 2, wn = wave & 3u;  // 2 x 4 waves, 128 x 64 each
  const uint32_t ldb = K / 2u;                    // bytes per row
  const uint32_t rowsA = (M - m0) < BM ? (M - m0) : BM;
  const uint32_t rowsB = (N - n0) < BN ? (N - n0) : BN;
  const uint8_t* const a_tile = A + (size_t)m0 * ldb;
  const uint8_t* const b_tile = B + (size_t)n0 * ldb;
  const uint32_t a_bytes = rowsA * ldb, b_bytes = rowsB * ldb;
  const uint32_t KT = (K / 32u + 7u) / 8u;        // 256-value scale tiles per row
  const uint32_t RTA = (M + 31u) / 32u, RTB = (N + 31u) / 32u;
  const uint32_t srow = KT * 256u;                // bytes between 32-row scale tiles
  const uint8_t* const sa_tile = sA + (size_t)(m0 / 32u) * srow;
  const uint8_t* const sb_tile = sB + (size_t)(n0 / 32u) * srow;
  const uint32_t sa_bytes = (RTA > m0 / 32u ? RTA - m0 / 32u : 0u) * srow;
  const uint32_t sb_bytes = (RTB > n0 / 32u ? RTB - n0 / 32u : 0u) * srow;

  // ---- direct-to-LDS load plan (per step, per wave: 2 A + 2 B row groups of
  // 16 rows x 64 B, and one A and one B scale tile of 64 dwords).
  // Lane L of a row-group load fills LDS bytes 16L..16L+15 = row L/4, stored
  // chunk L%4, i.e. global chunk (L%4) ^ ((row >> 2) & 3).
  const uint32_t grow = lane >> 2;
  const uint32_t gchunk = (lane & 3u) ^ ((lane >> 4) & 3u);
  const uint32_t voff0 = (16u * wave + grow) * ldb + 16u * gchunk;
  const uint32_t voff1 = (16u * (wave + 8u) + grow) * ldb + 16u * gchunk;
  const uint32_t svoff = (wave * KT) * 256u + lane * 4u;  // scale tile `wave` of the 8

  auto dma = [&](uint32_t step) {
    const uint32_t kb = opaque(step * STEP_BYTES);
    const uint32_t ko = opaque((step >> 1) * 256u);
    uint8_t* st = lds + (step % NSTAGE) * STAGE_BYTES;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_tile + kb, uniform_rem(a_bytes, kb));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_tile + kb, uniform_rem(b_bytes, kb));
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa_tile + ko, uniform_rem(sa_bytes, ko));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sb_tile + ko, uniform_rem(sb_bytes, ko));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + 1024u * wave), 16, voff0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + 1024u * (wave + 8u)), 16, voff1, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + REGION + 1024u * wave), 16, voff0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + REGION + 1024u * (wave + 8u)), 16, voff1, 0, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + 2u * REGION + 256u * wave), 4, svoff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + 2u * REGION + SCALE_REGION + 256u * wave), 4,
                                             svoff, 0, 0, 0);
  };

  // ---- operand read offsets: lane (j = chunk, i = row) of a 32-row block
  const uint32_t li = lane & 31u, lj = lane >> 5;
  const uint32_t rd0 = 64u * li + 16u * ((0u + lj) ^ ((li >> 2) & 3u));  // sub-step 0 (chunks 0,1)
  const uint32_t rd1 = 64u * li + 16u * ((2u + lj) ^ ((li >> 2) & 3u));  // sub-step 1 (chunks 2,3)
  const uint32_t a_rows = 64u * (128u * wm);   // byte offset of this wave's first A row
  const uint32_t b_rows = 64u * (64u * wn);

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // One K step: wait for its stage, barrier (all waves' loads landed, and all
  // waves are done with the stage the next load overwrites), issue the load of
  // step s+2, then read this wave's operands and scales and run 16 MFMAs.
  // U selects the scale byte pair (two steps per 256-value scale tile).
  auto step = [&](auto U, uint32_t s) {
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __syncthreads();
    dma(s + 2u);
    const uint8_t* st = lds + (s % NSTAGE) * STAGE_BYTES;
    v4i a0[4], a1[4], b0[2], b1[2];
#pragma unroll
    for (int r = 0; r < 4; ++r) a0[r] = *reinterpret_cast<const v4i*>(st + a_rows + 2048u * r + rd0);
#pragma unroll
    for (int c = 0; c < 2; ++c) b0[c] = *reinterpret_cast<const v4i*>(st + REGION + b_rows + 2048u * c + rd0);
#pragma unroll
    for (int r = 0; r < 4; ++r) a1[r] = *reinterpret_cast<const v4i*>(st + a_rows + 2048u * r + rd1);
#pragma unroll
    for (int c = 0; c < 2; ++c) b1[c] = *reinterpret_cast<const v4i*>(st + REGION + b_rows + 2048u * c + rd1);
    uint32_t sa[4], sb[2];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sa[r] = *reinterpret_cast<const uint32_t*>(st + 2u * REGION + 256u * (4u * wm + r) + 4u * lane);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      sb[c] = *reinterpret_cast<const uint32_t*>(st + 2u * REGION + SCALE_REGION + 256u * (2u * wn + c) + 4u * lane);
    constexpr int u = decltype(U)::value;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v8i a8 = __builtin_shufflevector(a0[r], a0[r], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const v8i b8 = __builtin_shufflevector(b0[c], b0[c], 0, 1, 2, 3, -1, -1, -1, -1);
        acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[r][c], 4, 4, 2 * u, (int)sa[r],
                                                                     2 * u, (int)sb[c]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v8i a8 = __builtin_shufflevector(a1[r], a1[r], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const v8i b8 = __builtin_shufflevector(b1[c], b1[c], 0, 1, 2, 3, -1, -1, -1, -1);
        acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[r][c], 4, 4, 2 * u + 1,
                                                                     (int)sa[r], 2 * u + 1, (int)sb[c]);
      }
    }
  };

  // Two steps per 256-value scale tile.  A last, partial tile runs its second
  // step over codes past K; their scales are the tile's padding bytes (0, i.e.
  // 2^-127 on both operands), so those products (<= 36 * 2^-254) are zero in
  // FP32 and add nothing.
  if (KT > 0) {
    dma(0);
    dma(1);
    for (uint32_t kt = 0; kt < KT; ++kt) {
      step(std::integral_constant<int, 0>{}, 2u * kt);
      step(std::integral_constant<int, 1>{}, 2u * kt + 1u);
    }
  }

  // ---- epilogue: x tsA * tsB, FP32 or BF16 (round to nearest even).  Lane L
  // of a 32x32 block holds column L%32, rows 8*(i/4) + 4*(L/32) + i%4.
  const float scale = (tsA ? *tsA : 1.0f) * (tsB ? *tsB : 1.0f);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t col = n0 + 64u * wn + 32u * c + li;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t row = m0 + 128u * wm + 32u * r + 8u * (i >> 2) + 4u * lj + (i & 3);
        if (row < M && col < N) {
          const float v = acc[r][c][i] * scale;
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
    gemm_mx_kernel<0><<<grid, dim3(512), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, (uint32_t)M, (uint32_t)N,
                                                      (uint32_t)K, tilesM, tilesN);
  else
    gemm_mx_kernel<1><<<grid, dim3(512), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, (uint32_t)M, (uint32_t)N,
                                                      (uint32_t)K, tilesM, tilesN);
  return hipGetLastError();
}

}  // namespace fp4
