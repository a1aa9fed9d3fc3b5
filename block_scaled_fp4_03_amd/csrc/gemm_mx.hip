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
//     (no VGPRs), through a ring of 4 stages: while step s is multiplied, the
//     operands of s+1 are read from LDS into a second register set and the
//     loads of s+2 and s+3 are in flight.  Every wave issues the same 6 loads
//     per step, so "stage s+1 has landed" is one s_waitcnt vmcnt(6) plus a
//     barrier.
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
#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

constexpr uint32_t BM = 256, BN = 256;
constexpr uint32_t STEP_BYTES = 128;                // 256 FP4 values per row per stage
constexpr uint32_t REGION = 256 * STEP_BYTES;       // 32 KB: one operand's rows of a stage
constexpr uint32_t SCALE_REGION = 8 * 256;          // 8 scale tiles (256 rows x 256 K)
constexpr uint32_t STAGE_BYTES = 2 * REGION + 2 * SCALE_REGION;  // 68 KB
constexpr uint32_t NSTAGE = 2;
constexpr uint32_t GROUP_M = 4;

// Operands of one 64-value K sub-step of a wave's 128 x 64 sub-tile.
struct Ops {
  v4i a[4], b[2];
};

// 8 MFMAs of one sub-step; OPSEL picks the sub-step's byte of each scale dword.
template <int OPSEL>
__device__ __forceinline__ void mma_sub(v16f (&acc)[4][2], const Ops& o, const uint32_t (&sa)[4],
                                        const uint32_t (&sb)[2]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const v8i a8 = __builtin_shufflevector(o.a[r], o.a[r], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const v8i b8 = __builtin_shufflevector(o.b[c], o.b[c], 0, 1, 2, 3, -1, -1, -1, -1);
      acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[r][c], 4, 4, OPSEL, (int)sa[r], OPSEL,
                                                                   (int)sb[c]);
    }
  }
}

// One LDS read of the next sub-step's operands after each MFMA.
__device__ __forceinline__ void interleave_mfma_reads() {
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

template <int OUT>
__global__ __launch_bounds__(512, 1) void gemm_mx_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB,
                                                        const float* __restrict__ tsA, const float* __restrict__ tsB,
                                                        void* __restrict__ C, uint32_t M, uint32_t N, uint32_t K,
                                                        uint32_t tilesM, uint32_t tilesN) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE_BYTES];

  uint32_t tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, GROUP_M, tm, tn);
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
  const uint32_t KT = (K / 32u + 7u) / 8u;        // 256-value stages (= scale tiles) per row
  const uint32_t RTA = (M + 31u) / 32u, RTB = (N + 31u) / 32u;
  const uint32_t srow = KT * 256u;                // bytes between 32-row scale tiles
  const uint8_t* const sa_tile = sA + (size_t)(m0 / 32u) * srow;
  const uint8_t* const sb_tile = sB + (size_t)(n0 / 32u) * srow;
  const uint32_t sa_bytes = (RTA > m0 / 32u ? RTA - m0 / 32u : 0u) * srow;
  const uint32_t sb_bytes = (RTB > n0 / 32u ? RTB - n0 / 32u : 0u) * srow;

  // ---- direct-to-LDS load plan.  A stage holds 256 rows x 128 B of A and of
  // B; LDS row r keeps its eight 16-byte chunks c at position c ^ ((r>>1)&7).
  // One load (1 KB) fills 8 rows; wave w loads row groups w, w+8, w+16, w+24
  // of A and of B, plus scale tile w of A and of B (64 dwords each).  Lane L
  // fills row L/8, position L%8, i.e. it fetches global chunk
  // (L%8) ^ ((row >> 1) & 7); the rows' swizzle term is 4*(w&1) + L/16.
  const uint32_t gchunk = (lane & 7u) ^ ((4u * (wave & 1u) + (lane >> 4)) & 7u);
  uint32_t voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = (8u * (wave + 8u * q) + (lane >> 3)) * ldb + 16u * gchunk;
  const uint32_t svoff = (wave * KT) * 256u + lane * 4u;

  auto dma = [&](uint32_t stage_k) {
    const uint32_t kb = opaque(stage_k * STEP_BYTES);
    const uint32_t ko = opaque(stage_k * 256u);
    uint8_t* st = lds + (stage_k % NSTAGE) * STAGE_BYTES;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_tile + kb, uniform_rem(a_bytes, kb));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_tile + kb, uniform_rem(b_bytes, kb));
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa_tile + ko, uniform_rem(sa_bytes, ko));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sb_tile + ko, uniform_rem(sb_bytes, ko));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + 1024u * (wave + 8u * q)), 16, voff[q], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + REGION + 1024u * (wave + 8u * q)), 16, voff[q], 0,
                                               0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + 2u * REGION + 256u * wave), 4, svoff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + 2u * REGION + SCALE_REGION + 256u * wave), 4,
                                             svoff, 0, 0, 0);
  };

  // ---- operand reads: lane (j = L/32, i = L%32) of a 32-row block reads row
  // i, chunk 2q + j of sub-step q, stored at position (2q + j) ^ ((i>>1)&7).
  const uint32_t li = lane & 31u, lj = lane >> 5;
  uint32_t rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rd[q] = 128u * li + 16u * ((2u * q + lj) ^ ((li >> 1) & 7u));
  const uint32_t a_rows = 128u * (128u * wm);   // byte offset of this wave's first A row
  const uint32_t b_rows = 128u * (64u * wn);

  auto read_ops = [&](uint32_t stage_k, int q, Ops& o) {
    const uint8_t* st = lds + (stage_k % NSTAGE) * STAGE_BYTES;
#pragma unroll
    for (int r = 0; r < 4; ++r) o.a[r] = *reinterpret_cast<const v4i*>(st + a_rows + 4096u * r + rd[q]);
#pragma unroll
    for (int c = 0; c < 2; ++c) o.b[c] = *reinterpret_cast<const v4i*>(st + REGION + b_rows + 4096u * c + rd[q]);
  };
  auto read_scales = [&](uint32_t stage_k, uint32_t (&sa)[4], uint32_t (&sb)[2]) {
    const uint8_t* st = lds + (stage_k % NSTAGE) * STAGE_BYTES + 2u * REGION;
#pragma unroll
    for (int r = 0; r < 4; ++r) sa[r] = *reinterpret_cast<const uint32_t*>(st + 256u * (4u * wm + r) + 4u * lane);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      sb[c] = *reinterpret_cast<const uint32_t*>(st + SCALE_REGION + 256u * (2u * wn + c) + 4u * lane);
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // Stage k covers K values [256k, 256k + 256) in four 64-value sub-steps.
  // Per stage: sub-steps 0-2 each run 8 MFMAs while the next sub-step's
  // operands are read from LDS; then wait for this wave's loads of stage k+1,
  // barrier (all of stage k+1 has landed; every wave is done reading stage k),
  // launch the loads of stage k+2 into stage k's buffer, read sub-step 0 of
  // k+1 and its scales, and run sub-step 3.  A last, partial stage runs over
  // codes past K; their scales are the tile's padding bytes (0, i.e. 2^-127 on
  // both operands), so those products (<= 36 * 2^-254) are zero in FP32.
  if (KT > 0) {
    Ops o0, o1;
    uint32_t sa[4], sb[2], sa_n[4], sb_n[2];
    dma(0);
    dma(1);
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_ops(0, 0, o0);
    read_scales(0, sa, sb);
    for (uint32_t k = 0; k < KT; ++k) {
      read_ops(k, 1, o1);
      mma_sub<0>(acc, o0, sa, sb);
      interleave_mfma_reads();
      read_ops(k, 2, o0);
      mma_sub<1>(acc, o1, sa, sb);
      interleave_mfma_reads();
      read_ops(k, 3, o1);
      mma_sub<2>(acc, o0, sa, sb);
      interleave_mfma_reads();
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      dma(k + 2u);
      read_ops(k + 1u, 0, o0);
      read_scales(k + 1u, sa_n, sb_n);
      mma_sub<3>(acc, o1, sa, sb);
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sa[r] = sa_n[r];
#pragma unroll
      for (int c = 0; c < 2; ++c) sb[c] = sb_n[c];
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
