// gemm_w4a8.hip -- mixed-format block-scaled GEMM for gfx950: MXFP8 (E4M3)
// activations times MXFP4 (E2M1) weights, FP32 accumulation.
//
// C[m,n] = sum_k A^[m,k] B^[n,k] (+ bias[n], ReLU), A^ the E4M3 codes of A
// times their 32-block E8M0 scales, B^ the E2M1 codes of B times theirs
// ("Rubin FP4 GEMM deep dive", §3.4: weights and activations may differ in
// precision, e.g. FP8 activations with FP4 weights; §3.1: MX block scales;
// §3.2 and §4.2: FP32 accumulators, scale, bias and activation in the
// epilogue).
//
// Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4 with A as FP8 (cbsz 0) and
// B as FP4 (blgp 4).  It issues at the FP8 rate (64 cycles, half the FP4
// rate).
// Exactness: the instruction sums each 16-value K group's products in a
// fixed-point window anchored at the group's largest E4M3 exponent plus its
// largest E2M1 exponent (zero and subnormal codes counted at the lowest
// normal exponent) and truncates each product to a multiple of 2^(anchor -
// 13) (measured on the device).  A product a * b has its lowest bit at
// 2^(e_a - 3 + e_b' - 1) (E4M3 keeps 3 fraction bits, E2M1 one; e_b' =
// max(e_b, 0)), so it is exact when (E_A - e_a) + (E_B - e_b') <= 9; with
// e_b' in 0..2 that holds whenever the A element is within 7 binades of its
// group's largest.  Each step therefore runs twice: once on the A bytes
// whose exponent field is >= 8 (|a| >= 2 before the block scale: exponents
// 1..8) and once on the others (exponents -6..0, subnormals at -6).  Within
// either part every nonzero element is within 7 binades of the part's
// largest, so every product is exact and the accumulator receives the exact
// group sums: C is the FP32-accumulated exact product, within 1e-5 *
// sum |a * b| of the FP64 reference.  Both parts are plain E4M3 bytes under
// the block's own scale, so the E8M0 scales still ride in the instruction.
// The price is two FP8 instructions per step (the exact W4A8 product runs
// at half the FP8 rate).
// Per lane of a 32-row block (row i = lane % 32, half j = lane / 32)
// and 64-value K step:
//   A (FP8): bytes 0-15 hold K [16j, 16j + 16), bytes 16-31 hold
//            K [32 + 16j, 32 + 16j + 16);
//   B (FP4): the 32 nibbles hold K [32j, 32j + 32);
//   scales:  the lane's E8M0 byte scales K block j, [32j, 32j + 32), of its
//            row, for either operand (whichever lanes hold the block's data).
//
// Data path: one 256 x 256 output tile per workgroup of 8 wavefronts (2 per
// SIMD, 64 x 128 each, 8 accumulator blocks per lane).  K advances in stages
// of 128 values, three stages in flight in LDS (52 KB each): A 256 rows x
// 128 B, B 256 rows x 64 B, and the 32-row scale tiles of both operands,
// copied from global memory straight into LDS with buffer_load ... lds.
//   A row r keeps its eight 16-byte chunks c at position c ^ ((r >> 1) & 7).
//   B rows 2l and 2l + 1 share 128-byte line l: chunk c (of 4) of row 2l + h
//   sits at position (4h + c) ^ (l & 3).
// In both, every 16-lane group of an operand read (ds_read_b128) touches 8
// distinct 16-byte positions twice, which the LDS serves without conflicts,
// while each copy instruction still fills 8 whole 128-byte lines.  The
// epilogue stages the tile through LDS so that C is written with 16-byte
// row-contiguous stores.
#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

constexpr uint32_t WBM = 256, WBN = 256;
constexpr uint32_t WSTAGE_K = 128;                  // K values per stage
constexpr uint32_t A_ROW = WSTAGE_K;                // FP8: 128 B per row per stage
constexpr uint32_t B_ROW = WSTAGE_K / 2;            // FP4: 64 B per row per stage
constexpr uint32_t A_REGION = WBM * A_ROW;          // 32 KB
constexpr uint32_t B_REGION = WBN * B_ROW;          // 16 KB
constexpr uint32_t S_REGION = 8u * 256u;            // 8 scale tiles of 32 rows x 256 K
constexpr uint32_t W_STAGE_BYTES = A_REGION + B_REGION + 2u * S_REGION;
constexpr uint32_t W_NSTAGE = 3;
constexpr uint32_t W_GROUP_M = 4;

// Operands of one 64-value K step of a wave's 64 x 128 sub-tile.  a holds
// the A bytes as read from LDS; after split_w, a keeps the bytes with
// exponent field >= 8 and alo the others (zeros in the other's places).
struct OpsW {
  v8i a[2], alo[2];
  v4i b[4];
};

// Split every E4M3 byte of A by bit 6, the top bit of its exponent field:
// v_perm with selector byte 12 gives 0x00, 13 gives 0xFF, so the mask byte
// is 0xFF exactly where bit 6 is set.
__device__ __forceinline__ void split_w(OpsW& o) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t d = (uint32_t)o.a[r][k];
      const uint32_t sel = ((d >> 6) & 0x01010101u) | 0x0C0C0C0Cu;
      const uint32_t hi = d & __builtin_amdgcn_perm(0u, 0u, sel);
      o.a[r][k] = (int)hi;
      o.alo[r][k] = (int)(d ^ hi);
    }
}

// The 8 MFMAs of one step on one part of A (LO: the small-exponent part);
// op_sel SUB picks the step's scale byte.
template <int SUB, bool LO>
__device__ __forceinline__ void mma_w(v16f (&acc)[2][4], const OpsW& o, const uint32_t (&sa)[2],
                                      const uint32_t (&sb)[4]) {
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v8i b8 = __builtin_shufflevector(o.b[c], o.b[c], 0, 1, 2, 3, -1, -1, -1, -1);
      acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(LO ? o.alo[r] : o.a[r], b8, acc[r][c], 0, 4, SUB,
                                                                   (int)sa[r], SUB, (int)sb[c]);
    }
}

// One LDS read of the next operands after each of the first part's MFMAs: a
// step has 8 operand reads (A: 2 x 2, B: 4).
__device__ __forceinline__ void interleave_w() {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
}

// The split of the next operands (80 VALU instructions) among the second
// part's 8 MFMAs.
__device__ __forceinline__ void interleave_split() {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0); // VALU
  }
}

template <int OUT, bool EPI>
__global__ __launch_bounds__(512, 1) void gemm_w4a8_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ sA,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ sB, void* __restrict__ C,
                                                          uint32_t M, uint32_t N, uint32_t K, uint32_t tilesM,
                                                          uint32_t tilesN, const float* __restrict__ bias,
                                                          uint32_t act) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[W_NSTAGE * W_STAGE_BYTES];

  const uint32_t ldA = K, ldB = K / 2u;
  const uint32_t NS = (K + WSTAGE_K - 1u) / WSTAGE_K;   // stages
  const uint32_t KT = (K + 255u) / 256u;                // scale tiles per 32 rows
  const uint32_t srow = KT * 256u;                      // bytes between 32-row scale tiles
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wm = wave >> 1, wn = wave & 1u;        // 4 x 2 waves, 64 x 128 each

  uint32_t tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, W_GROUP_M, tm, tn);
  const uint32_t m0 = tm * WBM, n0 = tn * WBN;
  const uint32_t rowsA = (M - m0) < WBM ? (M - m0) : WBM;
  const uint32_t rowsB = (N - n0) < WBN ? (N - n0) : WBN;
  const uint8_t* a_tile = A + (size_t)m0 * ldA;
  const uint8_t* b_tile = B + (size_t)n0 * ldB;
  const uint32_t a_bytes = rowsA * ldA, b_bytes = rowsB * ldB;
  const uint32_t RTA = (M + 31u) / 32u, RTB = (N + 31u) / 32u;
  const uint8_t* sa_tile = sA + (size_t)(m0 / 32u) * srow;
  const uint8_t* sb_tile = sB + (size_t)(n0 / 32u) * srow;
  // The tile reads at most its own 8 scale rows (this bounds the range to
  // 8 * srow, well inside 32 bits).
  const uint32_t sa_bytes = __builtin_amdgcn_readfirstlane(min(RTA > m0 / 32u ? RTA - m0 / 32u : 0u, 8u) * srow);
  const uint32_t sb_bytes = __builtin_amdgcn_readfirstlane(min(RTB > n0 / 32u ? RTB - n0 / 32u : 0u, 8u) * srow);

  // ---- copy plan.  A: wave w fills lines w + 8q (q < 4) of 8 rows each;
  // lane L fills row 8(w + 8q) + L/8 at position L%8, i.e. fetches chunk
  // (L%8) ^ ((row >> 1) & 7).  B: wave w fills 1 KB blocks w + 8q (q < 2) of
  // 8 lines; lane L fills line l = 8(w + 8q) + L/8, position p = L%8, which
  // holds row 2l + (v >> 2), chunk v & 3, v = p ^ (l & 3).  Scales: tile w of
  // each operand (rows 32w .. 32w + 31 of the workgroup tile).
  uint32_t voffA[4], voffB[2];
  {
    const uint32_t ach = (lane & 7u) ^ ((4u * (wave & 1u) + (lane >> 4)) & 7u);
#pragma unroll
    for (int q = 0; q < 4; ++q) voffA[q] = (8u * (wave + 8u * q) + (lane >> 3)) * ldA + 16u * ach;
    const uint32_t v = (lane & 7u) ^ ((lane >> 3) & 3u);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t l = 8u * (wave + 8u * q) + (lane >> 3);
      voffB[q] = (2u * l + (v >> 2)) * ldB + 16u * (v & 3u);
    }
  }
  const uint32_t svoff = wave * srow + lane * 4u;

  // Stage s into LDS buffer `buf`; stages past K read out of range (zero
  // fill, no traffic, same instruction count).
  auto dma = [&](uint32_t s, uint32_t buf) {
    const bool live = s < NS;
    // (read into a scalar register before the pin: with a constant s the
    // select would otherwise be a vector instruction)
    const uint32_t ka = opaque(__builtin_amdgcn_readfirstlane(live ? s * A_ROW : 0xFFFFFFFFu));
    const uint32_t kb = opaque(__builtin_amdgcn_readfirstlane(live ? s * B_ROW : 0xFFFFFFFFu));
    const uint32_t ks = opaque(__builtin_amdgcn_readfirstlane(live ? (s >> 1) * 256u : 0xFFFFFFFFu));
    uint8_t* st = lds + buf * W_STAGE_BYTES;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_tile + (live ? ka : 0u), uniform_rem(a_bytes, ka));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_tile + (live ? kb : 0u), uniform_rem(b_bytes, kb));
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa_tile + (live ? ks : 0u), uniform_rem(sa_bytes, ks));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sb_tile + (live ? ks : 0u), uniform_rem(sb_bytes, ks));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + 1024u * (wave + 8u * q)), 16, voffA[q], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + A_REGION + 1024u * (wave + 8u * q)), 16, voffB[q],
                                               0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + A_REGION + B_REGION + 256u * wave), 4, svoff, 0, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + A_REGION + B_REGION + S_REGION + 256u * wave), 4,
                                             svoff, 0, 0, 0);
  };

  // ---- operand reads.  Lane (j, i): A rows 64 wm + 32 r + i, chunks
  // 4q + j and 4q + 2 + j of step q; B rows 128 wn + 32 c + i, chunk 2q + j.
  const uint32_t li = lane & 31u, lj = lane >> 5;
  const uint32_t sw = (li >> 1) & 7u;
  uint32_t rdA[2][2], rdB[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    rdA[q][0] = 128u * li + 16u * ((4u * q + lj) ^ sw);
    rdA[q][1] = 128u * li + 16u * ((4u * q + 2u + lj) ^ sw);
    rdB[q] = 128u * (li >> 1) + 16u * ((4u * (li & 1u) + 2u * q + lj) ^ ((li >> 1) & 3u));
  }
  const uint32_t a_rows = 128u * (64u * wm);          // byte offset of the wave's first A row
  const uint32_t b_lines = 128u * (64u * wn);         // byte offset of the wave's first B line

  auto read_ops = [&](uint32_t buf, int q, OpsW& o) {
    const uint8_t* st = lds + buf * W_STAGE_BYTES;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const v4i lo = *reinterpret_cast<const v4i*>(st + a_rows + 4096u * r + rdA[q][0]);
      const v4i hi = *reinterpret_cast<const v4i*>(st + a_rows + 4096u * r + rdA[q][1]);
      o.a[r] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o.b[c] = *reinterpret_cast<const v4i*>(st + A_REGION + b_lines + 2048u * c + rdB[q]);
  };
  // The lane's scale dwords of stage s: bytes 2h, 2h + 1 (h = s & 1) are the
  // stage's two steps; shifted down so that op_sel 0 / 1 picks them.
  auto read_scales = [&](uint32_t buf, uint32_t s, uint32_t (&sa)[2], uint32_t (&sb)[4]) {
    const uint8_t* st = lds + buf * W_STAGE_BYTES + A_REGION + B_REGION;
    const uint32_t sh = 16u * (s & 1u);
#pragma unroll
    for (int r = 0; r < 2; ++r) sa[r] = *reinterpret_cast<const uint32_t*>(st + 256u * (2u * wm + r) + 4u * lane) >> sh;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      sb[c] = *reinterpret_cast<const uint32_t*>(st + S_REGION + 256u * (4u * wn + c) + 4u * lane) >> sh;
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  // Stage s lives in buffer s % 3.  At the top of iteration s, stage s has
  // landed everywhere (barrier) and stages s+1, s+2 are in flight.  Step 0
  // multiplies while step 1's operands are read; then wait for this wave's
  // copies of stage s+1, barrier (stage s+1 complete; every wave is done
  // reading stage s), copy stage s+3 into stage s's buffer, read stage s+1's
  // first operands and scales, and multiply step 1.
  if (NS > 0) {
    OpsW o0, o1;
    uint32_t sa[2], sb[4], sa_n[2], sb_n[4];
    dma(0, 0);
    dma(1, 1);
    dma(2, 2);
    // 8 copies per wave per stage: 4 of A, 2 of B, one scale tile of each.
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_ops(0, 0, o0);
    read_scales(0, 0, sa, sb);
    split_w(o0);
    uint32_t buf = 0;
    for (uint32_t s = 0; s < NS; ++s) {
      // (kept in a scalar register: the copies take their LDS address from one)
      const uint32_t nbuf = __builtin_amdgcn_readfirstlane(buf == 2u ? 0u : buf + 1u);
      read_ops(buf, 1, o1);
      mma_w<0, false>(acc, o0, sa, sb);
      interleave_w();
      split_w(o1);
      mma_w<0, true>(acc, o0, sa, sb);
      interleave_split();
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      dma(s + 3u, buf);
      read_ops(nbuf, 0, o0);
      read_scales(nbuf, s + 1u, sa_n, sb_n);
      mma_w<1, false>(acc, o1, sa, sb);
      interleave_w();
      split_w(o0);
      mma_w<1, true>(acc, o1, sa, sb);
      interleave_split();
#pragma unroll
      for (int r = 0; r < 2; ++r) sa[r] = sa_n[r];
#pragma unroll
      for (int c = 0; c < 4; ++c) sb[c] = sb_n[c];
      buf = nbuf;
    }
    // Every copy (the zero-fill ones past K included) lands before LDS is
    // reused by the epilogue.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // ---- epilogue ("Rubin FP4 GEMM deep dive" §3.2, §4.2): v = acc (+ bias
  // [column]) (ReLU: v > 0 ? v : +0), then FP32 or BF16 (round to nearest
  // even).  Lane L of a 32 x 32 block holds column L % 32, rows
  // 8 (i / 4) + 4 (L / 32) + i % 4.
  const bool use_bias = EPI && bias != nullptr, use_act = EPI && act != 0u;
  float bcol[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (use_bias) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t col = n0 + 128u * wn + 32u * c + li;
      bcol[c] = col < N ? bias[col] : 0.0f;
    }
  }
  auto epi = [&](float a, int c) {
    float v = a;
    if (use_bias) v = v + bcol[c];
    if (use_act) v = v > 0.0f ? v : 0.0f;
    return v;
  };
  constexpr uint32_t EB = OUT == 1 ? 2u : 4u;
  const bool vec_ok = ((N * EB) % 16u == 0u) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0u);
  if (vec_ok) {
    // BF16 in one pass, FP32 in two passes of 128 rows (waves wm = 2p, 2p + 1).
    constexpr uint32_t PASS_ROWS = OUT == 1 ? 256u : 128u;
    constexpr uint32_t LROW = WBN * EB + 16u;
    static_assert(PASS_ROWS * LROW <= W_NSTAGE * W_STAGE_BYTES, "epilogue tile must fit in LDS");
    __syncthreads();
#pragma unroll
    for (uint32_t pass = 0; pass < 256u / PASS_ROWS; ++pass) {
      if (PASS_ROWS == 256u || (wm >> 1) == pass) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t lcol = 128u * wn + 32u * c + li;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t lrow = 64u * wm - pass * PASS_ROWS + 32u * r + 8u * (i >> 2) + 4u * lj + (i & 3);
              const float val = epi(acc[r][c][i], c);
              if (OUT != 1)
                *reinterpret_cast<float*>(lds + lrow * LROW + 4u * lcol) = val;
              else
                *reinterpret_cast<uint16_t*>(lds + lrow * LROW + 2u * lcol) = f32_to_bf16(val);
            }
          }
      }
      __syncthreads();
      constexpr uint32_t CPR = WBN * EB / 16u;
      constexpr uint32_t STEPS = PASS_ROWS * CPR / 512u;
#pragma unroll
      for (uint32_t st = 0; st < STEPS; ++st) {
        const uint32_t q = st * 512u + threadIdx.x;
        const uint32_t lrow = q / CPR, ch = q % CPR;
        const uint32_t row = pass * PASS_ROWS + lrow;
        const uint32_t col = n0 + ch * (16u / EB);
        // N * EB is a multiple of 16 and col a multiple of 16 / EB, so a
        // chunk that starts inside the row lies wholly inside it.
        if (row < rowsA && col < N)
          *reinterpret_cast<v4i*>(static_cast<uint8_t*>(C) + ((size_t)(m0 + row) * N + col) * EB) =
              *reinterpret_cast<const v4i*>(lds + lrow * LROW + 16u * ch);
      }
      if (PASS_ROWS != 256u) __syncthreads();
    }
    return;
  }
  // Per-element stores (row pitch of C not a multiple of 16 bytes, or C
  // not 16-byte aligned).
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t row = 64u * wm + 32u * r + 8u * (i >> 2) + 4u * lj + (i & 3);
      if (row >= rowsA) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t col = n0 + 128u * wn + 32u * c + li;
        if (col < N) {
          const size_t e = (size_t)(m0 + row) * N + col;
          const float val = epi(acc[r][c][i], c);
          if (OUT == 0)
            static_cast<float*>(C)[e] = val;
          else
            static_cast<uint16_t*>(C)[e] = f32_to_bf16(val);
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm_w4a8(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                            const float* bias, int act, void* C, int64_t M, int64_t N, int64_t K, int out,
                            hipStream_t stream) {
  const uint32_t tilesM = (uint32_t)((M + WBM - 1) / WBM), tilesN = (uint32_t)((N + WBN - 1) / WBN);
  const dim3 grid(tilesM * tilesN), block(512);
  const uint32_t m = (uint32_t)M, n = (uint32_t)N, k = (uint32_t)K, a = (uint32_t)act;
  const bool epi = bias != nullptr || act != 0;
  if (out == 0) {
    if (epi)
      gemm_w4a8_kernel<0, true><<<grid, block, 0, stream>>>(A, sA, B, sB, C, m, n, k, tilesM, tilesN, bias, a);
    else
      gemm_w4a8_kernel<0, false><<<grid, block, 0, stream>>>(A, sA, B, sB, C, m, n, k, tilesM, tilesN, nullptr, 0u);
  } else {
    if (epi)
      gemm_w4a8_kernel<1, true><<<grid, block, 0, stream>>>(A, sA, B, sB, C, m, n, k, tilesM, tilesN, bias, a);
    else
      gemm_w4a8_kernel<1, false><<<grid, block, 0, stream>>>(A, sA, B, sB, C, m, n, k, tilesM, tilesN, nullptr, 0u);
  }
  return hipGetLastError();
}

}  // namespace fp4
