// gemv_nv.hip -- NVFP4 decode GEMV / skinny GEMM (M <= 32 activation rows)
// for gfx950.
//
// C[m,n] = (sum_k A^[m,k] W^[n,k]) * tsA * tsW with NVFP4 operands (NVFP4
// video transcript: 16-value blocks, E4M3 block scale, FP32 tensor scale).
// Decoding streams every weight once, so the path is bound by HBM bandwidth
// ("Rubin FP4 GEMM deep dive", §1.2, §6.2); operands are decoded exactly to
// FP16 and multiplied on the FP16 matrix core (see gemm.hip for why FP16).
#include <float.h>

#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

// ---------------------------------------------------------------------------
// Decode GEMV / skinny GEMM: M <= 32 activation rows against N x K NVFP4
// weights ("Rubin FP4 GEMM deep dive" §1.2, §6.2: decoding streams every
// weight once, so it is bound by memory bandwidth).
//
// Workgroup = 16 wavefronts (4 per SIMD, so loads of some waves overlap the
// decode and MFMAs of others) = one 32-row block of W over the whole of K,
// more blocks in a grid-stride loop when N is large.  Wave w takes the
// 256-value tiles kt = w, w + 16, ...; per tile a lane loads 32 bytes of its
// W row (chunk 2s + j of the row, the scale layout's lane order) and the 8
// scale bytes of its lane.  A wave asks for its next tile only once the
// current one is decoded (ring depth GV_PD = 1): the chip then receives the
// weights in K order, tile column by tile column, and decodes one column while
// the next is in flight; requesting everything at once (depth 2) makes every
// tile land near the end of the transfer and measured 20% slower.
//
// The activation is staged once per workgroup in LDS, in one of two forms:
//   AF16  (small M x K): the exact FP16 values, row-major, rows padded by 16 B
//         so the MFMA operand reads are free of bank conflicts; rows >= M
//         read a zeroed 512-byte block.  No decode work per MFMA.
//   ACODE (otherwise): the packed codes in MFMA operand order
//         ([tile][sub-step][lane] x 16 B) and the scale tiles verbatim; each
//         MFMA decodes its A operand.  Rows >= M are zero codes.  Each wave
//         stages the tiles it reads itself and starts without a barrier
//         (per-wave timeline at M = 32: main loop start 8.5 -> 6.0 us median,
//         kernel 17.4 -> 14.8 us).
// At the end of a row block the 16 waves' partial sums are added in a fixed
// order through LDS (deterministic): for M <= 8 all at once after one
// barrier; for larger M likewise in the workgroup's last row block (in the
// then dead activation staging area), otherwise in three rounds.  No exchange
// between workgroups and no workspace.
// ---------------------------------------------------------------------------
constexpr uint32_t GV_WAVES = 16;               // wavefronts per workgroup (K split)
// Weight tiles in flight per wave (ring depth), both paths.  Depth 1 measured
// best also for the fused path: with depth 2 the whole weight matrix is asked
// for at once and the main loop starts later (M = 1: 16.3 -> 20.8 us, M = 8:
// 22.3 -> 30.0 us at 8192 x 8192).
#define GV_FUSED_PD 1
constexpr uint32_t GV_RED_BYTES = 4u * 32u * 32u * 4u;         // 4 partial-sum slots
constexpr uint32_t GV_A_BYTES = 160u * 1024u - GV_RED_BYTES;    // activation staging
// 16-byte activation loads per thread (at most): FP16 staging, code staging.
constexpr uint32_t GV_A_LOADS_F16 = 3;
constexpr uint32_t GV_A_LOADS_CODE = 8;

// Fused: the activation arrives unquantised (FP32 or BF16); every workgroup
// takes its maximum and quantises it itself (the same NVFP4 steps as the
// quantiser), staging the exact FP16 values as in kAF16.  X blocks per thread.
constexpr uint32_t GV_X_BLOCKS_BF16 = 4;
constexpr uint32_t GV_X_BLOCKS_F32 = 2;

enum { kAF16 = 0, kACode = 1, kFused = 2 };

struct GvTile {
  v4i w[4];   // codes: 32 values per lane per 64-value sub-step
  u32x2 ws;   // the lane's 8 scale bytes (4 sub-steps x 2 blocks)
};

template <int AMODE, int OUT, int XDT, int PD>
__global__ __launch_bounds__(GV_WAVES * 64, 1) void gemv_nv_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ sW, const float* __restrict__ tsA, const float* __restrict__ tsW, void* __restrict__ C,
    uint32_t M, uint32_t N, uint32_t K, const void* __restrict__ X, float* __restrict__ ts_out, uint32_t flags) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a[GV_A_BYTES];
  __shared__ float red[4][32][32];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t li = lane & 31u, lj = lane >> 5;
  const uint32_t KT = (K + 255u) / 256u;
  const uint32_t Kp = KT * 256u;
  // Tiles per wave per row block (at least one, so that K == 0 still stores zeros).
  const uint32_t NJ = KT > GV_WAVES ? (KT + GV_WAVES - 1u) / GV_WAVES : 1u;
  const uint32_t ldb = K / 2u;
  const uint32_t srow = KT * 512u;                         // scale bytes per 32-row tile row
  const uint32_t nblocks = (N + 31u) / 32u;
  const uint32_t nrb = (nblocks - blockIdx.x + gridDim.x - 1u) / gridDim.x;  // row blocks of this workgroup
  const uint32_t T = NJ * nrb;                              // work items of this wave
  const uint32_t RS = 2u * Kp + 16u;                        // AF16 row stride (bytes)
  const uint32_t zero_off = M * RS;                         // AF16: 512 zero bytes

  // ---- activation loads (issued before the weights: waits are in order)
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, M * ldb);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sA, srow);
  constexpr int NA = AMODE == kACode ? (int)GV_A_LOADS_CODE : AMODE == kAF16 ? (int)GV_A_LOADS_F16 : 1;
  v4i ald[NA];
  uint32_t asc[NA];
  v4i ascl = v4i{};
  // Fused: 16-value blocks of X (rows < M, K padded to Kp with zeros); block
  // b = tid + 1024 i is row b / (Kp/16), block b % (Kp/16) of that row.
  constexpr uint32_t XEB = XDT == kDtBF16 ? 2u : 4u;              // bytes per X value
  constexpr int XNB = AMODE == kFused ? (XDT == kDtBF16 ? (int)GV_X_BLOCKS_BF16 : (int)GV_X_BLOCKS_F32) : 1;
  constexpr int XLPB = (int)(16u * XEB / 16u);                     // 16-byte loads per block
  v4i xl[XNB][XLPB];
  const uint32_t xbpr = Kp / 16u;                                   // blocks per (padded) row
  if (AMODE != kFused) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint32_t c = tid + 1024u * i;   // 16-byte chunk handled by this thread
      uint32_t off = 0x80000000u, soff = 0x80000000u;
      if (AMODE == kAF16) {
        const uint32_t cpr = Kp / 32u;       // chunks per row
        const uint32_t row = c / cpr, cc = c % cpr;
        if (row < M && cc * 16u < ldb) {
          off = row * ldb + cc * 16u;
          soff = scale_offset<kFmtNV>(row, 2u * cc, KT);
        }
        asc[i] = __builtin_amdgcn_raw_buffer_load_b16(rsa, soff, 0, 0);
      } else {
        // This wave's tiles only (kt = wave + 16 j, the tiles its main loop
        // reads): operand-order chunk (tile, sub-step, lane).
        const uint32_t kt = wave + GV_WAVES * ((uint32_t)i >> 2), blk = 4u * kt + ((uint32_t)i & 3u);
        if (kt < KT && li < M) off = li * ldb + (blk >> 2) * 128u + (blk & 3u) * 32u + 16u * lj;
      }
      ald[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
    }
    if (AMODE == kACode) {
      // The scale tiles of this wave's tiles verbatim: 32 chunks of 16 B per
      // tile, lanes 32 j + q for tile wave + 16 j.
      const uint32_t kt = wave + GV_WAVES * lj;
      ascl = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rsa, kt < KT ? (kt * 32u + li) * 16u : 0x80000000u,
                                                                          0, 0));
    }
  } else {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, M * K * XEB);
#pragma unroll
    for (int i = 0; i < XNB; ++i) {
      const uint32_t b = tid + 1024u * i;
      const uint32_t row = b / xbpr, bk = b % xbpr;
      const bool ok = row < M && 16u * bk < K;
#pragma unroll
      for (int l = 0; l < XLPB; ++l)
        xl[i][l] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (row * K + 16u * bk) * XEB + 16u * l : 0x80000000u, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- weight ring prologue.  Work item j of this wave is tile
  // kt = wave + 16 (j % NJ) of row block blockIdx.x + (j / NJ) gridDim.x.
  // PD = 1: the ring holds one tile, refilled one 64-value sub-step at a
  // time: once sub-step s of item j is multiplied, sub-step s of item j + 1
  // is requested into the same registers (its scales with sub-step 0), so
  // the weights stream without a pause while item j is computed.
  static_assert(PD == 1, "the sub-step ring holds one tile");
  const uint32_t lane_off = li * ldb + 16u * lj;
  struct TileSrc {
    __amdgpu_buffer_rsrc_t rw, rsw;
    uint32_t off;    // this lane's code offset of the tile (out of range if none)
    uint32_t soff;   // this lane's scale offset
  };
  // Item j's sources; past the last item, out-of-range offsets (the loads
  // return zeros without touching memory), so that every iteration issues
  // the same loads into the same registers.
  auto tile_src = [&](uint32_t j) {
    const uint32_t rb = blockIdx.x + (j / NJ) * gridDim.x;
    const uint32_t kt = wave + GV_WAVES * (j % NJ);
    const uint32_t n0 = rb * 32u;
    const bool item = j < T;              // else rb may lie past the last row block: empty ranges
    const uint32_t rows = __builtin_amdgcn_readfirstlane(item ? (N - n0 < 32u ? N - n0 : 32u) : 0u);
    TileSrc t;
    t.rw = make_rsrc(W + (size_t)n0 * ldb, rows * ldb);
    t.rsw = make_rsrc(sW + (size_t)rb * srow, item ? srow : 0u);
    const bool ok = kt < KT && item;
    t.off = ok ? lane_off + kt * 128u : 0x80000000u;
    t.soff = ok ? kt * 512u + 8u * lane : 0x80000000u;
    return t;
  };
  auto load_codes = [&](const TileSrc& t, int s2) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(t.rw, t.off + 32u * (uint32_t)s2, 0, 0));
  };
  auto load_scales = [&](const TileSrc& t) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(t.rsw, t.soff, 0, 0));
  };
  // Issued unconditionally (out of range when T == 0): on both paths the
  // same loads follow the activation's, so the waits for the activation
  // below count past them and do not wait for the weights.
  GvTile cur;
  {
    const TileSrc t0 = tile_src(0);
    cur.ws = load_scales(t0);   // scales first, as in the loop (the same wait counts on entry)
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) cur.w[s2] = load_codes(t0, s2);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- activation -> LDS
  float s_x = 1.0f;   // activation tensor scale (fused)
  if (AMODE != kFused) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint32_t c = tid + 1024u * i;
      if (AMODE == kAF16) {
        const uint32_t cpr = Kp / 32u;
        const uint32_t row = c / cpr, cc = c % cpr;
        if (row < M) {
          const v2h s0 = scale_pair(asc[i] & 0xFFu), s1 = scale_pair((asc[i] >> 8) & 0xFFu);
          uint8_t* dst = lds_a + row * RS + cc * 64u;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<v8h*>(dst + 16u * g) = decode8((uint32_t)ald[i][g], g < 2 ? s0 : s1);
        }
      } else {
        const uint32_t kt = wave + GV_WAVES * ((uint32_t)i >> 2), blk = 4u * kt + ((uint32_t)i & 3u);
        if (kt < KT) *reinterpret_cast<v4i*>(lds_a + 1024u * blk + 16u * lane) = ald[i];
      }
    }
    if (AMODE == kACode) {
      const uint32_t kt = wave + GV_WAVES * lj;
      if (kt < KT) *reinterpret_cast<v4i*>(lds_a + KT * 4096u + 16u * (kt * 32u + li)) = ascl;
    }
  } else {
    // The block's 16 values, FP32.
    float xv[XNB][16];
#pragma unroll
    for (int i = 0; i < XNB; ++i)
#pragma unroll
      for (int l = 0; l < XLPB; ++l)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = (uint32_t)xl[i][l][e];
          if (XDT == kDtBF16) {
            xv[i][8 * l + 2 * e] = u2f(w << 16);
            xv[i][8 * l + 2 * e + 1] = u2f(w & 0xFFFF0000u);
          } else {
            xv[i][4 * l + e] = u2f(w);
          }
        }
    // Tensor scale (NVFP4 video transcript: one FP32 scale for the global
    // range): s = amax / (6 * 448), 1 for an all-zero X, at least FLT_MIN; or
    // the caller's.  Each workgroup reduces the whole of X itself.
    if (flags & 1u) {
      s_x = *tsA;
    } else {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < XNB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(xv[i][e]));
      m = wave_fmax(m);
      if (lane == 0) red[0][0][wave] = m;
      __syncthreads();
      float amax = 0.0f;
#pragma unroll
      for (int w = 0; w < (int)GV_WAVES; ++w) amax = fmaxf(amax, red[0][0][w]);
      if (amax > 0.0f) {
        s_x = amax / 2688.0f;
        if (s_x < FLT_MIN) s_x = FLT_MIN;
      }
      if (blockIdx.x == 0 && tid == 0 && ts_out) *ts_out = s_x;
    }
    // Quantise each block exactly as the quantiser does and stage the
    // dequantised values E2M1 * E4M3 (exact in FP16; s_x waits for the end).
#pragma unroll
    for (int i = 0; i < XNB; ++i) {
      const uint32_t b = tid + 1024u * i;
      const uint32_t row = b / xbpr, bk = b % xbpr;
      if (row < M) {
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(xv[i][e]));
        const uint32_t sb = e4m3_encode((am / 6.0f) / s_x);
        float y[16];
        if (sb == 0u) {
#pragma unroll
          for (int e = 0; e < 16; ++e) y[e] = __builtin_copysignf(0.0f, xv[i][e]);   // x / inf
        } else {
          const float d = e4m3_value(sb) * s_x;
          const float rd = 1.0f / d;
#pragma unroll
          for (int e = 0; e < 16; ++e) y[e] = nv_div(xv[i][e], d, rd);
        }
        const v2h sp = scale_pair(sb);
        uint8_t* dst = lds_a + row * RS + 32u * bk;
        *reinterpret_cast<v8h*>(dst) = decode8(pack8(y), sp);
        *reinterpret_cast<v8h*>(dst + 16u) = decode8(pack8(y + 8), sp);
      }
    }
  }
  if (AMODE != kACode && tid < 32u) *reinterpret_cast<v4i*>(lds_a + zero_off + 16u * tid) = v4i{};
  // Code staging: each wave staged the tiles it reads itself (LDS operations
  // of one wave complete in order), so it starts without waiting for the
  // others' activation loads.
  if (AMODE != kACode) __syncthreads();

  // ---- main loop
  const float scale = (AMODE == kFused ? s_x : *tsA) * *tsW;
  // AF16: lanes of rows >= M read a 512-byte zero block at a fixed place.
  const uint32_t a_row_off = li * RS + 64u * lj;
  v16f acc0 = v16f{}, acc1 = v16f{};
  {
    for (uint32_t j = 0; j < T; ++j) {
      const uint32_t kt = wave + GV_WAVES * (j % NJ);
      const TileSrc tn = tile_src(j + 1u);
      // The tile's scales (bytes 2 s2 and 2 s2 + 1 of sub-step s2: blocks of
      // code words 0, 1 and 2, 3), converted before their registers take
      // item j + 1's.
      v2h wsp[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        wsp[s2] = (s2 & 1) ? e4m3x2_to_f16<true>(cur.ws[s2 >> 1]) : e4m3x2_to_f16<false>(cur.ws[s2 >> 1]);
      // The conversions stay ahead of the new load (the empty asm takes their
      // results), so that the new scales reuse the old ones' registers: a
      // copy at the loop's end would wait for the load.
      asm volatile("" : : "v"(wsp[0]), "v"(wsp[1]), "v"(wsp[2]), "v"(wsp[3]));
      cur.ws = load_scales(tn);
      const bool live = kt < KT;
      const uint32_t abase = li < M ? a_row_off + kt * 512u : zero_off;
      u32x2 as2 = u32x2{};
      if (AMODE == kACode && live) as2 = *reinterpret_cast<const u32x2*>(lds_a + KT * 4096u + kt * 512u + 8u * lane);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        GvTile& d = cur;
        if (live) {
          const v2h w0 = splat_lo(wsp[s2]), w1 = splat_hi(wsp[s2]);
          v4i acodes = v4i{};
          v2h a0 = v2h{}, a1 = v2h{};
          if (AMODE == kACode) {
            acodes = *reinterpret_cast<const v4i*>(lds_a + (kt * 4u + s2) * 1024u + 16u * lane);
            const v2h asp = (s2 & 1) ? e4m3x2_to_f16<true>(as2[s2 >> 1]) : e4m3x2_to_f16<false>(as2[s2 >> 1]);
            a0 = splat_lo(asp);
            a1 = splat_hi(asp);
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v8h b = decode8((uint32_t)d.w[s2][g], g < 2 ? w0 : w1);
            v8h a;
            if (AMODE != kACode)
              a = *reinterpret_cast<const v8h*>(lds_a + abase + s2 * 128u + 16u * g);
            else
              a = decode8((uint32_t)acodes[g], g < 2 ? a0 : a1);
            if (g & 1)
              acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc1, 0, 0, 0);
            else
              acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc0, 0, 0, 0);
          }
        }
        // Sub-step s2 is decoded: its registers take item j + 1's.
        d.w[s2] = load_codes(tn, s2);
      }

      if (j % NJ == NJ - 1u) {
        // End of a row block.  Lane L holds column n0 + L%32 and rows
        // 8(i/4) + 4(L/32) + i%4 of the wave's partial sums.
        const uint32_t n0 = (blockIdx.x + (j / NJ) * gridDim.x) * 32u;
        v16f acc = acc0 + acc1;
        if (M <= 8u) {
          // Rows < 8 sit in registers 0-3: all 16 waves' partials fit the
          // slots at once ([wave][row][column]); one barrier, then thread
          // (row, column) adds them in wave order, scales and stores.
          float(*part)[8][32] = reinterpret_cast<float(*)[8][32]>(&red[0][0][0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t m = 4u * lj + (uint32_t)i;
            if (m < M) part[wave][m][li] = acc[i];
          }
          __syncthreads();
          if (tid < 32u * M) {
            const uint32_t m = tid >> 5, c = tid & 31u, col = n0 + c;
            float v = part[0][m][c];
#pragma unroll
            for (uint32_t w = 1; w < GV_WAVES; ++w) v += part[w][m][c];
            v *= scale;
            if (col < N) {
              if (OUT == 0)
                static_cast<float*>(C)[(size_t)m * N + col] = v;
              else
                static_cast<uint16_t*>(C)[(size_t)m * N + col] = f32_to_bf16(v);
            }
          }
          if (j + 1u < T) __syncthreads();   // the slots are reused by the next row block
        } else if (j + 1u == T) {
          // The workgroup's last row block: the activation staging is dead, so
          // all 16 waves' partials ([wave][row][column], 64 KB) go there at
          // once; one barrier, then thread (row, column) adds them in wave
          // order, scales and stores.
          static_assert(GV_WAVES * 32u * 32u * 4u <= GV_A_BYTES, "partials fit the staging area");
          float(*part)[32][32] = reinterpret_cast<float(*)[32][32]>(lds_a);
          __syncthreads();   // every wave is done reading the staged activation
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t m = 8u * (i >> 2) + 4u * lj + (i & 3);
            if (m < M) part[wave][m][li] = acc[i];
          }
          __syncthreads();
          const uint32_t m = tid >> 5, c = tid & 31u, col = n0 + c;
          if (m < M && col < N) {
            float v = part[0][m][c];
#pragma unroll
            for (uint32_t w = 1; w < GV_WAVES; ++w) v += part[w][m][c];
            v *= scale;
            if (OUT == 0)
              static_cast<float*>(C)[(size_t)m * N + col] = v;
            else
              static_cast<uint16_t*>(C)[(size_t)m * N + col] = f32_to_bf16(v);
          }
        } else {
          // Waves 0..3 gather waves 4..15 (in order of w), then wave 0
          // gathers 1..3, scales and stores.
#pragma unroll
          for (uint32_t r = 1; r < GV_WAVES / 4u; ++r) {
            if (wave / 4u == r) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const uint32_t m = 8u * (i >> 2) + 4u * lj + (i & 3);
                if (m < M) red[wave & 3u][m][li] = acc[i];
              }
            }
            __syncthreads();
            if (wave < 4u) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const uint32_t m = 8u * (i >> 2) + 4u * lj + (i & 3);
                if (m < M) acc[i] += red[wave][m][li];
              }
            }
            __syncthreads();
          }
          if (wave >= 1u && wave < 4u) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t m = 8u * (i >> 2) + 4u * lj + (i & 3);
              if (m < M) red[wave][m][li] = acc[i];
            }
          }
          __syncthreads();
          if (wave == 0) {
            const uint32_t col = n0 + li;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t m = 8u * (i >> 2) + 4u * lj + (i & 3);
              if (m < M && col < N) {
                const float v = (((acc[i] + red[1][m][li]) + red[2][m][li]) + red[3][m][li]) * scale;
                if (OUT == 0)
                  static_cast<float*>(C)[(size_t)m * N + col] = v;
                else
                  static_cast<uint16_t*>(C)[(size_t)m * N + col] = f32_to_bf16(v);
              }
            }
          }
          __syncthreads();
        }
        acc0 = v16f{};
        acc1 = v16f{};
      }
    }
  }
}

// Which activation staging fits (or -1: the decode kernel does not apply).
static int gemv_amode(int64_t M, int64_t K) {
  const int64_t KT = (K + 255) / 256, Kp = KT * 256;
  const int64_t af16 = M * (2 * Kp + 16) + 512;
  const int64_t af16_chunks = M * (Kp / 32);
  if (af16 <= (int64_t)GV_A_BYTES && af16_chunks <= 1024 * (int64_t)GV_A_LOADS_F16) return kAF16;
  if (KT * 4608 <= (int64_t)GV_A_BYTES && KT * 256 <= 1024 * (int64_t)GV_A_LOADS_CODE && KT * 32 <= 1024)
    return kACode;
  return -1;
}

// The fused path stages X as FP16 (as kAF16) and holds XNB blocks per thread.
static bool gemv_fused_fits(int64_t M, int64_t K, int x_dtype) {
  const int64_t KT = (K + 255) / 256, Kp = KT * 256;
  const int64_t nb = x_dtype == kDtBF16 ? GV_X_BLOCKS_BF16 : GV_X_BLOCKS_F32;
  return M * (2 * Kp + 16) + 512 <= (int64_t)GV_A_BYTES && M * (Kp / 16) <= 1024 * nb;
}

}  // namespace

bool gemv_nv_applies(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 32 && N >= 1 && gemv_amode(M, K) >= 0;
}

bool gemv_nv_fused_applies(int64_t M, int64_t N, int64_t K, int x_dtype) {
  return M >= 1 && M <= 32 && N >= 1 && gemv_fused_fits(M, K, x_dtype);
}

static dim3 gemv_grid(int64_t N) {
  const uint32_t nblocks = (uint32_t)((N + 31) / 32);
  return dim3(nblocks < 256u ? nblocks : 256u);
}

hipError_t launch_gemv_nv(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                          int out_dtype, hipStream_t stream) {
  const dim3 grid = gemv_grid(N), block(GV_WAVES * 64);
  const uint32_t m = (uint32_t)M, n = (uint32_t)N, k = (uint32_t)K;
  const int mode = gemv_amode(M, K);
#define GV_LAUNCH(MODE, OUTT) \
  gemv_nv_kernel<MODE, OUTT, kDtBF16, 1><<<grid, block, 0, stream>>>(A, sA, B, sB, tsA, tsB, C, m, n, k, nullptr, \
                                                                     nullptr, 0u)
  if (mode == kAF16) {
    if (out_dtype == 0) GV_LAUNCH(kAF16, 0);
    else GV_LAUNCH(kAF16, 1);
  } else {
    if (out_dtype == 0) GV_LAUNCH(kACode, 0);
    else GV_LAUNCH(kACode, 1);
  }
#undef GV_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemv_nv_fused(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags,
                                const uint8_t* B, const uint8_t* sB, const float* tsB, void* C, int64_t M,
                                int64_t N, int64_t K, int out_dtype, hipStream_t stream) {
  const dim3 grid = gemv_grid(N), block(GV_WAVES * 64);
  const uint32_t m = (uint32_t)M, n = (uint32_t)N, k = (uint32_t)K;
  const float* ts_in = x_tensor_scale;
  float* ts_out = (flags & 1u) ? nullptr : x_tensor_scale;
#define GV_LAUNCH(OUTT, XT)                                                                                      \
  gemv_nv_kernel<kFused, OUTT, XT, GV_FUSED_PD><<<grid, block, 0, stream>>>(nullptr, nullptr, B, sB, ts_in, tsB, C, \
                                                                              m, n, k, X, ts_out, flags)
  if (x_dtype == kDtBF16) {
    if (out_dtype == 0) GV_LAUNCH(0, kDtBF16);
    else GV_LAUNCH(1, kDtBF16);
  } else {
    if (out_dtype == 0) GV_LAUNCH(0, kDtF32);
    else GV_LAUNCH(1, kDtF32);
  }
#undef GV_LAUNCH
  return hipGetLastError();
}

}  // namespace fp4
