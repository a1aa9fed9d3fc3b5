// gemm.hip -- tiled FP4 block-scaled GEMM for gfx950: MXFP4 and NVFP4, dense
// and grouped (mixture-of-experts).
//
// C[m,n] = (sum_k A^[m,k] B^[n,k]) * tsA * tsB, A^ and B^ the block-scaled
// E2M1 operands, FP32 accumulation ("Rubin FP4 GEMM deep dive", §1.1: FP4
// inputs, FP32 accumulation; §3.1, §4.2: the result is multiplied by the
// product of the scales; §3.2: global -> shared -> registers -> matrix core ->
// FP32 accumulators -> epilogue).
//
// Matrix core per format:
//   MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 -- the E8M0 scales ride in the
//     instruction (one byte per lane per 32-value chunk), so the accumulators
//     hold the scaled product.  (32x32x64 is the full-rate FP4 form on gfx950;
//     16x16x128 runs at half rate.)
//   NVFP4: the instruction scales take only E8M0, so E4M3 16-blocks cannot
//     ride in it exactly.  E2M1 * E4M3 is exact in FP16, so each wave decodes
//     its operands to FP16 in registers (v_cvt_scalef32_pk_f16_fp4, then a
//     packed FP16 multiply by the block scale) and runs
//     v_mfma_f32_32x32x16_f16; the FP32 tensor scales go to the epilogue.
//
// Data path (both formats): one 256 x 256 output tile per workgroup of 8
// wavefronts (2 per SIMD, 128 x 64 each, 128 accumulators per lane).  K
// advances in stages of 256 values: the stage's codes (256 rows x 128 B of A
// and of B) and scale tiles are copied from global memory straight into LDS
// with buffer_load ... lds, double-buffered.  LDS row r keeps its eight 16-byte
// chunks c at position c ^ ((r >> 1) & 7), so the operand reads (lane = 32 *
// chunk parity + row, ds_read_b128) are free of bank conflicts while each
// load instruction still reads 8 whole 128-byte row segments.  Within a stage,
// the operands of the next 64-value sub-step are read while the current one
// multiplies; one barrier per stage.  The epilogue goes through LDS so that C
// is written with 16-byte row-contiguous stores.
//
// Grouped: the tiles of all experts form one list, ordered expert by expert;
// every workgroup derives its (expert, m-tile, n-tile) from the device-side
// group offsets (no host round trip), gathers its A rows through row_idx
// (codes per lane, scale dwords per lane) and multiplies by that expert's B.
#include <atomic>

#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

constexpr uint32_t BM = 256, BN = 256;
constexpr uint32_t STAGE_K = 256;                   // K values per stage
constexpr uint32_t ROW_BYTES = STAGE_K / 2;         // 128 B of codes per row per stage
constexpr uint32_t REGION = 256 * ROW_BYTES;        // 32 KB of codes per operand per stage
constexpr uint32_t NSTAGE = 2;
constexpr uint32_t GROUP_M = 4;

template <int FMT>
struct Fmt;
template <>
struct Fmt<kFmtMX> {
  static constexpr uint32_t STILE = 256;  // 32 rows x 8 blocks of 32
  typedef uint32_t S;                     // per-lane scales of one 32-row block (4 sub-steps)
};
template <>
struct Fmt<kFmtNV> {
  static constexpr uint32_t STILE = 512;  // 32 rows x 16 blocks of 16
  typedef u32x2 S;
};

// Operands of one 64-value K sub-step of a wave's 128 x 64 sub-tile.
struct Ops {
  v4i a[4], b[2];
};

template <int N>
struct IntC {
  static constexpr int value = N;
};

// MXFP4: 8 MFMAs of one sub-step (2 R when only the wave's first R 32-row
// blocks hold rows); op_sel SUB picks the sub-step's scale byte.
template <int SUB, int R = 4>
__device__ __forceinline__ void mma_sub(v16f (&acc)[4][2], const Ops& o, const uint32_t (&sa)[4],
                                        const uint32_t (&sb)[2]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const v8i a8 = __builtin_shufflevector(o.a[r], o.a[r], 0, 1, 2, 3, -1, -1, -1, -1);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const v8i b8 = __builtin_shufflevector(o.b[c], o.b[c], 0, 1, 2, 3, -1, -1, -1, -1);
      acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[r][c], 4, 4, SUB, (int)sa[r], SUB,
                                                                   (int)sb[c]);
    }
  }
}

// NVFP4: the lane's 32 codes of each block split into four groups of 8 (group
// g lies in the chunk's 16-block g/2), decoded to FP16, one 32x32x16 MFMA per
// block pair and group.
template <int SUB, int R = 4>
__device__ __forceinline__ void mma_sub(v16f (&acc)[4][2], const Ops& o, const u32x2 (&sa)[4],
                                        const u32x2 (&sb)[2]) {
  // Scale bytes 2 SUB, 2 SUB + 1 of the lane's 8 (groups 0-1, 2-3) as FP16,
  // two per conversion.
  v2h spa[4], spb[2];
#pragma unroll
  for (int r = 0; r < R; ++r)
    spa[r] = (SUB & 1) ? e4m3x2_to_f16<true>(sa[r][SUB >> 1]) : e4m3x2_to_f16<false>(sa[r][SUB >> 1]);
#pragma unroll
  for (int c = 0; c < 2; ++c)
    spb[c] = (SUB & 1) ? e4m3x2_to_f16<true>(sb[c][SUB >> 1]) : e4m3x2_to_f16<false>(sb[c][SUB >> 1]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    v8h a[4], b[2];
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = decode8((uint32_t)o.a[r][g], g < 2 ? splat_lo(spa[r]) : splat_hi(spa[r]));
#pragma unroll
    for (int c = 0; c < 2; ++c) b[c] = decode8((uint32_t)o.b[c][g], g < 2 ? splat_lo(spb[c]) : splat_hi(spb[c]));
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[r], b[c], acc[r][c], 0, 0, 0);
  }
}

// One LDS read of the next operands after each MFMA (MXFP4): NR of them
// among the sub-step's 8 MFMAs.
template <int FMT, int NR = 6>
__device__ __forceinline__ void interleave_mfma_reads() {
  if (FMT == kFmtMX) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    if (NR < 8) __builtin_amdgcn_sched_group_barrier(0x008, 8 - NR, 0);
  }
}

// Grouped problem description (device pointers).
struct Groups {
  const int32_t* row_idx;    // output row -> A row (NULL: A is in output-row order)
  const int32_t* group_off;  // E + 1 prefix offsets of the output rows
  int32_t E;
  uint32_t A_rows;           // rows of A (tokens)
  size_t b_codes_stride;     // bytes between experts' codes
  size_t b_scales_stride;    // bytes between experts' scale buffers
};

// A load of read-only memory at a uniform address through the scalar cache.
// The kernels never write the arrays read this way; without the constant
// address space the compiler falls back to vector loads once the kernel has
// stored anything, and those wait behind every operand copy in flight.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Rows [lo, hi) of expert e, clamped so that 0 <= lo <= hi <= total: a
// malformed group_off (negative, decreasing or past the end) can then only
// drop rows, never address rows of C past the end.
__device__ __forceinline__ void group_rows(const Groups& gp, int32_t e, uint32_t total, uint32_t& lo,
                                           uint32_t& hi) {
  const int32_t a = sload(gp.group_off + e), b = sload(gp.group_off + e + 1);
  lo = a < 0 ? 0u : ((uint32_t)a < total ? (uint32_t)a : total);
  hi = b < 0 ? 0u : ((uint32_t)b < total ? (uint32_t)b : total);
  if (hi < lo) hi = lo;
}

// The M-tile of each group.  A group of cnt rows is cut into cnt / 256
// m-tiles of 256 rows and a last m-tile of the remaining cnt % 256 rows.
// Inside the kernel a wave multiplies only the 32-row blocks of its 128 rows
// that hold group rows, so that last m-tile is in effect a 32-, 64-, 128-,
// 160-, 192- or 256-row tile (16 or fewer rows: 32).  A last m-tile of at
// most 128 rows keeps half the waves off the matrix core ("light"); every
// other m-tile is "heavy".
__device__ __forceinline__ void expert_mtiles(uint32_t cnt, uint32_t& heavy, uint32_t& light) {
  const uint32_t rem = cnt % BM;
  light = (rem != 0u && rem <= BM / 2u) ? 1u : 0u;
  heavy = cnt / BM + (rem > BM / 2u ? 1u : 0u);
}

// Locate tile t in the grouped list.  The list is cost-first: segment s < E
// holds expert s's heavy m-tiles x tilesN n-tiles (grouped raster within the
// expert), segment E + e the n-tiles of expert e's light m-tile, if any.
// Returns false past the last tile.  Uniform per workgroup (scalar loads of
// group_off).  The search starts at the cursor (scur, fcur) = (segment, its
// first tile) of the last call, since a workgroup's tiles only increase; t
// below the cursor restarts it from segment 0.
__device__ __forceinline__ bool grouped_tile(const Groups& gp, uint32_t total_rows, uint32_t t, uint32_t tilesN,
                                             uint32_t& e_out, uint32_t& row0, uint32_t& rows, uint32_t& tm,
                                             uint32_t& tn, int32_t& scur, uint32_t& fcur) {
  if (t < fcur) {
    scur = 0;
    fcur = 0;
  }
  uint32_t first = fcur;
  for (int32_t s = scur; s < 2 * gp.E; ++s) {
    const bool heavy_seg = s < gp.E;
    const int32_t e = heavy_seg ? s : s - gp.E;
    uint32_t lo, hi, hm, lm;
    group_rows(gp, e, total_rows, lo, hi);
    const uint32_t cnt = hi - lo;
    expert_mtiles(cnt, hm, lm);
    const uint32_t mt = heavy_seg ? hm : lm;
    const uint32_t n = mt * tilesN;
    if (t < first + n) {
      uint32_t a, b;
      if (heavy_seg) {
        raster_coords(t - first, mt, tilesN, GROUP_M, a, b);
      } else {
        a = hm;             // the light m-tile follows the heavy ones
        b = t - first;
      }
      e_out = (uint32_t)e;
      row0 = lo;
      rows = cnt;
      tm = a;
      tn = b;
      scur = s;
      fcur = first;
      return true;
    }
    first += n;
  }
  return false;
}

// Heavy and light tile counts of the grouped list.
__device__ __forceinline__ void grouped_tile_counts(const Groups& gp, uint32_t total_rows, uint32_t tilesN,
                                                    uint32_t& heavy, uint32_t& light) {
  heavy = 0;
  light = 0;
  for (int32_t e = 0; e < gp.E; ++e) {
    uint32_t lo, hi, hm, lm;
    group_rows(gp, e, total_rows, lo, hi);
    expert_mtiles(hi - lo, hm, lm);
    heavy += hm * tilesN;
    light += lm * tilesN;
  }
}

// Operand addressing of one output tile: scalar bases and byte ranges, plus
// the per-lane source offsets of A (gathered rows when grouped).
struct TileAddr {
  const uint8_t* a_base;
  const uint8_t* sa_base;
  const uint8_t* b_tile;
  const uint8_t* sb_tile;
  uint32_t a_bytes, sa_bytes, b_bytes, sb_bytes;
  uint32_t m0, n0, rowsA, row0;
  uint32_t voffA[4];
  uint32_t svoffA;
  uint32_t expert;   // grouped: the tile's expert
};

// PERSIST: workgroups walk tiles (grid <= resident workgroups) with the next
// tile's first stages copied during this one's last iterations, and store C
// from registers; else one tile per workgroup, C stored through LDS.  EPI:
// the epilogue reads bias and act (otherwise they are not even loaded, which
// keeps the plain kernels' registers as they were).
template <int FMT, int OUT, bool GROUPED, bool PERSIST, bool EPI>
__global__ __launch_bounds__(512, 1) void gemm_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
                                                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB,
                                                     const float* __restrict__ tsA, const float* __restrict__ tsB,
                                                     void* __restrict__ C, uint32_t M, uint32_t N, uint32_t K,
                                                     uint32_t tilesM, uint32_t tilesN, Groups gp,
                                                     const float* __restrict__ bias, uint32_t act,
                                                     uint8_t* __restrict__ Cs, const float* __restrict__ tsC) {
  static_assert(OUT < 2 || (!PERSIST && !GROUPED), "FP4 output: one tile per workgroup, dense");
  typedef typename Fmt<FMT>::S S;
  constexpr uint32_t STILE = Fmt<FMT>::STILE;
  constexpr uint32_t SCALE_REGION = 8 * STILE;
  constexpr uint32_t STAGE_BYTES = 2 * REGION + 2 * SCALE_REGION;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE_BYTES];

  const uint32_t ldb = K / 2u;                    // bytes per row of codes
  const uint32_t KT = (K + 255u) / 256u;          // stages (= scale tiles per row tile)
  const uint32_t srow = KT * STILE;               // bytes between 32-row scale tiles
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const uint32_t wm = wave >> 2, wn = wave & 3u;  // 2 x 4 waves, 128 x 64 each

  // ---- tile schedule.  Workgroup b takes the virtual tiles v = b, b + G, ...
  // (G = grid size, a multiple of 8, so that v % 8 and with it the XCD stay
  // fixed).  Dense: v -> tile as tile_coords.  Grouped: XCD x = v % 8 owns
  // the x-th eighth of the heavy tiles followed by the x-th eighth of the
  // light ones, walked in that order (j = v / 8), so every XCD ends on cheap
  // tiles, and the first of them go to the workgroups that drew one heavy
  // tile fewer.
  uint32_t total, nheavy = 0, nlight = 0;
  if (GROUPED) {
    grouped_tile_counts(gp, M, tilesN, nheavy, nlight);
    total = nheavy + nlight;
  } else {
    total = tilesM * tilesN;
  }
  // Dense persistent: when the tiles leave a last round that fills at most
  // half the grid, its tiles run as two 128-row halves each (items), so that
  // every workgroup ends after the same whole tiles plus at most one half
  // (whose 128 idle rows' waves only copy); e.g. 896 tiles on 256 workgroups:
  // 768 + 2 x 128 items, 3.5 tiles of work each instead of 4 or 3.
  const uint32_t tail = !GROUPED && PERSIST && total > gridDim.x ? total % gridDim.x : 0u;
  const uint32_t first_half = tail != 0u && 2u * tail <= gridDim.x ? total - tail : total;
  const uint32_t items = total + (total - first_half);
  auto tile_of = [&](uint32_t v, uint32_t& t) -> bool {
    if constexpr (GROUPED) {
      const uint32_t x = v & 7u, j = v >> 3;
      const uint32_t hx = (nheavy + 7u) >> 3, lx = (nlight + 7u) >> 3;
      const uint32_t hb = x * hx, lb = x * lx;
      const uint32_t hc = nheavy > hb ? (nheavy - hb < hx ? nheavy - hb : hx) : 0u;
      const uint32_t lc = nlight > lb ? (nlight - lb < lx ? nlight - lb : lx) : 0u;
      if (j < hc) {
        t = hb + j;
        return true;
      }
      t = nheavy + lb + (j - hc);
      return j - hc < lc;
    }
    t = v;
    return v < items;
  };

  // ---- direct-to-LDS load plan.  One code load (1 KB) fills 8 rows: lane L
  // fills LDS row L/8, position L%8, i.e. fetches the row's chunk
  // (L%8) ^ ((row >> 1) & 7).  Wave w loads row groups w + 8q (q < 4) of A and
  // of B and scale tile w of A and of B.
  const uint32_t grow = lane >> 3;
  // Grouped: the tile row whose scale bytes this lane copies (see gather_offsets).
  const uint32_t scale_row = FMT == kFmtNV ? lane >> 1 : lane & 31u;
  const uint32_t gchunk = (lane & 7u) ^ ((4u * (wave & 1u) + (lane >> 4)) & 7u);
  uint32_t voffB[4];
  const uint32_t svoffB = (wave * KT) * STILE + lane * 4u;
#pragma unroll
  for (int q = 0; q < 4; ++q) voffB[q] = (8u * (wave + 8u * q) + grow) * ldb + 16u * gchunk;

  int32_t g_ecur = 0;     // grouped: search cursor of grouped_tile
  uint32_t g_fcur = 0;
  auto make_tile = [&](uint32_t t, TileAddr& T) {
    uint32_t rowsA, row0 = 0, expert = 0, m0, n0;
    const uint8_t* Bx = B;
    const uint8_t* sBx = sB;
    if (GROUPED) {
      uint32_t cnt, tm, tn;
      grouped_tile(gp, M, t, tilesN, expert, row0, cnt, tm, tn, g_ecur, g_fcur);
      m0 = tm * BM;
      n0 = tn * BN;
      rowsA = (cnt - m0) < BM ? (cnt - m0) : BM;
      Bx += (size_t)expert * gp.b_codes_stride;
      sBx += (size_t)expert * gp.b_scales_stride;
    } else {
      uint32_t tm, tn, tile = t, half = 0u, hrows = BM;
      if (t >= first_half) {   // item t: half (t - first_half) % 2 of tile first_half + (t - first_half) / 2
        tile = first_half + ((t - first_half) >> 1);
        half = (t - first_half) & 1u;
        hrows = BM / 2u;
      }
      tile_coords(tile, tilesM, tilesN, GROUP_M, tm, tn);
      m0 = tm * BM + half * (BM / 2u);
      n0 = tn * BN;
      rowsA = M > m0 ? ((M - m0) < hrows ? (M - m0) : hrows) : 0u;
    }
    T.m0 = m0;
    T.n0 = n0;
    T.rowsA = rowsA;
    T.row0 = row0;
    if constexpr (GROUPED) T.expert = expert;
    const uint32_t rowsB = (N - n0) < BN ? (N - n0) : BN;
    T.b_tile = Bx + (size_t)n0 * ldb;
    T.b_bytes = rowsB * ldb;
    const uint32_t RTB = (N + 31u) / 32u;
    T.sb_tile = sBx + (size_t)(n0 / 32u) * srow;
    T.sb_bytes = (RTB > n0 / 32u ? RTB - n0 / 32u : 0u) * srow;
    if (GROUPED) {
      // Gathered rows: lane offsets from the A row of each tile row; rows past
      // the group get an out-of-range offset and load zeros.
      T.a_base = A;
      T.a_bytes = gp.A_rows * ldb;
      // The token indices (rows past the group read the tile's first row);
      // turned into offsets by gather_offsets.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t r = 8u * (wave + 8u * q) + grow;
        const uint32_t o = row0 + m0 + (r < rowsA ? r : 0u);
        T.voffA[q] = gp.row_idx ? (uint32_t)gp.row_idx[o] : o;
      }
      const uint32_t r = 32u * wave + scale_row;
      const uint32_t o = row0 + m0 + (r < rowsA ? r : 0u);
      T.svoffA = gp.row_idx ? (uint32_t)gp.row_idx[o] : o;
      T.sa_base = sA;
      T.sa_bytes = ((gp.A_rows + 31u) / 32u) * srow;
    } else {
      // Dense tiles read A with B's per-lane offsets (voffA unused).
      T.a_base = A + (size_t)m0 * ldb;
      T.a_bytes = rowsA * ldb;
      const uint32_t RTA = (M + 31u) / 32u;
      T.sa_base = sA + (size_t)(m0 / 32u) * srow;
      T.sa_bytes = (RTA > m0 / 32u ? RTA - m0 / 32u : 0u) * srow;
    }
  };

  // Grouped: the loaded token indices of T become its lane offsets; rows
  // past the group get an out-of-range offset and load zeros.  Scale dwords
  // of scale block `wave`, each taken from the gathered row's own scale tile:
  // MXFP4: lane L = 32j + i copies entry (row i, chunk parity j), 4 bytes;
  // NVFP4: lane L copies dword L % 2 of entry (row L / 2, parity h) of 8
  // bytes, h the half of the 512-byte tile being copied (its copy adds 256 h).
  auto gather_offsets = [&](TileAddr& T) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t r = 8u * (wave + 8u * q) + grow;
      T.voffA[q] = r < T.rowsA ? T.voffA[q] * ldb + 16u * gchunk : 0x80000000u;
    }
    const uint32_t tok = T.svoffA;
    const uint32_t in_tile = FMT == kFmtNV ? (tok & 31u) * 8u + (lane & 1u) * 4u : ((lane & 32u) + (tok & 31u)) * 4u;
    T.svoffA = 32u * wave + scale_row < T.rowsA ? (tok >> 5) * srow + in_tile : 0x80000000u;
  };

  // Copy stage `stage_k` of tile T into LDS buffer `buf`; stages past K (or
  // live == false) read out of range: zero fill, no memory traffic, and the
  // same instruction count, so that the wait counts stay exact.
  auto dma = [&](const TileAddr& T, uint32_t stage_k, uint32_t buf, bool live) {
    // Stage offsets are folded into the descriptors (scalar registers), so
    // the per-lane offsets stay loop-invariant.
    const uint32_t kb = opaque(live ? stage_k * ROW_BYTES : 0xFFFFFFFFu);
    const uint32_t ko = opaque(live ? stage_k * STILE : 0xFFFFFFFFu);
    uint8_t* st = lds + buf * STAGE_BYTES;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(T.a_base + (live ? kb : 0u), uniform_rem(T.a_bytes, kb));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(T.b_tile + (live ? kb : 0u), uniform_rem(T.b_bytes, kb));
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(T.sa_base + (live ? ko : 0u), uniform_rem(T.sa_bytes, ko));
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(T.sb_tile + (live ? ko : 0u), uniform_rem(T.sb_bytes, ko));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + 1024u * (wave + 8u * q)), 16,
                                               GROUPED ? T.voffA[q] : voffB[q], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + REGION + 1024u * (wave + 8u * q)), 16, voffB[q], 0,
                                               0, 0);
    }
#pragma unroll
    for (uint32_t h = 0; h < STILE / 256u; ++h) {
      // NVFP4 lanes own 8 bytes: the two halves of a 512-byte tile are lanes
      // 0-31 and 32-63 of the dword copy.
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + 2u * REGION + STILE * wave + 256u * h), 4,
                                               (GROUPED ? T.svoffA : svoffB) + 256u * h, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + 2u * REGION + SCALE_REGION + STILE * wave + 256u * h),
                                               4, svoffB + 256u * h, 0, 0, 0);
    }
  };
  constexpr int LOADS_PER_STAGE = 8 + 2 * (int)(STILE / 256u);

  // ---- operand reads: lane (j = L/32, i = L%32) of a 32-row block reads row
  // i, chunk 2q + j of sub-step q, stored at position (2q + j) ^ ((i>>1)&7).
  const uint32_t li = lane & 31u, lj = lane >> 5;
  uint32_t rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rd[q] = 128u * li + 16u * ((2u * q + lj) ^ ((li >> 1) & 7u));
  const uint32_t a_rows = 128u * (128u * wm);   // byte offset of this wave's first A row
  const uint32_t b_rows = 128u * (64u * wn);

  auto read_ops = [&](uint32_t buf, int q, Ops& o) {
    const uint8_t* st = lds + buf * STAGE_BYTES;
#pragma unroll
    for (int r = 0; r < 4; ++r) o.a[r] = *reinterpret_cast<const v4i*>(st + a_rows + 4096u * r + rd[q]);
#pragma unroll
    for (int c = 0; c < 2; ++c) o.b[c] = *reinterpret_cast<const v4i*>(st + REGION + b_rows + 4096u * c + rd[q]);
  };
  auto read_scales = [&](uint32_t buf, S (&sa)[4], S (&sb)[2]) {
    const uint8_t* st = lds + buf * STAGE_BYTES + 2u * REGION;
    constexpr uint32_t LB = STILE / 64u;  // bytes per lane
#pragma unroll
    for (int r = 0; r < 4; ++r) sa[r] = *reinterpret_cast<const S*>(st + STILE * (4u * wm + r) + LB * lane);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      sb[c] = *reinterpret_cast<const S*>(st + SCALE_REGION + STILE * (2u * wn + c) + LB * lane);
  };

  uint32_t v = blockIdx.x, t;
  if (!tile_of(v, t)) return;
  TileAddr cur;
  make_tile(t, cur);
  if (GROUPED) gather_offsets(cur);
  const float scale = (tsA ? *tsA : 1.0f) * (tsB ? *tsB : 1.0f);

  // Stage k of a tile covers K values [256k, 256k + 256) in four 64-value
  // sub-steps; stages alternate between the two LDS buffers in one sequence
  // over all the workgroup's tiles (g = stage number in that sequence).
  // Sub-steps 0-2 each multiply while the next sub-step's operands are read
  // from LDS; then wait for this wave's copies of stage g+1, barrier (stage
  // g+1 has landed everywhere; every wave is done reading stage g), copy stage
  // g+2 into stage g's buffer, read stage g+1's first operands and scales, and
  // multiply sub-step 3.  Once a tile has no stages left to copy, its last two
  // iterations copy the first two stages of the workgroup's next tile, so
  // that tile starts without waiting while this one's results are stored.  A
  // last, partial stage runs over codes past K; their scale bytes are the
  // tile's padding (0), which makes those products zero (E8M0: 2^-127 on both
  // operands, <= 36 * 2^-254, zero in FP32; E4M3: an FP16 zero).
  Ops o0, o1;
  S sa[4], sb[2], sa_n[4], sb_n[2];
  if (KT > 0) {
    dma(cur, 0, 0, true);
    dma(cur, 1, 1, KT > 1u);
    if (LOADS_PER_STAGE == 10)
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  uint32_t g = 0;                                // sequence number of cur's stage 0
  while (true) {
    // The tile's first operands (its stage 0 landed at the last barrier).
    read_ops(g & 1u, 0, o0);
    read_scales(g & 1u, sa, sb);
    uint32_t vn = v + gridDim.x, tn_;
    // Tiles of one K stage leave no iteration to copy a next tile in: one
    // tile per workgroup (the host sizes the grid accordingly).
    const bool has_next = PERSIST && KT >= 2u && tile_of(vn, tn_);
    TileAddr nxt = cur;
    if (has_next) make_tile(tn_, nxt);

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

    // The second 128 rows of a tile of at most 128 rows (a dense half tile, a
    // grouped light tile): those waves only take their part of the stage
    // copies (same waits, barriers and copies as the others).  Grouped: a
    // wave whose 128 rows hold at most 32 (64) group rows multiplies only its
    // first one (two) 32-row blocks, in a loop of its own with the same waits,
    // barriers and copies.
    const bool idle = PERSIST && cur.rowsA <= BM / 2u && wm == 1u;
    uint32_t nblk = 4u;   // 32-row blocks this wave multiplies
    if constexpr (GROUPED) {
      const uint32_t wrows = cur.rowsA > 128u * wm ? cur.rowsA - 128u * wm : 0u;
      nblk = idle ? 4u : (wrows <= 32u ? 1u : (wrows <= 64u ? 2u : 4u));
    }
    for (uint32_t k = 0; idle && k < KT; ++k) {
      const uint32_t buf = (g + k) & 1u;
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (GROUPED && k == 0u && has_next) gather_offsets(nxt);
      const bool own = k + 2u < KT;
      dma(own ? cur : nxt, own ? k + 2u : k + 2u - KT, buf, own || has_next);
    }
    if constexpr (GROUPED) {
      // read_ops for a wave that multiplies only its first R 32-row blocks.
      auto read_ops_n = [&](uint32_t buf, int q, Ops& o, auto rc) {
        constexpr int R = decltype(rc)::value;
        const uint8_t* st = lds + buf * STAGE_BYTES;
#pragma unroll
        for (int r = 0; r < R; ++r) o.a[r] = *reinterpret_cast<const v4i*>(st + a_rows + 4096u * r + rd[q]);
#pragma unroll
        for (int c = 0; c < 2; ++c) o.b[c] = *reinterpret_cast<const v4i*>(st + REGION + b_rows + 4096u * c + rd[q]);
      };
      auto short_loop = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        for (uint32_t k = 0; k < KT; ++k) {
          const uint32_t buf = (g + k) & 1u, nbuf = buf ^ 1u;
          read_ops_n(buf, 1, o1, rc);
          mma_sub<0, R>(acc, o0, sa, sb);
          read_ops_n(buf, 2, o0, rc);
          mma_sub<1, R>(acc, o1, sa, sb);
          read_ops_n(buf, 3, o1, rc);
          mma_sub<2, R>(acc, o0, sa, sb);
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if (k == 0u && has_next) gather_offsets(nxt);
          const bool own = k + 2u < KT;
          dma(own ? cur : nxt, own ? k + 2u : k + 2u - KT, buf, own || has_next);
          read_ops_n(nbuf, 0, o0, rc);
          read_scales(nbuf, sa_n, sb_n);
          mma_sub<3, R>(acc, o1, sa, sb);
#pragma unroll
          for (int r = 0; r < 4; ++r) sa[r] = sa_n[r];
#pragma unroll
          for (int c = 0; c < 2; ++c) sb[c] = sb_n[c];
        }
      };
      if (nblk == 1u)
        short_loop(IntC<1>{});
      else if (nblk == 2u)
        short_loop(IntC<2>{});
    }
    for (uint32_t k = 0; !idle && nblk == 4u && k < KT; ++k) {
      const uint32_t buf = (g + k) & 1u, nbuf = buf ^ 1u;
      read_ops(buf, 1, o1);
      mma_sub<0>(acc, o0, sa, sb);
      interleave_mfma_reads<FMT>();
      read_ops(buf, 2, o0);
      mma_sub<1>(acc, o1, sa, sb);
      interleave_mfma_reads<FMT>();
      read_ops(buf, 3, o1);
      mma_sub<2>(acc, o0, sa, sb);
      interleave_mfma_reads<FMT>();
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // The next tile's token indices, loaded at the tile's start, have
      // arrived with this wait: a wait right after their loads would also
      // wait for the previous tile's C stores (loads and stores retire in
      // order), about 2.6 us per tile.
      if (GROUPED && k == 0u && has_next) gather_offsets(nxt);
      // Stage g+k+2 goes into this buffer: this tile's stage k+2, or the next
      // tile's stage k+2-KT.
      const bool own = k + 2u < KT;
      const TileAddr& src = own ? cur : nxt;
      const uint32_t sk = own ? k + 2u : k + 2u - KT;
      const bool live = own || has_next;
      // Waves w and w + 4 share a SIMD.  Dense MXFP4: waves 0-3 issue their
      // copies first and waves 4-7 after their sub-step 3 MFMAs, so that on
      // every SIMD one wave keeps the matrix core busy while the other feeds
      // the address unit (all eight issuing at once after the barrier left
      // the matrix core idle for much of the copy issue).  The NVFP4 and
      // grouped kernels keep one order: two copies of their sub-step code
      // exceed the register budget.
      constexpr bool STAGGER = FMT == kFmtMX && !GROUPED;
      if (!STAGGER || wave < 4u) {
        dma(src, sk, buf, live);
        read_ops(nbuf, 0, o0);
        read_scales(nbuf, sa_n, sb_n);
        mma_sub<3>(acc, o1, sa, sb);
        interleave_mfma_reads<FMT, 8>();
      } else {
        read_ops(nbuf, 0, o0);
        read_scales(nbuf, sa_n, sb_n);
        mma_sub<3>(acc, o1, sa, sb);
        interleave_mfma_reads<FMT, 8>();
        dma(src, sk, buf, live);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sa[r] = sa_n[r];
#pragma unroll
      for (int c = 0; c < 2; ++c) sb[c] = sb_n[c];
    }

    // ---- epilogue ("Rubin FP4 GEMM deep dive" §3.2, §4.2): v = acc x tsA x
    // tsB (+ bias[column]) (ReLU: v > 0 ? v : +0), each step one FP32
    // rounding, then FP32, BF16 (round to nearest even) or FP4 (OUT 2/3:
    // MXFP4 along N, ceil / OCP scale rule).  Lane L of a 32x32 block holds
    // column L%32, rows 8*(i/4) + 4*(L/32) + i%4.
    const bool use_bias = EPI && bias != nullptr, use_act = EPI && act != 0u;
    float bcol[2] = {0.0f, 0.0f};
    if (use_bias) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t col = cur.n0 + 64u * wn + 32u * c + li;
        bcol[c] = col < N ? bias[col] : 0.0f;
      }
    }
    // Grouped NVFP4: each expert's weights carry their own tensor scale.
    float tile_scale = scale;
    if constexpr (GROUPED && FMT == kFmtNV) tile_scale = sload(tsA) * sload(tsB + cur.expert);
    auto epi = [&](float a, int c) {
      float v = a * tile_scale;
      if (use_bias) v = v + bcol[c];
      if (use_act) v = v > 0.0f ? v : 0.0f;
      return v;
    };
    if constexpr (!PERSIST) {
      // One tile per workgroup: the tile goes through LDS (free once every wave is
      // past its last stage) so that global stores are 16-byte, row-contiguous;
      // BF16 in one pass, FP32 in two passes of 128 rows.  A row pitch of C
      // that is not a multiple of 16 bytes, or an unaligned C, takes
      // per-element stores.
      constexpr uint32_t EB = OUT == 1 ? 2u : 4u;              // bytes per staged element
      constexpr uint32_t PASS_ROWS = OUT == 1 ? 256u : 128u;    // tile rows per pass
      constexpr uint32_t LROW = BN * EB + 16u;                  // LDS row pitch (bank shift of 4 per row)
      static_assert(PASS_ROWS * LROW <= NSTAGE * STAGE_BYTES, "epilogue tile must fit in LDS");
      // FP4 output: N % 32 == 0 and a 16-byte aligned C are required.
      const bool vec_ok =
          OUT >= 2 || (((N * EB) % 16u == 0u) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0u));
      const size_t crow0 = (size_t)cur.row0 + cur.m0;
      // The last iterations' zero-fill copies must have landed before LDS is
      // reused.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (vec_ok) {
        __syncthreads();
#pragma unroll
        for (uint32_t pass = 0; pass < 256u / PASS_ROWS; ++pass) {
          if (PASS_ROWS == 256u || wm == pass) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const uint32_t lcol = 64u * wn + 32u * c + li;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const uint32_t lrow =
                      (PASS_ROWS == 256u ? 128u * wm : 0u) + 32u * r + 8u * (i >> 2) + 4u * lj + (i & 3);
                  const float val = epi(acc[r][c][i], c);
                  if (OUT != 1)
                    *reinterpret_cast<float*>(lds + lrow * LROW + 4u * lcol) = val;
                  else
                    *reinterpret_cast<uint16_t*>(lds + lrow * LROW + 2u * lcol) = f32_to_bf16(val);
                }
              }
          }
          __syncthreads();
          if constexpr (OUT == 4) {
            // NVFP4 along N under the caller's tensor scale s_c (NVFP4 video
            // transcript: 16-value blocks, E4M3 block scale, FP32 tensor
            // scale; the deep dive §3.2 converts C to FP4 when asked), as
            // fp4_quantize with a given tensor scale does for a rows x N
            // matrix.  Item (row, j): 32-column chunks j, 2+j, 4+j, 6+j, two
            // 16-blocks each, whose eight scale bytes are the two dwords of
            // scale-tile lane 32j + row%32 (bytes 2s, 2s+1: chunk 2s + j).
            // Rows past M and blocks past N get scale byte 0 (the tiles'
            // padding) and no codes.
            const float s_c = *tsC;
            const uint32_t t = threadIdx.x;
            if (t < 256u) {
              const uint32_t lrow = t >> 1, j = t & 1u;
              const uint32_t row = pass * 128u + lrow;
              const uint32_t grow = cur.m0 + row;
              const bool row_in = row < cur.rowsA;
              uint32_t dw[2] = {0u, 0u};
#pragma unroll 1
              for (uint32_t sq = 0; sq < 4u; ++sq) {
                const uint32_t chunk = 2u * sq + j, col0 = cur.n0 + 32u * chunk;
                const bool blk_in = row_in && col0 < N;
                float v[32];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                  const v4i w4 = *reinterpret_cast<const v4i*>(lds + lrow * LROW + 128u * chunk + 16u * (uint32_t)q);
#pragma unroll
                  for (int e = 0; e < 4; ++e) v[4 * q + e] = u2f((uint32_t)w4[e]);
                }
                v4i cw;
                uint32_t pair = 0u;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  float* x = v + 16 * h;
                  float am = 0.0f;
#pragma unroll
                  for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(x[e]));
                  const uint32_t sb = blk_in ? e4m3_encode((am / 6.0f) / s_c) : 0u;
                  if (sb == 0u) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) x[e] = __builtin_copysignf(0.0f, x[e]);   // x / inf
                  } else {
                    const float d = e4m3_value(sb) * s_c;
                    const float rd = 1.0f / d;
#pragma unroll
                    for (int e = 0; e < 16; ++e) x[e] = nv_div(x[e], d, rd);
                  }
                  cw[2 * h] = (int)pack8(x);
                  cw[2 * h + 1] = (int)pack8(x + 8);
                  pair |= sb << (8 * h);
                }
                if (blk_in)
                  *reinterpret_cast<v4i*>(static_cast<uint8_t*>(C) + (size_t)grow * (N / 2u) + col0 / 2u) = cw;
                dw[sq >> 1] |= pair << (16u * (sq & 1u));
              }
              const uint32_t rows_pad = (M + 31u) & ~31u;
              if (grow < rows_pad) {
                const uint32_t KTo = (N + 255u) / 256u;
                const size_t off = ((size_t)(grow >> 5) * KTo + cur.n0 / 256u) * 512u + (32u * j + (grow & 31u)) * 8u;
                *reinterpret_cast<u32x2*>(Cs + off) = u32x2{dw[0], dw[1]};
              }
            }
            __syncthreads();
            continue;
          } else if constexpr (OUT >= 2) {
            // Re-quantise the pass's 128 rows x 8 blocks of 32 columns
            // (MXFP4 along N, as fp4_quantize does for a rows x N matrix).
            // Item (row, j): blocks j, 2+j, 4+j, 6+j, whose scale bytes form
            // the dword of scale-tile lane 32j + row%32.  Rows past M and
            // blocks past N get scale byte 0 (the tiles' padding) and no codes.
            constexpr int FMTO = OUT == 2 ? kFmtMX : kFmtMXOcp;
            const uint32_t t = threadIdx.x;
            if (t < 256u) {
              const uint32_t lrow = t >> 1, j = t & 1u;
              const uint32_t row = pass * 128u + lrow;
              const uint32_t grow = cur.m0 + row;
              const bool row_in = row < cur.rowsA;
              uint32_t dw = 0u;
#pragma unroll 1
              for (uint32_t sq = 0; sq < 4u; ++sq) {
                const uint32_t blk = 2u * sq + j, col0 = cur.n0 + 32u * blk;
                const bool blk_in = row_in && col0 < N;
                float v[32];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                  const v4i w4 = *reinterpret_cast<const v4i*>(lds + lrow * LROW + 128u * blk + 16u * (uint32_t)q);
#pragma unroll
                  for (int e = 0; e < 4; ++e) v[4 * q + e] = u2f((uint32_t)w4[e]);
                }
                float am = 0.0f;
#pragma unroll
                for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(v[e]));
                const uint32_t sbyte = blk_in ? mx_scale_byte<FMTO>(am) : 0u;
                if (blk_in) {
                  // x * 2^-e, exact: 2^(127 - e) is a normal float for bytes 0..253.
                  const float inv = u2f((254u - sbyte) << 23);
                  v4i cw;
#pragma unroll
                  for (int q = 0; q < 4; ++q) {
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = v[8 * q + e] * inv;
                    cw[q] = (int)pack8(y);
                  }
                  *reinterpret_cast<v4i*>(static_cast<uint8_t*>(C) + (size_t)grow * (N / 2u) + col0 / 2u) = cw;
                }
                dw |= sbyte << (8u * sq);
              }
              const uint32_t rows_pad = (M + 31u) & ~31u;
              if (grow < rows_pad) {
                const uint32_t KTo = (N + 255u) / 256u;
                const size_t off = ((size_t)(grow >> 5) * KTo + cur.n0 / 256u) * 256u + (32u * j + (grow & 31u)) * 4u;
                *reinterpret_cast<uint32_t*>(Cs + off) = dw;
              }
            }
            __syncthreads();
            continue;
          }
          // 16-byte chunks: BN * EB / 16 per row; 512 threads cover 512 chunks per step.
          constexpr uint32_t CPR = BN * EB / 16u;
          constexpr uint32_t STEPS = PASS_ROWS * CPR / 512u;
#pragma unroll
          for (uint32_t st = 0; st < STEPS; ++st) {
            const uint32_t q = st * 512u + threadIdx.x;
            const uint32_t lrow = q / CPR, ch = q % CPR;
            const uint32_t row = pass * PASS_ROWS + lrow;
            const uint32_t col = cur.n0 + ch * (16u / EB);
            // N * EB is a multiple of 16 and col a multiple of 16 / EB, so a
            // chunk that starts inside the row lies wholly inside it.
            if (row < cur.rowsA && col < N)
              *reinterpret_cast<v4i*>(static_cast<uint8_t*>(C) + ((crow0 + row) * N + col) * EB) =
                  *reinterpret_cast<const v4i*>(lds + lrow * LROW + 16u * ch);
          }
          if (PASS_ROWS != 256u) __syncthreads();
        }
        break;
      }
    }
    // Stores straight from registers (LDS may hold the next tile's first
    // stages, or C's layout does not allow 16-byte stores).  One per-lane base per
    // tile plus uniform row offsets (from an opaque N, so that they are not
    // hoisted out of the tile loop into registers).
    if constexpr (OUT < 2) {
      const uint32_t Nu = opaque(N);
      const uint32_t lrow0 = 128u * wm + 4u * lj;                 // this lane's first row in the tile
      const uint32_t lcol0 = cur.n0 + 64u * wn + li;              // this lane's first column
      const size_t lbase = ((size_t)cur.row0 + cur.m0 + lrow0) * Nu + lcol0;
      auto store = [&](int r, int i, int c) {
        const uint32_t rr = 32u * r + 8u * (i >> 2) + (i & 3);  // row offset from lrow0
        const float val = epi(acc[r][c][i], c);
        const size_t e = lbase + (size_t)rr * Nu + 32u * c;
        if (OUT == 0)
          static_cast<float*>(C)[e] = val;
        else
          static_cast<uint16_t*>(C)[e] = f32_to_bf16(val);
      };
      // A whole tile stores without per-element masks: a masked store is a
      // branch of its own (exec mask saved, tested and restored), and those
      // made up most of the epilogue's instructions.
      if (cur.rowsA == BM && cur.n0 + BN <= N) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int c = 0; c < 2; ++c) store(r, i, c);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // Grouped: 32-row blocks past the group's rows store nothing (a
          // uniform test instead of 32 masked stores).
          if (GROUPED && 128u * wm + 32u * (uint32_t)r >= cur.rowsA) continue;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t rr = 32u * r + 8u * (i >> 2) + (i & 3);
            const bool row_ok = lrow0 + rr < cur.rowsA;
#pragma unroll
            for (int c = 0; c < 2; ++c)
              if (row_ok && lcol0 + 32u * c < N) store(r, i, c);
          }
        }
      }
    }
    if (!has_next) break;
    cur = nxt;
    v = vn;
    g += KT;
  }
  // No copy into LDS may still be in flight when the workgroup's LDS is
  // released (the zero-fill copies of the last iterations).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// out: 0 FP32, 1 BF16, 2 MXFP4 (ceil rule), 3 MXFP4 (OCP rule), 4 NVFP4 (given
// tensor scale); FP4 output only with one tile per workgroup.
template <int FMT, bool GROUPED, bool PERSIST, bool EPI>
hipError_t launch(dim3 grid, int out, const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                  const float* tsA, const float* tsB, void* C, uint32_t M, uint32_t N, uint32_t K, uint32_t tilesM,
                  uint32_t tilesN, const Groups& gp, const float* bias, uint32_t act, uint8_t* Cs,
                  const float* tsC, hipStream_t stream) {
#define GEMM_LAUNCH(O)                                                                                           \
  gemm_kernel<FMT, O, GROUPED, PERSIST, EPI><<<grid, dim3(512), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, M, N, K, tilesM, \
                                                                        tilesN, gp, bias, act, Cs, tsC)
  if (out == 0)
    GEMM_LAUNCH(0);
  else if (out == 1)
    GEMM_LAUNCH(1);
  else if constexpr (!PERSIST && !GROUPED && EPI) {
    if (out == 2)
      GEMM_LAUNCH(2);
    else if (out == 3)
      GEMM_LAUNCH(3);
    else
      GEMM_LAUNCH(4);
  } else {
    return hipErrorInvalidValue;
  }
#undef GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

// Workgroups that a persistent launch keeps resident: one per compute unit
// (a multiple of 8, so that each workgroup stays on one XCD).  Cached per
// device; the value never changes, so concurrent first calls are harmless.
static uint32_t resident_workgroups() {
  static std::atomic<uint32_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256u;
  uint32_t n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0u) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
    n = (uint32_t)cus / 8u * 8u;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Grid for `tiles` tiles of K/256 stages: every tile its own workgroup when
// there is a single stage (nothing to overlap) or when not `persistent`, else
// at most one resident wave of workgroups that walk the tiles (a persistent
// kernel given one workgroup per tile finds no next tile and stops after one).  Measured:
// walking the tiles (the next tile's first stages copied during this one's
// last iterations, C stored from registers) helps the NVFP4 GEMM (4096 x
// 14336 x 4096: +5%) and the grouped GEMM (MoE: +8%); the dense MXFP4 GEMM is
// faster one tile per workgroup with C stored through LDS (8192^3: 3709 vs
// 3670 TFLOP/s).
static uint32_t tiled_grid(uint64_t tiles, int64_t K, bool persistent) {
  const uint64_t KT = (uint64_t)((K + 255) / 256);
  if (KT < 2u || !persistent) return (uint32_t)tiles;
  const uint64_t g = resident_workgroups();
  return (uint32_t)(tiles < g ? tiles : g);
}

hipError_t launch_gemm_ex(int fmt, const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, const float* bias, int act, void* C, uint8_t* Cs,
                          const float* tsC, int64_t M, int64_t N, int64_t K, int out, hipStream_t stream) {
  const uint32_t tilesM = (uint32_t)((M + BM - 1) / BM), tilesN = (uint32_t)((N + BN - 1) / BN);
  const Groups none{nullptr, nullptr, 0, 0, 0, 0};
  const uint32_t m = (uint32_t)M, n = (uint32_t)N, k = (uint32_t)K, a = (uint32_t)act;
  const bool epi = bias != nullptr || act != 0 || out >= 2;
  // NVFP4 walks tiles persistently, except with FP4 output (LDS epilogue).
  if (fmt == kFmtNV && out < 2) {
    const dim3 pgrid(tiled_grid((uint64_t)tilesM * tilesN, K, true));
    if (epi)
      return launch<kFmtNV, false, true, true>(pgrid, out, A, sA, B, sB, tsA, tsB, C, m, n, k, tilesM, tilesN, none,
                                               bias, a, Cs, nullptr, stream);
    return launch<kFmtNV, false, true, false>(pgrid, out, A, sA, B, sB, tsA, tsB, C, m, n, k, tilesM, tilesN, none,
                                              nullptr, 0u, nullptr, nullptr, stream);
  }
  const dim3 grid(tilesM * tilesN);
  if (fmt == kFmtNV)   // FP4 output
    return launch<kFmtNV, false, false, true>(grid, out, A, sA, B, sB, tsA, tsB, C, m, n, k, tilesM, tilesN, none,
                                              bias, a, Cs, tsC, stream);
  if (epi)
    return launch<kFmtMX, false, false, true>(grid, out, A, sA, B, sB, tsA, tsB, C, m, n, k, tilesM, tilesN, none,
                                              bias, a, Cs, tsC, stream);
  return launch<kFmtMX, false, false, false>(grid, out, A, sA, B, sB, tsA, tsB, C, m, n, k, tilesM, tilesN, none,
                                             nullptr, 0u, nullptr, nullptr, stream);
}

hipError_t launch_gemm_tiled(int fmt, const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                             const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                             int out_dtype, hipStream_t stream) {
  return launch_gemm_ex(fmt, A, sA, B, sB, tsA, tsB, nullptr, 0, C, nullptr, nullptr, M, N, K, out_dtype, stream);
}

namespace {

// Token rows gathered into output-row order (the grouped GEMM's optional
// pre-pass): row r of (Ag, sAg) = row row_idx[r] of (A, sA), codes and scale
// entries (ENT bytes: 4 for MXFP4; 8 would serve NVFP4), in the same tiled
// layout.
// One wave per row of the 32-row-padded output; padding rows get zero scale
// entries and no codes.  Reads go through buffer ranges (an index outside A
// reads zeros).
template <uint32_t ENT>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
                                                          uint32_t A_rows, const int32_t* __restrict__ row_idx,
                                                          uint32_t total, uint32_t K, uint8_t* __restrict__ Ag,
                                                          uint8_t* __restrict__ sAg) {
  constexpr uint32_t STILE = 64u * ENT;            // 32 rows x 2 entries of ENT bytes
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t r = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t total_pad = (total + 31u) & ~31u;
  if (r >= total_pad) return;
  const bool live = r < total;
  const uint32_t ldb = K / 2u, KT = (K + 255u) / 256u;
  const int32_t si = live ? row_idx[r] : 0;
  const uint32_t src = (uint32_t)si;
  const bool ok = live && si >= 0 && src < A_rows;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, A_rows * ldb);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(sA, ((A_rows + 31u) / 32u) * KT * STILE);
  if (live) {
    for (uint32_t off = 16u * lane; off < ldb; off += 1024u) {
      const v4i c = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? src * ldb + off : 0x80000000u, 0, 0));
      *reinterpret_cast<v4i*>(Ag + (size_t)r * ldb + off) = c;
    }
  }
  for (uint32_t e = lane; e < 2u * KT; e += 64u) {
    const uint32_t kt = e >> 1, j = e & 1u;
    const uint32_t so = ((src >> 5) * KT + kt) * STILE + (32u * j + (src & 31u)) * ENT;
    uint8_t* dst = sAg + ((size_t)(r >> 5) * KT + kt) * STILE + (32u * j + (r & 31u)) * ENT;
    if (ENT == 4u) {
      *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? so : 0x80000000u, 0, 0);
    } else {
      *reinterpret_cast<u32x2*>(dst) =
          __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, ok ? so : 0x80000000u, 0, 0));
    }
  }
}

// Bytes of the gathered codes (padded to 256) and of their scale tiles.
size_t gathered_code_bytes(int64_t total_rows, int64_t K) {
  return ((size_t)total_rows * (size_t)(K / 2) + 255u) & ~(size_t)255u;
}
size_t gathered_scale_bytes(int fmt, int64_t total_rows, int64_t K) {
  return (size_t)((total_rows + 31) / 32) * (size_t)((K + 255) / 256) * (fmt == kFmtNV ? 512u : 256u);
}

}  // namespace

// MXFP4 only: the NVFP4 GEMM's stages are long enough (FP16 matrix core) to
// hide the gathered rows' latency, and there the copy cost more than it saved
// (MoE step 1.97-1.99 -> 1.99-2.01 ms, against 0.82-0.83 -> 0.78-0.79 ms for
// MXFP4).
size_t gemm_grouped_workspace(int fmt, int64_t total_rows, int64_t, int64_t K, int32_t) {
  if (fmt == kFmtNV) return 0;
  return gathered_code_bytes(total_rows, K) + gathered_scale_bytes(fmt, total_rows, K);
}

bool gemm_grouped_supports(int) { return true; }

hipError_t launch_gemm_grouped(const uint8_t* A, const uint8_t* sA, int64_t A_rows, const int32_t* row_idx,
                               const int32_t* group_off, int32_t E, const uint8_t* B, const uint8_t* sB,
                               const float* tsA, const float* tsB, void* C, int64_t total_rows, int64_t N,
                               int64_t K, int fmt, int out_dtype, void* workspace, hipStream_t stream) {
  const uint32_t tilesN = (uint32_t)((N + BN - 1) / BN);
  // With a workspace: gather the token rows into output-row order first, so
  // that the GEMM reads contiguous rows (a tile's scale entries then come
  // from whole 32-row tiles instead of one scale tile per gathered row).
  if (workspace != nullptr && total_rows > 0 && fmt != kFmtNV) {
    uint8_t* Ag = static_cast<uint8_t*>(workspace);
    uint8_t* sAg = Ag + gathered_code_bytes(total_rows, K);
    const uint32_t total_pad = (uint32_t)((total_rows + 31) / 32 * 32);
    const dim3 ggrid((total_pad + 3u) / 4u);
    gather_rows_kernel<4u><<<ggrid, dim3(256), 0, stream>>>(A, sA, (uint32_t)A_rows, row_idx, (uint32_t)total_rows,
                                                             (uint32_t)K, Ag, sAg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    A = Ag;
    sA = sAg;
    A_rows = total_rows;
    row_idx = nullptr;
  }
  // Upper bound on the tile count (each expert rounds up at most once), a
  // multiple of 8 so the XCD-contiguous order covers every tile; workgroups
  // past the real count return at once.
  const uint64_t max_tiles = ((uint64_t)(total_rows + BM - 1) / BM + (uint64_t)E) * tilesN;
  const uint64_t grid = tiled_grid((max_tiles + 7) / 8 * 8, K, true);
  const uint32_t KT = (uint32_t)((K + 255) / 256);
  const size_t scale_stride = (size_t)((N + 31) / 32) * KT * (fmt == kFmtNV ? 512u : 256u);
  const Groups gp{row_idx, group_off, E, (uint32_t)A_rows, (size_t)N * (size_t)(K / 2), scale_stride};
  if (fmt == kFmtNV)   // tsB: one tensor scale per expert
    return launch<kFmtNV, true, true, false>(dim3((uint32_t)grid), out_dtype, A, sA, B, sB, tsA, tsB, C,
                                             (uint32_t)total_rows, (uint32_t)N, (uint32_t)K, 0, tilesN, gp, nullptr,
                                             0u, nullptr, nullptr, stream);
  return launch<kFmtMX, true, true, false>(dim3((uint32_t)grid), out_dtype, A, sA, B, sB, tsA, tsB, C, (uint32_t)total_rows,
                                    (uint32_t)N, (uint32_t)K, 0, tilesN, gp, nullptr, 0u, nullptr, nullptr,
                                    stream);
}

}  // namespace fp4
