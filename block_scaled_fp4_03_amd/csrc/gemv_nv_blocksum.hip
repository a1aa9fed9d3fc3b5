// gemv_nv_blocksum.hip -- NVFP4 decode GEMV for M <= 8 activation rows
// (gfx950): the FP4 x FP4 matrix core forms the exact dot product of every
// pair of 16-value blocks, and the two E4M3 block scales multiply those block
// sums in FP32.
//
//   C[m,n] = tsA tsW sum_b sA[m,b] sW[n,b] (sum_{k in b} e2m1(A[m,k]) e2m1(W[n,k]))
//
// (NVFP4 video transcript: 16-value blocks, E4M3 block scale, one FP32 tensor
// scale; "Rubin FP4 GEMM deep dive" §1.2, §6.2: decoding streams every weight
// once, so the kernel is built around the HBM stream.)
//
// Why a second decode kernel.  gfx950's scaled matrix core takes power-of-two
// scales per 32 values, not E4M3 scales per 16, so gemv_nv.hip decodes every
// weight to FP16 first -- about one vector instruction per weight, which made
// it compute-bound at small M.  Here the weights go to the FP4 x FP4 matrix
// core as stored (unit E8M0 scales), and the activation operand is block-
// diagonal: operand row r carries one 16-value block of one activation row and
// zeros elsewhere, so accumulator row r of weight row n receives exactly that
// block pair's dot product.  E2M1 x E2M1 products are multiples of 1/4 of
// magnitude at most 36, so a block sum (at most 576) is exact in FP32.  Each
// block sum is then multiplied by sW[n,b] * sA[m,b] (a product of two E4M3
// values: at most 8 significant bits, exact) and added to a per-lane FP32 sum.
//
// Operand rows and accumulator registers.  In the 32x32 accumulator, lane
// L = 32h + n holds column n (weight row n of the 32-row block) and rows
// 8(q/4) + 4h + q%4 in its registers q = 0..15.  Register q of lane (h, n)
// takes activation row m = q / (16/MB), K step g' = (q % (16/MB)) / 2 of a
// window of 8/MB steps, and, in step g (64 values), the block 4g + 2h + q%2:
// the block whose scale byte lane (h, n) holds in the tiled scale layout and
// whose codes sit in K half h of the lane's weight operand.  A window fills
// each register once; MB (1, 2, 4, 8 >= M) activation rows share the 32
// operand rows, and the matrix core's spare rate covers the zero rows.
//
// Work split.  Workgroup = 16 wavefronts = one 32-row block of W over all of K
// (further row blocks in a grid-stride loop); wave w takes the 512-value units
// u = w, w + 16, ... .  Per unit a lane (h, n) loads 8 x 16 bytes of weight row
// n (bytes 256u + 32g + 16h: step g's K half h) and its 8 scale bytes in each
// of the tiles 2u and 2u + 1.  When step g of a unit has gone to the matrix
// core, the same registers receive step g of the wave's next unit, so the
// weights stream without a pause.  The activation is staged in LDS (by each
// wave for the units it reads, or, when X is quantised in the kernel, by the
// whole workgroup) as 16-byte operand slots (a block's 8 code bytes in the
// half of the slot its K half needs, zeros in the other) plus its block
// scales in FP32.  The 16 waves' sums are added in a fixed order through LDS
// at the end of each row block: the result is deterministic, and the fused
// path (X quantised in the kernel) stages the same values as fp4_quantize, so
// both calls return the same bits.
#include <float.h>

#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

typedef float v2f __attribute__((ext_vector_type(2)));

constexpr uint32_t BS_WAVES = 16;
constexpr uint32_t BS_LDS_BYTES = 160u * 1024u;
// Weight steps requested before the activation is staged (4 of 8).
#ifndef BS_HOLD
#define BS_HOLD 4
#endif

template <int MB>
struct BsGeom {
  static constexpr uint32_t WN = 8u / MB;              // steps per window
  static constexpr uint32_t QPM = 16u / MB;            // registers per activation row
  static constexpr uint32_t ZSLOT = 32u * MB * 16u;    // the unit's all-zero slot
  static constexpr uint32_t SA_OFF = ZSLOT + 16u;      // FP32 block scales [h][g][e][m]
  static constexpr uint32_t UNIT_BYTES = SA_OFF + 32u * MB * 4u;
  static constexpr uint32_t RED_BYTES = BS_WAVES * MB * 32u * 4u;
  static constexpr int XNB = MB >= 4 ? 4 : 2;          // fused: 16-value X blocks per thread (at most)
  static constexpr int NH = 2 * XNB;                   // fused: 8-value half blocks per thread
  static constexpr int NA = XNB / 2;                   // codes: 32-value chunks per thread
};

// HP: weight steps requested before the activation is staged (the rest
// right after), so that the activation's round trip does not queue behind
// the whole weight stream.
template <int MB, bool FUSED, int OUT, int XDT, int HP>
__global__ __launch_bounds__(BS_WAVES * 64, 1) void gemv_bs_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const uint8_t* __restrict__ W,
    const uint8_t* __restrict__ sW, const float* __restrict__ tsA, const float* __restrict__ tsW, void* __restrict__ C,
    uint32_t M, uint32_t N, uint32_t K, const void* __restrict__ X, float* __restrict__ ts_out, uint32_t flags) {
  using G = BsGeom<MB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[BS_LDS_BYTES];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t n = lane & 31u, h = lane >> 5;
  const uint32_t KT = (K + 255u) / 256u;                 // scale tiles per 32-row block
  const uint32_t NU = (K + 511u) / 512u;                 // units per row
  const uint32_t NJ = NU > BS_WAVES ? (NU + BS_WAVES - 1u) / BS_WAVES : 1u;   // units per wave per row block
  const uint32_t ldb = K / 2u, srow = KT * 512u, nb = K / 16u;
  const uint32_t nblocks = (N + 31u) / 32u;
  const uint32_t nrb = (nblocks - blockIdx.x + gridDim.x - 1u) / gridDim.x;    // row blocks of this workgroup
  const uint32_t T = NJ * nrb;                           // work items of this wave
  const uint32_t bpr = NU * 32u;                         // staged blocks per activation row
  float* red = reinterpret_cast<float*>(lds + NU * G::UNIT_BYTES);   // [wave][m][n]
  // FP32 activation block scale of unit-local block bl = 4g + 2h + e, row m:
  // stored [h][g][e][m], so that a window's 16 values for one K half are
  // contiguous.
  auto sa_index = [](uint32_t bl, uint32_t m) {
    return ((((bl >> 1) & 1u) * 8u + (bl >> 2)) * 2u + (bl & 1u)) * MB + m;
  };

  // ---- activation loads (first: the waits for them then count past the weights')
  constexpr uint32_t XEB = XDT == kDtBF16 ? 2u : 4u;     // bytes per X value
  constexpr int NX = FUSED ? G::NH : 1;
  constexpr int NXL = FUSED ? (int)XEB / 2 : 1;          // 16-byte loads per half block
  constexpr int NC = FUSED ? 1 : G::NA;
  v4i xl[NX][NXL];
  v4i ald[NC];
  uint32_t asc[NC];
  // Codes: each wave stages the units it reads (u = wave + 16 j), so that it
  // starts without waiting for the rest of the workgroup.  Its chunk q =
  // lane + 64 i is 32 values (blocks 2cu, 2cu + 1) of row m of unit u:
  // j = q / 16MB, then m = q % MB, cu = 16 u + (q % 16MB) / MB.
  auto own_chunk = [&](int i, uint32_t& m, uint32_t& cu) {
    const uint32_t q = lane + 64u * (uint32_t)i, j = q / (16u * MB), r = q % (16u * MB);
    m = r % MB;
    cu = 16u * (wave + BS_WAVES * j) + r / MB;
    return j < NJ;
  };
  if (!FUSED) {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, M * ldb);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sA, srow);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      uint32_t m, cu;
      const bool mine = own_chunk(i, m, cu);
      const bool ok = mine && m < M && 32u * cu < K;
      ald[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? m * ldb + 16u * cu : 0x80000000u,
                                                                            0, 0));
      asc[i] = __builtin_amdgcn_raw_buffer_load_b16(rsa, ok ? scale_offset<kFmtNV>(m, 2u * cu, KT) : 0x80000000u, 0, 0);
    }
  } else {
    // Half block hb = 8 values (half hb % 2 of block b = hb / 2, so that a
    // block's halves sit in adjacent lanes): row m = b % MB, block bk = b / MB.
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, M * K * XEB);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const uint32_t hb = tid + 1024u * i, b = hb >> 1;
      const uint32_t m = b % MB, bk = b / MB;
      const bool ok = m < M && bk < nb;
#pragma unroll
      for (int l = 0; l < NXL; ++l)
        xl[i][l] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(
                     rx, ok ? (m * K + 16u * bk + 8u * (hb & 1u)) * XEB + 16u * l : 0x80000000u, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- weight ring prologue.  Work item j of this wave is unit
  // u = wave + 16 (j % NJ) of row block blockIdx.x + (j / NJ) gridDim.x.  Past
  // the last item (or unit) the offsets are out of range: the loads return
  // zeros without touching memory, and every iteration issues the same loads
  // into the same registers.
  struct Src {
    __amdgpu_buffer_rsrc_t rw, rsw;
    uint32_t off;    // this lane's code offset of step 0
    uint32_t soff;   // this lane's scale offset in tile 2u
  };
  auto src = [&](uint32_t j) {
    const uint32_t rb = blockIdx.x + (j / NJ) * gridDim.x;
    const uint32_t u = wave + BS_WAVES * (j % NJ);
    const uint32_t n0 = rb * 32u;
    const bool item = j < T;
    const uint32_t rows = __builtin_amdgcn_readfirstlane(item ? (N - n0 < 32u ? N - n0 : 32u) : 0u);
    Src t;
    t.rw = make_rsrc(W + (size_t)n0 * ldb, rows * ldb);
    t.rsw = make_rsrc(sW + (size_t)rb * srow, item ? srow : 0u);
    const bool ok = item && u < NU;
    t.off = ok ? n * ldb + 256u * u + 16u * h : 0x80000000u;
    t.soff = ok ? 1024u * u + 8u * lane : 0x80000000u;
    return t;
  };
  auto load_code = [&](const Src& t, int g) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(t.rw, t.off + 32u * (uint32_t)g, 0, 0));
  };
  auto load_scale = [&](const Src& t, int tile) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(t.rsw, t.soff + 512u * (uint32_t)tile, 0, 0));
  };
  v4i wc[8];
  u32x2 ws[2];
  {
    const Src t0 = src(0);
    ws[0] = load_scale(t0, 0);   // scales first, as in the loop
    ws[1] = load_scale(t0, 1);
#pragma unroll
    for (int g = 0; g < HP; ++g) wc[g] = load_code(t0, g);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- activation -> LDS operand slots and FP32 block scales
  float s_x = 1.0f;   // activation tensor scale (fused)
  if (!FUSED) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      uint32_t m, cu;
      if (own_chunk(i, m, cu) && cu < NU * 16u) {
        const uint32_t u = cu >> 4, bl = 2u * (cu & 15u);
        uint8_t* ub = lds + u * G::UNIT_BYTES;
        *reinterpret_cast<v4i*>(ub + (bl * MB + m) * 16u) = v4i{ald[i][0], ald[i][1], 0, 0};
        *reinterpret_cast<v4i*>(ub + ((bl + 1u) * MB + m) * 16u) = v4i{0, 0, ald[i][2], ald[i][3]};
        const v2f s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(asc[i], 1.0f, false);
        float* sa = reinterpret_cast<float*>(ub + G::SA_OFF) + sa_index(bl, m);
        sa[0] = s[0];
        sa[MB] = s[1];
      }
    }
  } else {
    float xv[NX][8];
#pragma unroll
    for (int i = 0; i < NX; ++i)
#pragma unroll
      for (int l = 0; l < NXL; ++l)
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
    // Each half block's largest magnitude, then the block's (the partner
    // lane's half), in every lane.
    float am[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(xv[i][e]));
      am[i] = fmaxf(a, lane_xor1(a));
    }
    // Tensor scale (NVFP4 video transcript: one FP32 scale for the global
    // range): amax / (6 * 448), 1 for an all-zero X, at least FLT_MIN; or the
    // caller's.  Each workgroup reduces the whole of X itself.
    if (flags & 1u) {
      s_x = *tsA;
    } else {
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < NX; ++i) mx = fmaxf(mx, am[i]);
      mx = wave_fmax(mx);
      if (lane == 0) red[wave] = mx;
      __syncthreads();
      float amax = 0.0f;
#pragma unroll
      for (uint32_t w = 0; w < BS_WAVES; w += 4u) {
        const v4f r = *reinterpret_cast<const v4f*>(red + w);
        amax = fmaxf(fmaxf(amax, fmaxf(r[0], r[1])), fmaxf(r[2], r[3]));
      }
      if (amax > 0.0f) {
        s_x = amax / 2688.0f;
        if (s_x < FLT_MIN) s_x = FLT_MIN;
      }
      if (blockIdx.x == 0 && tid == 0 && ts_out) *ts_out = s_x;
    }
    // Quantise each half block exactly as the quantiser does its block (same
    // codes, zero signs included, and the same E4M3 scale byte).
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const uint32_t hb = tid + 1024u * i, b = hb >> 1, half = hb & 1u;
      const uint32_t m = b % MB, bk = b / MB;
      if (bk < bpr) {
        uint32_t c = 0u;
        float sv = 0.0f;
        if (m < M && bk < nb) {
          const uint32_t sb = e4m3_encode((am[i] / 6.0f) / s_x);
          float y[8];
          if (sb == 0u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = __builtin_copysignf(0.0f, xv[i][e]);   // x / inf
          } else {
            const float d = e4m3_value(sb) * s_x;
            const float rd = 1.0f / d;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = nv_div(xv[i][e], d, rd);
          }
          c = pack8(y);
          sv = e4m3_value(sb);
        }
        // The block's 8 code bytes fill half (bl % 2) of its slot, zeros the other.
        const uint32_t u = bk >> 5, bl = bk & 31u;
        uint8_t* ub = lds + u * G::UNIT_BYTES;
        uint32_t* slot = reinterpret_cast<uint32_t*>(ub + (bl * MB + m) * 16u);
        slot[2u * (bl & 1u) + half] = c;
        slot[2u * (~bl & 1u) + half] = 0u;
        if (half == 0u) reinterpret_cast<float*>(ub + G::SA_OFF)[sa_index(bl, m)] = sv;
      }
    }
  }
  if (FUSED) {
    if (tid < NU) *reinterpret_cast<v4i*>(lds + tid * G::UNIT_BYTES + G::ZSLOT) = v4i{};
    __syncthreads();
  } else if (lane < NJ && wave + BS_WAVES * lane < NU) {
    // this wave's units' zero slots (LDS operations of one wave complete in
    // order: its own reads below see them)
    *reinterpret_cast<v4i*>(lds + (wave + BS_WAVES * lane) * G::UNIT_BYTES + G::ZSLOT) = v4i{};
  }
  // The rest of the first unit's weight steps, requested once the
  // activation is staged (codes: this wave's units).  Requested earlier, they queue behind
  // the whole grid's weight stream and delay the activation's own loads (at
  // 8192 x 8192, M = 1: all 8 steps first 10.3 us, 4 first 9.7 us; waves that
  // request the rest as soon as their own share has arrived 10.4 us).
  if (HP < 8) {
    const Src t0 = src(0);
#pragma unroll
    for (int g = HP; g < 8; ++g) wc[g] = load_code(t0, g);
  }

  // ---- this lane's operand slot: A row r = n of K half j = h carries
  // register q(r) = 4(r/8) + r%4 of accumulator half (r/4)%2, live in window
  // step g_r of each window (dead lanes read the zero slot).
  const uint32_t hr = (n >> 2) & 1u, q_r = ((n >> 3) << 2) | (n & 3u);
  const uint32_t m_r = q_r / G::QPM, g_r = (q_r % G::QPM) >> 1, e_r = q_r & 1u;
  const bool a_live = h == hr && m_r < M;
  const uint32_t slot0 = a_live ? ((4u * g_r + 2u * h + e_r) * MB + m_r) * 16u : G::ZSLOT;
  const uint32_t slot_step = a_live ? 4u * G::WN * MB * 16u : 0u;   // per window

  // ---- main loop
  const float scale = (FUSED ? s_x : *tsA) * *tsW;
  float part[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) part[m] = 0.0f;

  for (uint32_t j = 0; j < T; ++j) {
    const uint32_t u = wave + BS_WAVES * (j % NJ);
    const Src tn = src(j + 1u);
    // The unit's weight scales in FP32, [step][block of the lane's K half],
    // converted before their registers take item j + 1's.
    v2f swf[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        swf[4 * t + 2 * d] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ws[t][d], 1.0f, false);
        swf[4 * t + 2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ws[t][d], 1.0f, true);
      }
    asm volatile("" : : "v"(swf[0]), "v"(swf[1]), "v"(swf[2]), "v"(swf[3]), "v"(swf[4]), "v"(swf[5]), "v"(swf[6]),
                 "v"(swf[7]));
    ws[0] = load_scale(tn, 0);
    ws[1] = load_scale(tn, 1);
    const bool live = u < NU;
    const uint8_t* ub = lds + u * G::UNIT_BYTES;
    // Window by window: the operand slot and the 16 scale products sW * sA
    // of the window's registers (all from LDS, ahead of the weights), the
    // window's steps on the matrix core, then register q times its product
    // into the row sums, in register order.
    v16f acc;
    v4i Q;
    float pr[16];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int w = g / (int)G::WN, gp = g % (int)G::WN;
      if (live) {
        if (gp == 0) {
          Q = *reinterpret_cast<const v4i*>(ub + slot0 + (uint32_t)w * slot_step);
          const v4f* sap = reinterpret_cast<const v4f*>(ub + G::SA_OFF) + (h * 8u + (uint32_t)w * G::WN) * MB / 2u;
          float sav[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const v4f v = sap[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) sav[4 * i + k] = v[k];
          }
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = q / (int)G::QPM, gq = (q % (int)G::QPM) >> 1, e = q & 1;
            pr[q] = swf[w * (int)G::WN + gq][e] * sav[(gq * 2 + e) * MB + m];
          }
        }
        const v4i a = (G::WN == 1u || (uint32_t)gp == g_r) ? Q : v4i{};
        const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
        const v8i b8 = __builtin_shufflevector(wc[g], wc[g], 0, 1, 2, 3, -1, -1, -1, -1);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, gp == 0 ? v16f{} : acc, 4, 4, 0, 127, 0, 127);
        if (gp == (int)G::WN - 1) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int m = q / (int)G::QPM;
            part[m] = __builtin_fmaf(acc[q], pr[q], part[m]);
          }
        }
      }
      // Step g has gone to the matrix core: its registers take item j + 1's.
      wc[g] = load_code(tn, g);
    }

    if (j % NJ == NJ - 1u) {
      // End of a row block: lanes n and 32 + n hold the same weight row's
      // sums over different blocks; add them, then the 16 waves' in order.
      const uint32_t n0 = (blockIdx.x + (j / NJ) * gridDim.x) * 32u;
#pragma unroll
      for (int m = 0; m < MB; ++m) part[m] += __shfl_xor(part[m], 32);
      if (h == 0u) {
#pragma unroll
        for (int m = 0; m < MB; ++m) red[(wave * MB + (uint32_t)m) * 32u + n] = part[m];
      }
      __syncthreads();
      if (tid < 32u * M) {
        const uint32_t m = tid >> 5, c = tid & 31u, col = n0 + c;
        float v = red[m * 32u + c];
#pragma unroll
        for (uint32_t w = 1; w < BS_WAVES; ++w) v += red[(w * MB + m) * 32u + c];
        v *= scale;
        if (col < N) {
          if (OUT == 0)
            static_cast<float*>(C)[(size_t)m * N + col] = v;
          else
            static_cast<uint16_t*>(C)[(size_t)m * N + col] = f32_to_bf16(v);
        }
      }
      if (j + 1u < T) __syncthreads();   // red is reused by the next row block
#pragma unroll
      for (int m = 0; m < MB; ++m) part[m] = 0.0f;
    }
  }
}

int bs_mb(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

template <int MB>
bool bs_fits(int64_t K) {
  using G = BsGeom<MB>;
  const int64_t nu = (K + 511) / 512, nj = nu > BS_WAVES ? (nu + BS_WAVES - 1) / BS_WAVES : 1;
  return MB * nu * 32 <= 1024 * (int64_t)G::XNB && 16 * MB * nj <= 64 * (int64_t)G::NA &&
         nu * (int64_t)G::UNIT_BYTES + (int64_t)G::RED_BYTES <= (int64_t)BS_LDS_BYTES;
}

dim3 bs_grid(int64_t N) {
  const uint32_t nblocks = (uint32_t)((N + 31) / 32);
  return dim3(nblocks < 256u ? nblocks : 256u);
}

template <int MB>
hipError_t bs_launch(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                     const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype, bool fused,
                     const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, hipStream_t stream) {
  const dim3 grid = bs_grid(N), block(BS_WAVES * 64);
  const uint32_t m = (uint32_t)M, n = (uint32_t)N, k = (uint32_t)K;
  if (!fused) {
    if (out_dtype == 0)
      gemv_bs_kernel<MB, false, 0, kDtBF16, BS_HOLD><<<grid, block, 0, stream>>>(A, sA, B, sB, tsA, tsB, C, m, n, k, nullptr,
                                                                        nullptr, 0u);
    else
      gemv_bs_kernel<MB, false, 1, kDtBF16, BS_HOLD><<<grid, block, 0, stream>>>(A, sA, B, sB, tsA, tsB, C, m, n, k, nullptr,
                                                                        nullptr, 0u);
    return hipGetLastError();
  }
  const float* ts_in = x_tensor_scale;
  float* ts_out = (flags & 1u) ? nullptr : x_tensor_scale;
#define BS_FUSED(OUTT, XT)                                                                                          \
  gemv_bs_kernel<MB, true, OUTT, XT, BS_HOLD><<<grid, block, 0, stream>>>(nullptr, nullptr, B, sB, ts_in, tsB, C, m, n, k, X, \
                                                                 ts_out, flags)
  if (x_dtype == kDtBF16) {
    if (out_dtype == 0) BS_FUSED(0, kDtBF16);
    else BS_FUSED(1, kDtBF16);
  } else {
    if (out_dtype == 0) BS_FUSED(0, kDtF32);
    else BS_FUSED(1, kDtF32);
  }
#undef BS_FUSED
  return hipGetLastError();
}

hipError_t bs_dispatch(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                       const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype, bool fused,
                       const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, hipStream_t stream) {
  switch (bs_mb(M)) {
    case 1: return bs_launch<1>(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, fused, X, x_dtype, x_tensor_scale, flags, stream);
    case 2: return bs_launch<2>(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, fused, X, x_dtype, x_tensor_scale, flags, stream);
    case 4: return bs_launch<4>(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, fused, X, x_dtype, x_tensor_scale, flags, stream);
    default: return bs_launch<8>(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, fused, X, x_dtype, x_tensor_scale, flags, stream);
  }
}

}  // namespace

bool gemv_bs_applies(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 8 || N < 1 || K < 0) return false;
  switch (bs_mb(M)) {
    case 1: return bs_fits<1>(K);
    case 2: return bs_fits<2>(K);
    case 4: return bs_fits<4>(K);
    default: return bs_fits<8>(K);
  }
}

hipError_t launch_gemv_bs(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                          const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                          hipStream_t stream) {
  return bs_dispatch(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, false, nullptr, kDtBF16, nullptr, 0u, stream);
}

hipError_t launch_gemv_bs_fused(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* B,
                                const uint8_t* sB, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                                int out_dtype, hipStream_t stream) {
  return bs_dispatch(nullptr, nullptr, B, sB, nullptr, tsB, C, M, N, K, out_dtype, true, X, x_dtype, x_tensor_scale,
                     flags, stream);
}

}  // namespace fp4
