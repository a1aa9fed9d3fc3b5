// gemm_nv.hip -- NVFP4 x NVFP4 GEMM for gfx950.
//
// C[m,n] = (sum_k A^[m,k] B^[n,k]) * tsA * tsB, with A^ = E2M1(code) * E4M3(
// block scale) per 16-value block and tsA, tsB the FP32 tensor scales (NVFP4
// video transcript: 16-value blocks with an E4M3 scale plus one FP32 scale per
// tensor; "Rubin FP4 GEMM deep dive" §3.1, §4.2: FP32 accumulation, result
// times the product of the scales).
//
// Design.  gfx950's block-scaled matrix instructions take only power-of-two
// (E8M0) scales per 32 values, so E4M3 16-blocks cannot ride in the
// instruction exactly.  E2M1 * E4M3 needs at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in FP16: each operand is decoded in
// registers to FP16 (v_cvt_scalef32_pk_f16_fp4 for the E2M1 values, then a
// packed FP16 multiply by the block's E4M3 scale) and fed to the FP16 matrix
// core (v_mfma_f32_32x32x16_f16) with FP32 accumulation; the tensor scales are
// applied in the epilogue.  The data path is the MXFP4 kernel's: 256 x 256
// tiles, 8 wavefronts of 128 x 64, FP4 codes and scales streamed into LDS with
// buffer_load ... lds through two 256-value K stages.
#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

constexpr uint32_t BM = 256, BN = 256;
constexpr uint32_t STEP_BYTES = 128;                // 256 FP4 values per row per stage
constexpr uint32_t REGION = 256 * STEP_BYTES;       // 32 KB of codes per operand per stage
constexpr uint32_t STILE = 512;                     // NVFP4 scale tile: 32 rows x 16 blocks
constexpr uint32_t SCALE_REGION = 8 * STILE;        // 4 KB of scales per operand per stage
constexpr uint32_t STAGE_BYTES = 2 * REGION + 2 * SCALE_REGION;  // 72 KB
constexpr uint32_t NSTAGE = 2;
constexpr uint32_t GROUP_M = 4;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_t;

struct Ops {
  v4i a[4], b[2];
};

// E4M3 byte (0..0x7E) -> FP16 bits (exact).  Normal values (byte >= 8) keep
// their 3 mantissa bits and rebias the exponent by 8; subnormals m * 2^-9
// are normal FP16 numbers and are converted through FP32.
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

// Eight FP16 values = E2M1 codes of one dword (low nibble first) times s.
__device__ __forceinline__ v8h decode8(uint32_t w, v2h s) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One 64-value K sub-step SUB of a wave's 128 x 64 sub-tile: the lane's 32
// codes of each operand block split into four groups of 8 (group g uses the
// chunk's 16-block g/2), one 32x32x16 FP16 MFMA per block pair and group.
template <int SUB>
__device__ __forceinline__ void mma_sub(v16f (&acc)[4][2], const Ops& o, const u32x2 (&sa)[4],
                                        const u32x2 (&sb)[2]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int byte = 2 * SUB + (g >> 1);  // scale byte of this group within the lane's 8 bytes
    v8h a[4], b[2];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = decode8((uint32_t)o.a[r][g], scale_pair((sa[r][byte >> 2] >> (8 * (byte & 3))) & 0xFFu));
#pragma unroll
    for (int c = 0; c < 2; ++c) b[c] = decode8((uint32_t)o.b[c][g], scale_pair((sb[c][byte >> 2] >> (8 * (byte & 3))) & 0xFFu));
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[r], b[c], acc[r][c], 0, 0, 0);
  }
}

template <int OUT>
__global__ __launch_bounds__(512, 1) void gemm_nv_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
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
  const uint32_t ldb = K / 2u;
  const uint32_t rowsA = (M - m0) < BM ? (M - m0) : BM;
  const uint32_t rowsB = (N - n0) < BN ? (N - n0) : BN;
  const uint8_t* const a_tile = A + (size_t)m0 * ldb;
  const uint8_t* const b_tile = B + (size_t)n0 * ldb;
  const uint32_t a_bytes = rowsA * ldb, b_bytes = rowsB * ldb;
  const uint32_t KT = (K + 255u) / 256u;
  const uint32_t RTA = (M + 31u) / 32u, RTB = (N + 31u) / 32u;
  const uint32_t srow = KT * STILE;
  const uint8_t* const sa_tile = sA + (size_t)(m0 / 32u) * srow;
  const uint8_t* const sb_tile = sB + (size_t)(n0 / 32u) * srow;
  const uint32_t sa_bytes = (RTA > m0 / 32u ? RTA - m0 / 32u : 0u) * srow;
  const uint32_t sb_bytes = (RTB > n0 / 32u ? RTB - n0 / 32u : 0u) * srow;

  // Code loads as in the MXFP4 kernel (LDS row r keeps chunk c at position
  // c ^ ((r >> 1) & 7)); scale tile w (512 B) of A and of B per wave.
  const uint32_t gchunk = (lane & 7u) ^ ((4u * (wave & 1u) + (lane >> 4)) & 7u);
  uint32_t voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) voff[q] = (8u * (wave + 8u * q) + (lane >> 3)) * ldb + 16u * gchunk;
  const uint32_t svoff = (wave * KT) * STILE + lane * 4u;

  auto dma = [&](uint32_t stage_k) {
    const uint32_t kb = opaque(stage_k * STEP_BYTES);
    const uint32_t ko = opaque(stage_k * STILE);
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
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(st + 2u * REGION + STILE * wave + 256u * h), 4,
                                               svoff + 256u * h, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(st + 2u * REGION + SCALE_REGION + STILE * wave + 256u * h),
                                               4, svoff + 256u * h, 0, 0, 0);
    }
  };

  const uint32_t li = lane & 31u, lj = lane >> 5;
  uint32_t rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rd[q] = 128u * li + 16u * ((2u * q + lj) ^ ((li >> 1) & 7u));
  const uint32_t a_rows = 128u * (128u * wm);
  const uint32_t b_rows = 128u * (64u * wn);

  auto read_ops = [&](uint32_t stage_k, int q, Ops& o) {
    const uint8_t* st = lds + (stage_k % NSTAGE) * STAGE_BYTES;
#pragma unroll
    for (int r = 0; r < 4; ++r) o.a[r] = *reinterpret_cast<const v4i*>(st + a_rows + 4096u * r + rd[q]);
#pragma unroll
    for (int c = 0; c < 2; ++c) o.b[c] = *reinterpret_cast<const v4i*>(st + REGION + b_rows + 4096u * c + rd[q]);
  };
  auto read_scales = [&](uint32_t stage_k, u32x2 (&sa)[4], u32x2 (&sb)[2]) {
    const uint8_t* st = lds + (stage_k % NSTAGE) * STAGE_BYTES + 2u * REGION;
#pragma unroll
    for (int r = 0; r < 4; ++r) sa[r] = *reinterpret_cast<const u32x2*>(st + STILE * (4u * wm + r) + 8u * lane);
#pragma unroll
    for (int c = 0; c < 2; ++c)
      sb[c] = *reinterpret_cast<const u32x2*>(st + SCALE_REGION + STILE * (2u * wn + c) + 8u * lane);
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // Same stage schedule as the MXFP4 kernel (see there).  Codes past K in a
  // last, partial stage carry padding scale bytes (0): their FP16 values are
  // zero, so they add nothing.
  if (KT > 0) {
    Ops o0, o1;
    u32x2 sa[4], sb[2], sa_n[4], sb_n[2];
    dma(0);
    dma(1);
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_ops(0, 0, o0);
    read_scales(0, sa, sb);
    for (uint32_t k = 0; k < KT; ++k) {
      read_ops(k, 1, o1);
      mma_sub<0>(acc, o0, sa, sb);
      read_ops(k, 2, o0);
      mma_sub<1>(acc, o1, sa, sb);
      read_ops(k, 3, o1);
      mma_sub<2>(acc, o0, sa, sb);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      dma(k + 2u);
      read_ops(k + 1u, 0, o0);
      read_scales(k + 1u, sa_n, sb_n);
      mma_sub<3>(acc, o1, sa, sb);
#pragma unroll
      for (int r = 0; r < 4; ++r) sa[r] = sa_n[r];
#pragma unroll
      for (int c = 0; c < 2; ++c) sb[c] = sb_n[c];
    }
  }

  // ---- epilogue: x tsA * tsB; lane L of a 32x32 block holds column L%32,
  // rows 8*(i/4) + 4*(L/32) + i%4.
  const float scale = *tsA * *tsB;
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

// ---------------------------------------------------------------------------
// Decode GEMV / skinny GEMM: M <= 32 activation rows against N x K NVFP4
// weights ("Rubin FP4 GEMM deep dive" §1.2, §6.2: decoding streams every
// weight once, so it is bound by memory bandwidth).
//
// Workgroup = 4 wavefronts = 128 weight rows x one K slice of SPLIT 256-value
// tiles.  Each wave owns 32 weight rows and issues all of its slice's code and
// scale loads at once (32 KB per wave in flight), then, while they land, the
// workgroup decodes its activation slice once into LDS as FP16 in the
// matrix-core operand order (rows >= M are zero).  Per 64-value sub-step a
// lane holds 32 weight codes (chunk 2s + j of its row, the scale layout's lane
// order) and runs four 32x32x16 FP16 MFMAs against the activation operands
// read from LDS.  Partial sums of the K slices go to the workspace; the last
// workgroup of a column block (atomic counter, reset afterwards) adds them in
// slice order, applies tsA * tsB and writes C.
// ---------------------------------------------------------------------------
constexpr uint32_t GV_ROWS = 128;       // weight rows per workgroup
constexpr uint32_t GV_MAX_SPLIT = 8;    // 256-value tiles per K slice

template <int OUT, int SPLIT>
__global__ __launch_bounds__(256, 2) void gemv_nv_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
                                                        const uint8_t* __restrict__ W, const uint8_t* __restrict__ sW,
                                                        const float* __restrict__ tsA, const float* __restrict__ tsW,
                                                        void* __restrict__ C, float* __restrict__ partial,
                                                        uint32_t* __restrict__ counters, uint32_t M, uint32_t N,
                                                        uint32_t K, uint32_t KS) {
  // A operands: [tile][sub-step s][group t][lane] x 16 B (8 FP16).
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a[SPLIT * 16 * 1024];
  __shared__ uint32_t last_flag;

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nb = blockIdx.x / KS, ks = blockIdx.x % KS;
  const uint32_t n0 = nb * GV_ROWS + 32u * wave;       // this wave's first weight row
  const uint32_t KT = (K + 255u) / 256u;
  const uint32_t kt0 = ks * SPLIT;                     // first 256-value tile of the slice
  const uint32_t ldb = K / 2u;
  const uint32_t li = lane & 31u, lj = lane >> 5;

  // ---- issue every weight load of the slice (codes 16 B per sub-step, scale
  // 8 B per tile); rows past N and tiles past K read as zero.
  const uint32_t wrows = N > n0 ? (N - n0 < 32u ? N - n0 : 32u) : 0u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * ldb, wrows * ldb);
  const uint32_t srow = KT * 512u;
  const __amdgpu_buffer_rsrc_t rsw =
      make_rsrc(sW + (size_t)(n0 / 32u) * srow, (n0 < N) ? srow : 0u);
  v4i wc[SPLIT][4];
  u32x2_t wsc[SPLIT];
#pragma unroll
  for (int t = 0; t < SPLIT; ++t) {
    const uint32_t kt = kt0 + t;
    const uint32_t ok = kt < KT;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const uint32_t off = ok ? li * ldb + kt * 128u + 32u * s2 + 16u * lj : 0x80000000u;
      wc[t][s2] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
    }
    const uint32_t soff = ok ? kt * 512u + 8u * lane : 0x80000000u;
    wsc[t] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rsw, soff, 0, 0));
  }

  // ---- activation slice -> LDS (FP16, operand order).  Thread = (row, chunk)
  // of each tile: row i = tid % 32, chunk c = tid / 32 (0..7).
  {
    const uint32_t tid = threadIdx.x;
    const uint32_t i = tid & 31u, c = tid >> 5;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, M * ldb);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sA, KT * 512u);
#pragma unroll
    for (int t = 0; t < SPLIT; ++t) {
      const uint32_t kt = kt0 + t;
      const bool ok = kt < KT && i < M;
      const uint32_t off = ok ? i * ldb + kt * 128u + 16u * c : 0x80000000u;
      const v4i codes = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
      const uint32_t slane = 32u * (c & 1u) + i, s = c >> 1;
      const uint32_t soff = ok ? kt * 512u + 8u * slane + 2u * s : 0x80000000u;
      const uint32_t sc2 = __builtin_amdgcn_raw_buffer_load_b16(rsa, soff, 0, 0);
      const v2h s0 = scale_pair(sc2 & 0xFFu), s1 = scale_pair(sc2 >> 8);
      uint8_t* dst = lds_a + ((t * 4u + s) * 4u) * 1024u + (32u * (c & 1u) + i) * 16u;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<v8h*>(dst + g * 1024u) = decode8((uint32_t)codes[g], g < 2 ? s0 : s1);
    }
  }
  __syncthreads();

  // ---- weights x activation
  v16f acc = v16f{};
#pragma unroll
  for (int t = 0; t < SPLIT; ++t) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const uint32_t sw = wsc[t][s2 >> 1] >> (16 * (s2 & 1));
      const v2h w0 = scale_pair(sw & 0xFFu), w1 = scale_pair((sw >> 8) & 0xFFu);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v8h b = decode8((uint32_t)wc[t][s2][g], g < 2 ? w0 : w1);
        const v8h a = *reinterpret_cast<const v8h*>(lds_a + ((t * 4u + s2) * 4u + g) * 1024u + lane * 16u);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
      }
    }
  }

  // ---- partials: lane L holds column n0 + L%32 and rows 8(i/4) + 4(L/32) + i%4
  const uint32_t col = n0 + li;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t m = 8u * (i >> 2) + 4u * lj + (i & 3);
    if (m < M && col < N) partial[((size_t)ks * M + m) * N + col] = acc[i];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = atomicAdd(&counters[nb], 1u);
    last_flag = (done == KS - 1u);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float scale = *tsA * *tsW;
  const uint32_t cbase = nb * GV_ROWS;
  for (uint32_t e = threadIdx.x; e < M * GV_ROWS; e += 256u) {
    const uint32_t m = e / GV_ROWS, n = cbase + e % GV_ROWS;
    if (n >= N) continue;
    float sum = 0.0f;
    for (uint32_t q = 0; q < KS; ++q) sum += partial[((size_t)q * M + m) * N + n];
    const float v = sum * scale;
    if (OUT == 0)
      static_cast<float*>(C)[(size_t)m * N + n] = v;
    else
      static_cast<uint16_t*>(C)[(size_t)m * N + n] = f32_to_bf16(v);
  }
  if (threadIdx.x == 0) counters[nb] = 0u;
}

// Split of K for the decode path: at least ~256 workgroups, at most
// GV_MAX_SPLIT tiles per slice.
struct GemvPlan {
  uint32_t nblocks, split, ks;
};

static GemvPlan gemv_plan(int64_t N, int64_t K) {
  GemvPlan p;
  p.nblocks = (uint32_t)((N + GV_ROWS - 1) / GV_ROWS);
  const uint32_t KT = (uint32_t)((K + 255) / 256);
  uint32_t want = (256u + p.nblocks - 1u) / p.nblocks;      // slices wanted for ~256 WGs
  if (want < 1u) want = 1u;
  uint32_t split = (KT + want - 1u) / want;
  if (split > GV_MAX_SPLIT) split = GV_MAX_SPLIT;
  if (split < 1u) split = 1u;
  // round the split up to a supported instantiation
  split = split <= 1u ? 1u : split <= 2u ? 2u : split <= 4u ? 4u : 8u;
  p.split = split;
  p.ks = (KT + split - 1u) / split;
  if (p.ks < 1u) p.ks = 1u;
  return p;
}

}  // namespace

// Decode-path workspace: GV_COUNTER_BYTES of per-column-block counters at the
// start (zero before and after every call, at the same place whatever the
// shape), then the split-K partial sums (scratch).
constexpr size_t GV_COUNTER_BYTES = 65536;
constexpr int64_t GV_MAX_N = (int64_t)(GV_COUNTER_BYTES / sizeof(uint32_t)) * GV_ROWS;

size_t gemm_nv_workspace(int64_t M, int64_t N, int64_t K) {
  if (M > 32 || M <= 0 || N <= 0 || N > GV_MAX_N) return 0;
  const GemvPlan p = gemv_plan(N, K);
  return GV_COUNTER_BYTES + (size_t)p.ks * (size_t)M * (size_t)N * sizeof(float);
}

template <int OUT>
static void launch_gemv(const GemvPlan& p, dim3 grid, const uint8_t* A, const uint8_t* sA, const uint8_t* W,
                        const uint8_t* sW, const float* tsA, const float* tsW, void* C, float* partial,
                        uint32_t* counters, uint32_t M, uint32_t N, uint32_t K, hipStream_t stream) {
  switch (p.split) {
    case 1: gemv_nv_kernel<OUT, 1><<<grid, 256, 0, stream>>>(A, sA, W, sW, tsA, tsW, C, partial, counters, M, N, K, p.ks); break;
    case 2: gemv_nv_kernel<OUT, 2><<<grid, 256, 0, stream>>>(A, sA, W, sW, tsA, tsW, C, partial, counters, M, N, K, p.ks); break;
    case 4: gemv_nv_kernel<OUT, 4><<<grid, 256, 0, stream>>>(A, sA, W, sW, tsA, tsW, C, partial, counters, M, N, K, p.ks); break;
    default: gemv_nv_kernel<OUT, 8><<<grid, 256, 0, stream>>>(A, sA, W, sW, tsA, tsW, C, partial, counters, M, N, K, p.ks); break;
  }
}

hipError_t launch_gemm_nv(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                          int out_dtype, void* workspace, size_t /*workspace_bytes*/, hipStream_t stream) {
  if (M <= 32 && N <= GV_MAX_N) {
    const GemvPlan p = gemv_plan(N, K);
    uint32_t* counters = static_cast<uint32_t*>(workspace);
    float* partial = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + GV_COUNTER_BYTES);
    const dim3 grid(p.nblocks * p.ks);
    if (out_dtype == 0)
      launch_gemv<0>(p, grid, A, sA, B, sB, tsA, tsB, C, partial, counters, (uint32_t)M, (uint32_t)N, (uint32_t)K,
                     stream);
    else
      launch_gemv<1>(p, grid, A, sA, B, sB, tsA, tsB, C, partial, counters, (uint32_t)M, (uint32_t)N, (uint32_t)K,
                     stream);
    return hipGetLastError();
  }
  const uint32_t tilesM = (uint32_t)((M + BM - 1) / BM), tilesN = (uint32_t)((N + BN - 1) / BN);
  const dim3 grid(tilesM * tilesN);
  if (out_dtype == 0)
    gemm_nv_kernel<0><<<grid, dim3(512), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, (uint32_t)M, (uint32_t)N,
                                                      (uint32_t)K, tilesM, tilesN);
  else
    gemm_nv_kernel<1><<<grid, dim3(512), 0, stream>>>(A, sA, B, sB, tsA, tsB, C, (uint32_t)M, (uint32_t)N,
                                                      (uint32_t)K, tilesM, tilesN);
  return hipGetLastError();
}

}  // namespace fp4
