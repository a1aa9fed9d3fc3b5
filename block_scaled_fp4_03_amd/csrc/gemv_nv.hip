// gemv_nv.hip -- NVFP4 decode GEMV / skinny GEMM (M <= 32 activation rows)
// for gfx950.
//
// C[m,n] = (sum_k A^[m,k] W^[n,k]) * tsA * tsW with NVFP4 operands (NVFP4
// video transcript: 16-value blocks, E4M3 block scale, FP32 tensor scale).
// Decoding streams every weight once, so the path is bound by HBM bandwidth
// ("Rubin FP4 GEMM deep dive", §1.2, §6.2); operands are decoded exactly to
// FP16 and multiplied on the FP16 matrix core (see gemm.hip for why FP16).
#include "fp4_launch.h"
#include "gemm_common.h"

namespace fp4 {

namespace {

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
__global__ __launch_bounds__(256) void gemv_nv_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA,
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
  u32x2 wsc[SPLIT];
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
    wsc[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsw, soff, 0, 0));
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

size_t gemv_nv_workspace(int64_t M, int64_t N, int64_t K) {
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

bool gemv_nv_applies(int64_t M, int64_t N) { return M >= 1 && M <= 32 && N <= GV_MAX_N; }

hipError_t launch_gemv_nv(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                          int out_dtype, void* workspace, hipStream_t stream) {
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

}  // namespace fp4
