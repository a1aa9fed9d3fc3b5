// quantize.hip -- FP32/BF16 -> MXFP4 / NVFP4 quantisers, tensor amax, and
// dequantisation, for gfx950.
//
// Method (Ultralytics glossary "FP4", "How FP4 works"; NVFP4 video transcript,
// prism.simon-ai.net): per block take the largest magnitude, choose the scale
// that maps it to 6 (MXFP4: a power of two, E8M0; NVFP4: an E4M3 value under
// one FP32 tensor scale), round each scaled element to the nearest E2M1 value
// and pack two codes per byte ("Rubin FP4 GEMM deep dive", §5.2).
//
// Work mapping: one wavefront per (row, 512-element K slice).  Each lane owns 8
// consecutive elements (32 B of FP32 or 16 B of BF16, one or two 16-byte
// loads; a wavefront reads 2 KB / 1 KB contiguous), the block maximum is a
// 4-lane (MXFP4) or 2-lane (NVFP4) butterfly, the lane writes its 4 code bytes
// as one dword, and the scale bytes of the slice are gathered with cross-lane
// shuffles into the dwords of the tiled layout, so every store is a dword.
#include "fp4_device.h"
#include "fp4_launch.h"
#include "gemm_common.h"

#include <float.h>

#include <atomic>
#include <mutex>

namespace fp4 {

// ---------------------------------------------------------------------------
// Library-held scratch for fp4_quantize_noalloc (callers that cannot
// allocate: code under graph capture, serving loops, allocation-free
// harnesses).  Each GPU the library runs on holds one copy of this array
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in): it takes the device address
// from hipGetSymbolAddress once per device, with that device current, and
// passes that.  Every call on one GPU shares its copy, so overlapping calls
// on one GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4u];

namespace {
__global__ void clear_words_kernel(uint32_t* __restrict__ w, uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}
}  // namespace

hipError_t scratch_for_current_device(hipStream_t stream, void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex init;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= (int)kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(init);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      // The control words must start at zero; every completed call leaves
      // them zero again.  A kernel, not a memset, so that a first call made
      // under graph capture records a plain kernel node.
      clear_words_kernel<<<1, 64, 0, stream>>>(static_cast<uint32_t*>(p), kScratchBytes / 4u);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

namespace {


template <int DT>
__device__ __forceinline__ void load8v(const void* x, size_t idx, float v[8]) {
  if (DT == kDtF32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + idx);
    const u32x4 a = __builtin_nontemporal_load(p);
    const u32x4 b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = u2f(a[k]);
      v[4 + k] = u2f(b[k]);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + idx);
    const u32x4 a = __builtin_nontemporal_load(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = u2f(a[k] << 16);
      v[2 * k + 1] = u2f(a[k] & 0xFFFF0000u);
    }
  }
}

// ---------------------------------------------------------------------------
// Tensor amax (NVFP4 tensor scale, NVFP4 video transcript: one FP32 scale for
// the global range).  Grid-stride max, one atomicMax per workgroup on the
// float's bit pattern (non-negative floats order like unsigned integers), and
// the last workgroup to finish turns the maximum into s_t = amax / (6 * 448),
// writes it, and clears the two workspace words for the next call.
// ---------------------------------------------------------------------------
// Each workgroup pass covers a span of TPB * NL * 16 bytes: every lane
// issues NL 16-byte loads (a wave's load reads 1 KB contiguous) before it
// folds any of them; buffer loads bound the last, partial span without a
// branch.  The max runs on the magnitude bits (for finite values and
// infinities the integer order is the order of |x|; NaNs are skipped).  A
// dword holds one FP32 value or two BF16 values (each the high half of an
// FP32 value).
//
// The grid is small (at most 128 workgroups): the completion protocol below
// costs two device-scope atomics per workgroup on one address, and those
// serialise (measured ~9.5 ns each: 2048 workgroups added ~38 us to an
// otherwise 20 us pass over 134 MB).
// NaN policy of every tensor maximum (this kernel, the one-launch small
// path, the fused decode kernels): a NaN element is skipped, as fmaxf skips
// it.  In magnitude bits a NaN is above +inf (0x7F800000), so it is taken as
// 0 here.
__device__ __forceinline__ uint32_t mag_bits_no_nan(uint32_t a) { return a <= 0x7F800000u ? a : 0u; }

template <int DT, int TPB, int NL>
__global__ __launch_bounds__(TPB) void tensor_amax_kernel(const void* __restrict__ x, size_t nbytes,
                                                          uint32_t* __restrict__ ws, float* __restrict__ ts) {
  constexpr uint32_t SPAN = (uint32_t)TPB * 16u * (uint32_t)NL;
  uint32_t mb = 0u;
  const size_t step = (size_t)gridDim.x * SPAN;
  for (size_t off = (size_t)blockIdx.x * SPAN; off < nbytes; off += step) {
    const size_t rem = nbytes - off;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(static_cast<const uint8_t*>(x) + off, rem < SPAN ? (uint32_t)rem : SPAN);
    u32x4 w[NL];
#pragma unroll
    for (uint32_t u = 0; u < (uint32_t)NL; ++u)
      w[u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (u * (uint32_t)TPB + threadIdx.x) * 16u, 0, 0));
#pragma unroll
    for (int u = 0; u < NL; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (DT == kDtF32) {
          mb = max(mb, mag_bits_no_nan(w[u][k] & 0x7FFFFFFFu));
        } else {
          mb = max(mb, mag_bits_no_nan((w[u][k] << 16) & 0x7FFF0000u));
          mb = max(mb, mag_bits_no_nan(w[u][k] & 0x7FFF0000u));
        }
      }
  }
  float m = u2f(mb);
  m = wave_fmax(m);
  __shared__ float red[TPB / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    // Device-scope atomics meet at one coherence point for all XCDs.  The max
    // must be performed before this block counts itself in, so wait for its
    // return before the add; the block that counts last then reads the final
    // max.  (A release fence here would write back and invalidate the XCD's
    // whole L2 once per block.)
#pragma unroll
    for (int i = 1; i < TPB / 64; ++i) m = fmaxf(m, red[i]);
    const uint32_t prev = __hip_atomic_fetch_max(&ws[0], f2u(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" : : "v"(prev) : "memory");
    const uint32_t done = __hip_atomic_fetch_add(&ws[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      const float amax = u2f(__hip_atomic_fetch_or(&ws[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      float s = 1.0f;
      if (amax > 0.0f) {
        s = amax / 2688.0f;
        if (s < FLT_MIN) s = FLT_MIN;
      }
      *ts = s;
      ws[0] = 0u;
      ws[1] = 0u;
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 quantiser.  One wave covers two 256-element scale tiles (8 blocks
// each) of one row; waves cover rows_pad = 32 * ceil(rows/32) rows so that the
// padding rows of the scale tiles are written (as 0).
// ---------------------------------------------------------------------------
// SR: the elements are rounded stochastically (Philox words keyed by seed);
// the scales are unchanged.  FMT kFmtMX8 / kFmtMX8Ocp: MXFP8 ("Rubin FP4 GEMM
// deep dive", §3.4: activations kept in FP8 beside FP4 weights), the same
// 32-blocks and scale tiles with E4M3 elements, one byte each (round to
// nearest even, saturating at 448; no stochastic rounding).
// One (row, 512-value slice) item of a wave: block maxima, scale bytes, codes
// and the slice's two scale dwords.  v holds the lane's 8 values (zeros where
// !valid).
template <int FMT, bool SR>
__device__ __forceinline__ void quantize_mx_item(const float (&v)[8], bool valid, uint32_t row, uint32_t kt2,
                                                 uint32_t lane, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, uint32_t K, uint32_t KT,
                                                 uint64_t seed) {
  const uint32_t k0 = kt2 * 512u + lane * 8u;
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(v[k]));
  am = fmaxf(am, lane_xor1(am));
  am = fmaxf(am, lane_xor2(am));
  constexpr bool FP8 = FMT == kFmtMX8 || FMT == kFmtMX8Ocp;
  static_assert(!(FP8 && SR), "stochastic rounding is defined for E2M1 only");
  const uint32_t sbyte = FP8 ? mx8_scale_byte<FMT>(am) : mx_scale_byte<FMT>(am);  // 0 for padding (am == 0)
  if (FP8 && valid) {
    const float inv = u2f((254u - sbyte) << 23);
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = v[k] * inv;
    uint2 w;
    w.x = e4m3x4_sat(y[0], y[1], y[2], y[3]);
    w.y = e4m3x4_sat(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2*>(codes + (size_t)row * K + k0) = w;
  } else if (valid) {
    // y = x * 2^-e with e = sbyte - 127: exact power of two, 2^(127 - e) is a
    // normal float for every byte 0..253.
    const float inv = u2f((254u - sbyte) << 23);
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = v[k] * inv;
    uint32_t w;
    if (SR) {
      uint32_t r[8];
      sr_words8(seed, (uint64_t)row * K + k0, r);
      w = pack8_sr(y, r);
    } else {
      w = pack8(y);
    }
    *reinterpret_cast<uint32_t*>(codes + (size_t)row * (K / 2) + k0 / 2) = w;
  }
  // Tile t = lane / 32 holds blocks 8t..8t+7 of the slice (block q of the
  // slice in lanes 4q..4q+3).  Its dword for chunk j (lanes 32t + j, j < 2)
  // holds blocks q = j, 2+j, 4+j, 6+j in bytes 0..3.
  const uint32_t base = lane & 32u, j = lane & 1u;
  const uint32_t b0 = __shfl(sbyte, base + 4 * j);
  const uint32_t b1 = __shfl(sbyte, base + 4 * j + 8);
  const uint32_t b2 = __shfl(sbyte, base + 4 * j + 16);
  const uint32_t b3 = __shfl(sbyte, base + 4 * j + 24);
  const uint32_t kt = 2u * kt2 + (lane >> 5);
  if ((lane & 31u) < 2u && kt < KT) {
    const uint32_t dw = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    const size_t off = ((size_t)(row >> 5) * KT + kt) * 256u + (32u * j + (row & 31u)) * 4u;
    *reinterpret_cast<uint32_t*>(scales + off) = dw;
  }
}

// IT consecutive items per wave: all their loads are issued before any is
// used (out-of-range lanes load element 0 and drop it, so the loads carry no
// branch and stay in flight together), then the items are quantised in turn.
template <int FMT, int DT, bool SR, int IT>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, uint32_t rows, uint32_t K,
                                                          uint32_t KT, uint32_t KT2, uint32_t total_waves,
                                                          uint64_t seed) {
  const uint32_t wave = blockIdx.x * 4u + (threadIdx.x >> 6);  // < 2^26: the host bounds the grid
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t w0 = wave * (uint32_t)IT;
  if (w0 >= total_waves) return;
  float v[IT][8];
  bool valid[IT];
#pragma unroll
  for (int t = 0; t < IT; ++t) {
    const uint32_t item = w0 + (uint32_t)t, row = item / KT2, k0 = (item % KT2) * 512u + lane * 8u;
    valid[t] = item < total_waves && row < rows && k0 < K;
    load8v<DT>(x, valid[t] ? (size_t)row * K + k0 : 0u, v[t]);
  }
#pragma unroll
  for (int t = 0; t < IT; ++t) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[t][k] = valid[t] ? v[t][k] : 0.0f;
    const uint32_t item = w0 + (uint32_t)t;
    if (item < total_waves)
      quantize_mx_item<FMT, SR>(v[t], valid[t], item / KT2, item % KT2, lane, codes, scales, K, KT, seed);
  }
}

// ---------------------------------------------------------------------------
// NVFP4 quantiser.  One wave covers two 256-element scale tiles of one row
// (lanes 0-31 the first, 32-63 the second); waves cover 32 * ceil(rows/32)
// rows so the tiles' padding rows are written (as 0).
//   r = (amax_b / 6) / s_t; sb = E4M3(r); d = E4M3value(sb) * s_t;
//   code = E2M1(x / d)   (x / inf = +-0 when sb == 0, so the block is all zero)
// All divisions are IEEE FP32 round-to-nearest-even.
// ---------------------------------------------------------------------------
// One wave: 512 values (two scale tiles) of one row.  The lane's 8 values
// (zeros past the matrix), then their quantisation with tensor scale s_t.
template <int DT>
__device__ __forceinline__ bool load_nv_wave(const void* __restrict__ x, uint32_t rows, uint32_t K, uint32_t KT2,
                                             uint32_t wave, uint32_t lane, float v[8]) {
  const uint32_t row = wave / KT2, kt2 = wave % KT2;
  const uint32_t k0 = kt2 * 512u + lane * 8u;
  const bool valid = row < rows && k0 < K;
  if (valid) {
    load8v<DT>(x, (size_t)row * K + k0, v);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.0f;
  }
  return valid;
}

// am_in >= 0: the block maximum to use (2-D scaling: the 16 x 16 patch's).
template <bool SR>
__device__ __forceinline__ void quantize_nv_wave(const float v[8], bool valid, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, float s_t, uint32_t K, uint32_t KT,
                                                 uint32_t KT2, uint32_t wave, uint32_t lane, uint64_t seed,
                                                 float am_in = -1.0f) {
  const uint32_t row = wave / KT2, kt2 = wave % KT2;
  const uint32_t k0 = kt2 * 512u + lane * 8u;
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(v[k]));
  am = fmaxf(am, lane_xor1(am));
  if (am_in >= 0.0f) am = am_in;
  const float r = (am / 6.0f) / s_t;
  const uint32_t sb = e4m3_encode(r);
  if (valid) {
    float y[8];
    if (sb == 0u) {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = __builtin_copysignf(0.0f, v[k]);   // x / inf
    } else {
      const float d = e4m3_value(sb) * s_t;
      const float rd = 1.0f / d;
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = nv_div(v[k], d, rd);
    }
    uint32_t w;
    if (SR) {
      uint32_t r[8];
      sr_words8(seed, (uint64_t)row * K + k0, r);
      w = pack8_sr(y, r);
    } else {
      w = pack8(y);
    }
    *reinterpret_cast<uint32_t*>(codes + (size_t)row * (K / 2) + k0 / 2) = w;
  }
  // Tile T = lane / 32 holds blocks q = 0..15 of 16 values (block q in lanes
  // 32T + 2q, 32T + 2q + 1).  Tile lane 32j + i (j = chunk parity) holds 8
  // bytes: dword d has blocks 8d + 2j + {0, 1, 4, 5}.  Writer lane 32T + 2j + d.
  const uint32_t base = lane & 32u, j = (lane >> 1) & 1u, d = lane & 1u;
  const uint32_t q0 = 8u * d + 2u * j;
  const uint32_t c0 = __shfl(sb, base + 2u * q0);
  const uint32_t c1 = __shfl(sb, base + 2u * (q0 + 1u));
  const uint32_t c2 = __shfl(sb, base + 2u * (q0 + 4u));
  const uint32_t c3 = __shfl(sb, base + 2u * (q0 + 5u));
  const uint32_t kt = 2u * kt2 + (lane >> 5);
  if ((lane & 31u) < 4u && kt < KT) {
    const uint32_t dw = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    const size_t off = ((size_t)(row >> 5) * KT + kt) * 512u + (32u * j + (row & 31u)) * 8u + 4u * d;
    *reinterpret_cast<uint32_t*>(scales + off) = dw;
  }
}

// IT consecutive items per wave, loads first (as quantize_mx_kernel).
template <int DT, bool SR, int IT>
__global__ __launch_bounds__(256) void quantize_nv_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          const float* __restrict__ tensor_scale, uint32_t rows,
                                                          uint32_t K, uint32_t KT, uint32_t KT2,
                                                          uint32_t total_waves, uint64_t seed) {
  const uint32_t wave = blockIdx.x * 4u + (threadIdx.x >> 6);  // < 2^26: the host bounds the grid
  const uint32_t w0 = wave * (uint32_t)IT;
  if (w0 >= total_waves) return;
  const uint32_t lane = threadIdx.x & 63u;
  float v[IT][8];
  bool valid[IT];
#pragma unroll
  for (int t = 0; t < IT; ++t) {
    const uint32_t item = w0 + (uint32_t)t, row = item / KT2, k0 = (item % KT2) * 512u + lane * 8u;
    valid[t] = item < total_waves && row < rows && k0 < K;
    load8v<DT>(x, valid[t] ? (size_t)row * K + k0 : 0u, v[t]);
  }
  const float s_t = *tensor_scale;
#pragma unroll
  for (int t = 0; t < IT; ++t) {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[t][k] = valid[t] ? v[t][k] : 0.0f;
    if (w0 + (uint32_t)t < total_waves)
      quantize_nv_wave<SR>(v[t], valid[t], codes, scales, s_t, K, KT, KT2, w0 + (uint32_t)t, lane, seed);
  }
}

// ---------------------------------------------------------------------------
// NVFP4 quantiser for small tensors (the activation of a decode step): every
// workgroup of 16 waves reduces the whole tensor's maximum itself (exact, so
// the same s_t as tensor_amax_kernel; the input stays in L2 after the first
// reads), then its waves quantise their own 512-value pieces as above.  One
// launch instead of two and no cross-workgroup exchange; workgroup 0 writes
// s_t.
// ---------------------------------------------------------------------------
constexpr uint32_t kNvSmallMaxBytes = 256u * 1024u;

// This thread's share of the whole tensor's largest magnitude (n8 chunks of 8
// values): loads in batches of 8 chunks per thread, all issued before their
// use; buffer loads past the end return zeros (no branch, so the batch stays
// in flight together).  fmaxf skips NaNs.
template <int DT>
__device__ __forceinline__ float whole_tensor_max(__amdgpu_buffer_rsrc_t rx, size_t n8, uint32_t tid) {
  constexpr uint32_t EB = DT == kDtF32 ? 4u : 2u;
  float m = 0.0f;
  for (uint32_t b = tid; b < (uint32_t)n8; b += 8u * 1024u) {
    u32x4 raw[8][EB / 2u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (uint32_t h = 0; h < EB / 2u; ++h)
        raw[u][h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (b + (uint32_t)u * 1024u) * 8u * EB + 16u * h, 0, 0));
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (uint32_t h = 0; h < EB / 2u; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wd = raw[u][h][k];
          if (DT == kDtF32) {
            m = fmaxf(m, fabsf(u2f(wd)));
          } else {
            m = fmaxf(m, fabsf(u2f(wd << 16)));
            m = fmaxf(m, fabsf(u2f(wd & 0xFFFF0000u)));
          }
        }
  }
  return m;
}

template <int DT, bool SR>
__global__ __launch_bounds__(1024) void quantize_nv_small_kernel(const void* __restrict__ x,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 float* __restrict__ tensor_scale, size_t n8,
                                                                 uint32_t rows, uint32_t K, uint32_t KT,
                                                                 uint32_t KT2, uint32_t total_waves, uint64_t seed) {
  __shared__ float red[16];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
  constexpr uint32_t EB = DT == kDtF32 ? 4u : 2u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)(n8 * 8u * EB));
  // This wave's own values first (they arrive while the maximum is reduced);
  // branch-free, so that nothing waits for them before the loads below.
  const uint32_t wave = blockIdx.x * 16u + w;
  const uint32_t row = wave / KT2, k0 = (wave % KT2) * 512u + lane * 8u;
  const bool valid = wave < total_waves && row < rows && k0 < K;
  const uint32_t voff = valid ? (row * K + k0) * EB : 0x80000000u;
  u32x4 own[EB / 2u];
#pragma unroll
  for (uint32_t h = 0; h < EB / 2u; ++h)
    own[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + 16u * h, 0, 0));
  // At most 256 KB: at most 2 batches per thread.
  float m = whole_tensor_max<DT>(rx, n8, tid);
  m = wave_fmax(m);
  if (lane == 0u) red[w] = m;
  __syncthreads();
  float amax = red[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) amax = fmaxf(amax, red[i]);
  float s_t = 1.0f;
  if (amax > 0.0f) {
    s_t = amax / 2688.0f;
    if (s_t < FLT_MIN) s_t = FLT_MIN;
  }
  if (blockIdx.x == 0 && tid == 0) *tensor_scale = s_t;
  float v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (DT == kDtF32) {
      v[k] = u2f(own[0][k]);
      v[4 + k] = u2f(own[EB / 2u - 1u][k]);
    } else {
      v[2 * k] = u2f(own[0][k] << 16);
      v[2 * k + 1] = u2f(own[0][k] & 0xFFFF0000u);
    }
  }
  if (wave < total_waves) quantize_nv_wave<SR>(v, valid, codes, scales, s_t, K, KT, KT2, wave, lane, seed);
}

// ---------------------------------------------------------------------------
// NVFP4 quantiser for mid-size tensors (above 256 KB, at most 1 MB: e.g. a
// 32-row decode activation), one launch without re-reading the tensor: each
// workgroup of 16 waves loads only its own 512-value pieces, folds their
// maximum into the workspace's running maximum (device-scope atomics, as
// tensor_amax_kernel) and counts itself in, waits until every workgroup has
// counted in, reads the maximum and quantises its pieces.  Workspace words:
// [0] the running maximum (magnitude bits), [1] workgroups counted in, [2]
// workgroups done with the maximum; the last of those clears all three for
// the next call.  The wait is bounded (spin_limit sleeps): a grid of at most
// 128 workgroups is resident at once on this part, but a workgroup that stops
// waiting reduces the whole tensor's maximum itself, which is the same exact
// value, so the result never depends on the wait.
// ---------------------------------------------------------------------------
constexpr uint32_t kNvGridMaxBytes = 1024u * 1024u;
constexpr uint32_t kNvGridSpin = 1u << 16;
constexpr uint32_t kNoMax = 0xFFFFFFFFu;

template <int DT, bool SR>
__global__ __launch_bounds__(1024) void quantize_nv_grid_kernel(const void* __restrict__ x,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales,
                                                                float* __restrict__ tensor_scale,
                                                                uint32_t* __restrict__ ws, size_t n8, uint32_t rows,
                                                                uint32_t K, uint32_t KT, uint32_t KT2,
                                                                uint32_t total_waves, uint32_t spin_limit,
                                                                uint64_t seed) {
  __shared__ float red[16];
  __shared__ uint32_t max_bits;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
  constexpr uint32_t EB = DT == kDtF32 ? 4u : 2u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)(n8 * 8u * EB));
  const uint32_t wave = blockIdx.x * 16u + w;
  const uint32_t row = wave / KT2, k0 = (wave % KT2) * 512u + lane * 8u;
  const bool valid = wave < total_waves && row < rows && k0 < K;
  const uint32_t voff = valid ? (row * K + k0) * EB : 0x80000000u;
  u32x4 own[EB / 2u];
#pragma unroll
  for (uint32_t h = 0; h < EB / 2u; ++h)
    own[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + 16u * h, 0, 0));
  float v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (DT == kDtF32) {
      v[k] = u2f(own[0][k]);
      v[4 + k] = u2f(own[EB / 2u - 1u][k]);
    } else {
      v[2 * k] = u2f(own[0][k] << 16);
      v[2 * k + 1] = u2f(own[0][k] & 0xFFFF0000u);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));   // pieces past the tensor loaded zeros
  m = wave_fmax(m);
  if (lane == 0u) red[w] = m;
  __syncthreads();
  if (tid == 0u) {
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, red[i]);
    // The max is performed before this workgroup counts itself in (wait for
    // its return), so a workgroup that sees every count sees every max.
    const uint32_t prev = __hip_atomic_fetch_max(&ws[0], f2u(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" : : "v"(prev) : "memory");
    __hip_atomic_fetch_add(&ws[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t bits = kNoMax;
    for (uint32_t it = 0; it < spin_limit; ++it) {
      if (__hip_atomic_load(&ws[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= gridDim.x) {
        bits = __hip_atomic_load(&ws[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    max_bits = bits;
  }
  __syncthreads();
  float amax;
  if (max_bits != kNoMax) {
    amax = u2f(max_bits);
  } else {
    // Stopped waiting: the whole tensor's maximum from every element.
    float mm = wave_fmax(whole_tensor_max<DT>(rx, n8, tid));
    if (lane == 0u) red[w] = mm;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) amax = fmaxf(amax, red[i]);
  }
  if (tid == 0u) {
    const uint32_t done = __hip_atomic_fetch_add(&ws[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1u) {
#pragma unroll
      for (int i = 0; i < 3; ++i) __hip_atomic_store(&ws[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  float s_t = 1.0f;
  if (amax > 0.0f) {
    s_t = amax / 2688.0f;
    if (s_t < FLT_MIN) s_t = FLT_MIN;
  }
  if (blockIdx.x == 0 && tid == 0) *tensor_scale = s_t;
  if (wave < total_waves) quantize_nv_wave<SR>(v, valid, codes, scales, s_t, K, KT, KT2, wave, lane, seed);
}

// ---------------------------------------------------------------------------
// NVFP4 with 2-D block scaling (NVFP4 video transcript, the training recipe's
// second part: a weight matrix serves as W forward and W^T backward, so its
// scales are shared by 16 x 16 patches and both directions quantise alike).
// A workgroup of 16 waves takes 16 rows of one 512-column slice; each wave
// reduces its row's 16-value block maxima, the 16 rows' maxima meet in LDS,
// and every row (inside the matrix) quantises with its patch maximum.  Rows
// past the matrix keep scale byte 0.
// ---------------------------------------------------------------------------
template <int DT, bool SR>
__global__ __launch_bounds__(1024) void quantize_nv2d_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             const float* __restrict__ tensor_scale, uint32_t rows,
                                                             uint32_t K, uint32_t KT, uint32_t KT2, uint64_t seed) {
  __shared__ float blk[16][32];
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  const uint32_t row = blockIdx.y * 16u + w, kt2 = blockIdx.x;
  const uint32_t wave = row * KT2 + kt2;      // the 1-D kernel's wave index of (row, slice)
  float v[8];
  const bool valid = load_nv_wave<DT>(x, rows, K, KT2, wave, lane, v);
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(v[k]));
  am = fmaxf(am, lane_xor1(am));
  if ((lane & 1u) == 0u) blk[w][lane >> 1] = am;
  __syncthreads();
  float pm = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) pm = fmaxf(pm, blk[r][lane >> 1]);
  quantize_nv_wave<SR>(v, valid, codes, scales, *tensor_scale, K, KT, KT2, wave, lane, seed, row < rows ? pm : 0.0f);
}

// ---------------------------------------------------------------------------
// Random Hadamard transform on 16-value blocks along K (NVFP4 video
// transcript, the training recipe's third part: the block's values are mixed
// so that an outlier no longer sets its scale alone; the transform is
// orthogonal, so norms and dot products along K are kept).  y = (1/4) H16 D x
// per block: D = the signs of column k (top bit of its Philox word under
// seed, so two matrices transformed with one seed keep their products), H16
// applied as butterflies of distance 1, 2, 4 (within the lane's 8 values)
// and 8 (with the neighbouring lane), the 1/4 exact.  A lane holds 8 columns
// and walks rows; its signs are computed once.
// ---------------------------------------------------------------------------
template <int DT, int OT>
__global__ __launch_bounds__(256) void hadamard16_kernel(const void* __restrict__ x, void* __restrict__ y,
                                                         uint32_t rows, uint32_t K, uint64_t seed) {
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  const uint32_t k0 = blockIdx.x * 512u + lane * 8u;
  const bool col_ok = k0 < K;
  uint32_t r8[8];
  sr_words8(seed, k0, r8);
  for (uint32_t row = blockIdx.y * 4u + w; row < rows; row += gridDim.y * 4u) {
    float v[8];
    if (col_ok) {
      load8v<DT>(x, (size_t)row * K + k0, v);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = (r8[k] >> 31) ? -v[k] : v[k];
#pragma unroll
    for (int h = 1; h < 8; h *= 2)
#pragma unroll
      for (int i = 0; i < 8; i += 2 * h)
#pragma unroll
        for (int m = i; m < i + h; ++m) {
          const float a = v[m], c = v[m + h];
          v[m] = a + c;
          v[m + h] = a - c;
        }
    // distance 8: positions m (even lane) and m + 8 (odd lane)
    const bool upper = (lane & 1u) != 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float o = lane_xor1(v[k]);
      v[k] = upper ? o - v[k] : v[k] + o;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] *= 0.25f;
    if (col_ok) {
      if (OT == kDtF32) {
        u32x4 a, b;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a[k] = f2u(v[k]);
          b[k] = f2u(v[4 + k]);
        }
        u32x4* p = reinterpret_cast<u32x4*>(static_cast<float*>(y) + (size_t)row * K + k0);
        p[0] = a;
        p[1] = b;
      } else {
        u32x4 a;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          a[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + (size_t)row * K + k0) = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantisation: one lane per 8 elements.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float mag = (m < 2u) ? 0.5f * (float)m : u2f(((m >> 1) + 126u) << 23) * (1.0f + 0.5f * (float)(m & 1u));
  return (c & 8u) ? -mag : mag;
}

template <int FMT, int OUT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ tensor_scale,
                                                         void* __restrict__ out, uint32_t rows, uint32_t K,
                                                         uint32_t KT) {
  const size_t t = (size_t)blockIdx.x * 256u + threadIdx.x;
  const uint32_t per_row = K / 8u;
  if (t >= (size_t)rows * per_row) return;
  const uint32_t row = (uint32_t)(t / per_row);
  const uint32_t k0 = (uint32_t)(t % per_row) * 8u;
  const uint32_t bs = (FMT == kFmtNV) ? 16u : 32u;
  const uint32_t sbyte = scales[scale_offset<FMT == kFmtNV ? kFmtNV : kFmtMX>(row, k0 / bs, KT)];
  float o[8];
  if (FMT == kFmtMX8) {
    // E4M3 bytes (the codes the quantiser writes: never the NaN pattern)
    // times 2^(byte - 127), both exact.
    const uint2 cw8 = *reinterpret_cast<const uint2*>(codes + (size_t)row * K + k0);
    const int e = (int)sbyte - 127;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t c = ((k < 4 ? cw8.x : cw8.y) >> (8 * (k & 3))) & 0xFFu;
      const float m = e4m3_value(c & 0x7Fu);
      o[k] = __builtin_ldexpf((c & 0x80u) ? -m : m, e);
    }
  } else if (FMT == kFmtNV) {
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + (size_t)row * (K / 2) + k0 / 2);
    const float s = e4m3_value(sbyte);
    const float st = *tensor_scale;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (e2m1_value(cw >> (4 * k)) * s) * st;
  } else {
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + (size_t)row * (K / 2) + k0 / 2);
    const int e = (int)sbyte - 127;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = __builtin_ldexpf(e2m1_value(cw >> (4 * k)), e);
  }
  const size_t idx = (size_t)row * K + k0;
  if (OUT == kDtF32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + idx);
    p[0] = float4{o[0], o[1], o[2], o[3]};
    p[1] = float4{o[4], o[5], o[6], o[7]};
  } else {
    uint4 w;
    w.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
    w.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
    w.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

}  // namespace

hipError_t launch_tensor_amax(const void* x, int in_dtype, int64_t n, uint32_t* ws, float* tensor_scale,
                              hipStream_t stream) {
  const size_t nbytes = (size_t)n * (in_dtype == kDtF32 ? 4u : 2u);
  // Measured (8192^2 BF16 = 134 MB: 21.8 us; 33.5 MB: 7.6 us; 4 MB: 4.7 us):
  // up to 8 MB, 256-thread workgroups with 32 KB spans, at most 64 of them;
  // beyond, 1024-thread workgroups with 64 KB spans, at most 128.
  const bool big = nbytes > (size_t(8) << 20);
  const size_t span = big ? 65536u : 32768u, cap = big ? 128u : 64u;
  size_t blocks = (nbytes + span - 1) / span;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks);
  if (in_dtype == kDtF32) {
    if (big)
      tensor_amax_kernel<kDtF32, 1024, 4><<<grid, dim3(1024), 0, stream>>>(x, nbytes, ws, tensor_scale);
    else
      tensor_amax_kernel<kDtF32, 256, 8><<<grid, dim3(256), 0, stream>>>(x, nbytes, ws, tensor_scale);
  } else {
    if (big)
      tensor_amax_kernel<kDtBF16, 1024, 4><<<grid, dim3(1024), 0, stream>>>(x, nbytes, ws, tensor_scale);
    else
      tensor_amax_kernel<kDtBF16, 256, 8><<<grid, dim3(256), 0, stream>>>(x, nbytes, ws, tensor_scale);
  }
  return hipGetLastError();
}

bool quantize_nv_grid_applies(int64_t rows, int64_t K, int in_dtype) {
  const int64_t bytes = rows * K * (in_dtype == kDtF32 ? 4 : 2);
  return rows >= 1 && K >= 16 && bytes > (int64_t)kNvSmallMaxBytes && bytes <= (int64_t)kNvGridMaxBytes;
}

bool quantize_nv_small_applies(int64_t rows, int64_t K, int in_dtype) {
  const int64_t bytes = rows * K * (in_dtype == kDtF32 ? 4 : 2);
  return rows >= 1 && K >= 16 && bytes <= (int64_t)kNvSmallMaxBytes;
}

namespace {
template <bool SR>
void launch_nv_small(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales, float* tensor_scale, int64_t rows,
                     int64_t K, uint64_t seed, hipStream_t stream) {
  const uint32_t r = (uint32_t)rows, k = (uint32_t)K;
  const uint32_t rows_pad = (r + 31u) / 32u * 32u;
  const uint32_t KT = (k + 255u) / 256u, KT2 = (KT + 1u) / 2u;
  const uint32_t waves = rows_pad * KT2;
  const dim3 grid((waves + 15u) / 16u);
  const size_t n8 = (size_t)rows * (size_t)K / 8u;
  if (in_dtype == kDtF32)
    quantize_nv_small_kernel<kDtF32, SR><<<grid, dim3(1024), 0, stream>>>(x, codes, scales, tensor_scale, n8, r, k,
                                                                         KT, KT2, waves, seed);
  else
    quantize_nv_small_kernel<kDtBF16, SR><<<grid, dim3(1024), 0, stream>>>(x, codes, scales, tensor_scale, n8, r, k,
                                                                          KT, KT2, waves, seed);
}

template <bool SR>
void launch_q(const void* x, int fmt, int in_dtype, uint8_t* codes, uint8_t* scales, const float* tensor_scale,
              int64_t rows, int64_t K, uint64_t seed, hipStream_t stream) {
  const uint32_t r = (uint32_t)rows, k = (uint32_t)K;
  const uint32_t rows_pad = (r + 31u) / 32u * 32u;
  const uint32_t KT = (k + 255u) / 256u, KT2 = (KT + 1u) / 2u;
  const uint32_t waves = rows_pad * KT2;
  const dim3 grid((waves + 3u) / 4u), block(256);
  // One item per wave for FP32 input (a lane's two 16-byte loads already keep
  // 2 KB per wave in flight); four for BF16 (1 KB each) on large inputs, where
  // that still leaves eight waves per SIMD.  Measured: MXFP4 16384 x 2880 BF16
  // 27.4 -> 23.4 us, NVFP4 8192^2 BF16 43.0 -> 41.3 us; 8192^2 FP32 56.3 us
  // with one item, 59.5 with two, 61.8 with four; a 32 x 8192 decode
  // activation (512 items) slower with four.  Stochastic rounding keeps one:
  // its Philox multiplies bound it, and NVFP4 8192^2 BF16 took 160.7 us with
  // one item, 162.5 with two, 162.0 with four.
  constexpr int IT = SR ? 1 : 4;
  const bool multi = waves >= 32768u;
  const dim3 gridm((waves + 4u * IT - 1u) / (4u * IT));
  const bool f32 = in_dtype == kDtF32;
  if (fmt == kFmtNV) {
    if (f32)
      quantize_nv_kernel<kDtF32, SR, 1><<<grid, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                    waves, seed);
    else if (multi)
      quantize_nv_kernel<kDtBF16, SR, IT><<<gridm, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                      waves, seed);
    else
      quantize_nv_kernel<kDtBF16, SR, 1><<<grid, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                     waves, seed);
  } else if (fmt == kFmtMX) {
    if (f32)
      quantize_mx_kernel<kFmtMX, kDtF32, SR, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2, waves, seed);
    else if (multi)
      quantize_mx_kernel<kFmtMX, kDtBF16, SR, IT><<<gridm, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2, waves, seed);
    else
      quantize_mx_kernel<kFmtMX, kDtBF16, SR, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2, waves, seed);
  } else if (fmt == kFmtMX8 || fmt == kFmtMX8Ocp) {
    if constexpr (!SR) {
      if (fmt == kFmtMX8) {
        if (f32)
          quantize_mx_kernel<kFmtMX8, kDtF32, false, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2,
                                                                                 waves, seed);
        else if (multi)
          quantize_mx_kernel<kFmtMX8, kDtBF16, false, IT><<<gridm, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2,
                                                                                  waves, seed);
        else
          quantize_mx_kernel<kFmtMX8, kDtBF16, false, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2,
                                                                                 waves, seed);
      } else {
        if (f32)
          quantize_mx_kernel<kFmtMX8Ocp, kDtF32, false, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2,
                                                                                    waves, seed);
        else if (multi)
          quantize_mx_kernel<kFmtMX8Ocp, kDtBF16, false, IT><<<gridm, block, 0, stream>>>(x, codes, scales, r, k, KT,
                                                                                     KT2, waves, seed);
        else
          quantize_mx_kernel<kFmtMX8Ocp, kDtBF16, false, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT,
                                                                                    KT2, waves, seed);
      }
    }
  } else {
    if (f32)
      quantize_mx_kernel<kFmtMXOcp, kDtF32, SR, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2, waves,
                                                                            seed);
    else if (multi)
      quantize_mx_kernel<kFmtMXOcp, kDtBF16, SR, IT><<<gridm, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2, waves,
                                                                             seed);
    else
      quantize_mx_kernel<kFmtMXOcp, kDtBF16, SR, 1><<<grid, block, 0, stream>>>(x, codes, scales, r, k, KT, KT2, waves,
                                                                            seed);
  }
}
}  // namespace

hipError_t launch_quantize_nv_small(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales,
                                    float* tensor_scale, int64_t rows, int64_t K, bool sr, uint64_t seed,
                                    hipStream_t stream) {
  if (sr)
    launch_nv_small<true>(x, in_dtype, codes, scales, tensor_scale, rows, K, seed, stream);
  else
    launch_nv_small<false>(x, in_dtype, codes, scales, tensor_scale, rows, K, seed, stream);
  return hipGetLastError();
}

hipError_t launch_quantize_nv_grid(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales,
                                   float* tensor_scale, uint32_t* ws, int64_t rows, int64_t K, bool sr, uint64_t seed,
                                   uint32_t spin_limit, hipStream_t stream) {
  const uint32_t r = (uint32_t)rows, k = (uint32_t)K;
  const uint32_t rows_pad = (r + 31u) / 32u * 32u;
  const uint32_t KT = (k + 255u) / 256u, KT2 = (KT + 1u) / 2u;
  const uint32_t waves = rows_pad * KT2;
  const dim3 grid((waves + 15u) / 16u);
  const size_t n8 = (size_t)rows * (size_t)K / 8u;
  const uint32_t spin = spin_limit ? spin_limit : kNvGridSpin;
#define NV_GRID(DT, SRB)                                                                                        \
  quantize_nv_grid_kernel<DT, SRB><<<grid, dim3(1024), 0, stream>>>(x, codes, scales, tensor_scale, ws, n8, r, k, KT, \
                                                                     KT2, waves, spin, seed)
  if (in_dtype == kDtF32) {
    if (sr)
      NV_GRID(kDtF32, true);
    else
      NV_GRID(kDtF32, false);
  } else {
    if (sr)
      NV_GRID(kDtBF16, true);
    else
      NV_GRID(kDtBF16, false);
  }
#undef NV_GRID
  return hipGetLastError();
}

hipError_t launch_quantize_nv2d(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales,
                                const float* tensor_scale, int64_t rows, int64_t K, bool sr, uint64_t seed,
                                hipStream_t stream) {
  const uint32_t r = (uint32_t)rows, k = (uint32_t)K;
  const uint32_t rows_pad = (r + 31u) / 32u * 32u;
  const uint32_t KT = (k + 255u) / 256u, KT2 = (KT + 1u) / 2u;
  const dim3 grid(KT2, rows_pad / 16u), block(1024);
  const bool f32 = in_dtype == kDtF32;
  if (sr) {
    if (f32)
      quantize_nv2d_kernel<kDtF32, true><<<grid, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                      seed);
    else
      quantize_nv2d_kernel<kDtBF16, true><<<grid, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                       seed);
  } else {
    if (f32)
      quantize_nv2d_kernel<kDtF32, false><<<grid, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                       seed);
    else
      quantize_nv2d_kernel<kDtBF16, false><<<grid, block, 0, stream>>>(x, codes, scales, tensor_scale, r, k, KT, KT2,
                                                                        seed);
  }
  return hipGetLastError();
}

hipError_t launch_hadamard16(const void* x, int in_dtype, void* y, int out_dtype, int64_t rows, int64_t K,
                             uint64_t seed, hipStream_t stream) {
  const uint32_t gx = (uint32_t)((K + 511) / 512);
  uint32_t gy = (uint32_t)((rows + 3) / 4);
  const uint32_t cap = gx >= 4096u ? 1u : 4096u / gx;
  if (gy > cap) gy = cap;
  const dim3 grid(gx, gy), block(256);
  const uint32_t r = (uint32_t)rows, k = (uint32_t)K;
  if (in_dtype == kDtF32) {
    if (out_dtype == kDtF32)
      hadamard16_kernel<kDtF32, kDtF32><<<grid, block, 0, stream>>>(x, y, r, k, seed);
    else
      hadamard16_kernel<kDtF32, kDtBF16><<<grid, block, 0, stream>>>(x, y, r, k, seed);
  } else {
    if (out_dtype == kDtF32)
      hadamard16_kernel<kDtBF16, kDtF32><<<grid, block, 0, stream>>>(x, y, r, k, seed);
    else
      hadamard16_kernel<kDtBF16, kDtBF16><<<grid, block, 0, stream>>>(x, y, r, k, seed);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int fmt, int in_dtype, uint8_t* codes, uint8_t* scales,
                           const float* tensor_scale, int64_t rows, int64_t K, bool sr, uint64_t seed,
                           hipStream_t stream) {
  if (sr)
    launch_q<true>(x, fmt, in_dtype, codes, scales, tensor_scale, rows, K, seed, stream);
  else
    launch_q<false>(x, fmt, in_dtype, codes, scales, tensor_scale, rows, K, seed, stream);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int fmt,
                             void* out, int out_dtype, int64_t rows, int64_t K, hipStream_t stream) {
  const uint32_t r = (uint32_t)rows, k = (uint32_t)K;
  const size_t threads = (size_t)r * (k / 8u);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const uint32_t KT = (k + 255u) / 256u;
  if (fmt == kFmtNV) {
    if (out_dtype == kDtF32)
      dequantize_kernel<kFmtNV, kDtF32><<<grid, dim3(256), 0, stream>>>(codes, scales, tensor_scale, out, r, k, KT);
    else
      dequantize_kernel<kFmtNV, kDtBF16><<<grid, dim3(256), 0, stream>>>(codes, scales, tensor_scale, out, r, k, KT);
  } else if (fmt == kFmtMX8 || fmt == kFmtMX8Ocp) {
    if (out_dtype == kDtF32)
      dequantize_kernel<kFmtMX8, kDtF32><<<grid, dim3(256), 0, stream>>>(codes, scales, tensor_scale, out, r, k, KT);
    else
      dequantize_kernel<kFmtMX8, kDtBF16><<<grid, dim3(256), 0, stream>>>(codes, scales, tensor_scale, out, r, k, KT);
  } else {
    if (out_dtype == kDtF32)
      dequantize_kernel<kFmtMX, kDtF32><<<grid, dim3(256), 0, stream>>>(codes, scales, tensor_scale, out, r, k, KT);
    else
      dequantize_kernel<kFmtMX, kDtBF16><<<grid, dim3(256), 0, stream>>>(codes, scales, tensor_scale, out, r, k, KT);
  }
  return hipGetLastError();
}

}  // namespace fp4
