// abi.cpp -- the C ABI of libfp4 (declared in include/fp4.h): argument
// validation, kernel selection and launch on the caller's stream.
//
// Validation runs on the host before any HIP call, so every argument error is
// reported synchronously with a negative status and nothing is enqueued.
#include "../../include/fp4.h"
#include "fp4_launch.h"

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <hip/hip_runtime.h>
#include <initializer_list>
#include <stdint.h>
#include <vector>

namespace {

// FP4 formats (every GEMM operand of fp4_gemm*), and the quantiser's formats
// (those plus MXFP8).
bool fmt_ok(int fmt) { return fmt == FP4_MXFP4 || fmt == FP4_NVFP4 || fmt == FP4_MXFP4_OCP; }
bool is_mx8(int fmt) { return fmt == FP4_MXFP8 || fmt == FP4_MXFP8_OCP; }
bool qfmt_ok(int fmt) { return fmt_ok(fmt) || is_mx8(fmt); }
bool dtype_ok(int dt) { return dt == FP4_F32 || dt == FP4_BF16; }
int64_t block_of(int fmt) { return fmt == FP4_NVFP4 ? 16 : 32; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Sizes are kept within what the kernels index with 32-bit arithmetic.
constexpr int64_t kMaxDim = int64_t(1) << 30;

// A launch's work-items per grid dimension are a 32-bit count, and the
// element-wise kernels form their wave and thread indices from it in 32
// bits.  The quantisers run one 64-lane wave per (row, 512-value slice) over
// 32 * ceil(rows / 32) rows; dequantisation one thread per 8 values.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;
bool quantize_grid_fits(int64_t rows, int64_t K) {
  const int64_t rows_pad = (rows + 31) / 32 * 32, slices = (K + 511) / 512;
  return rows_pad * slices * 64 <= kMaxWorkItems;
}
bool dequantize_grid_fits(int64_t rows, int64_t K) { return rows * (K / 8) + 255 <= kMaxWorkItems; }
// A 256-row operand tile must stay within one 32-bit buffer range.
constexpr int64_t kMaxGemmK = int64_t(1) << 24;


// The FP4 GEMM kernels address an operand's scale buffer (and the grouped
// kernel all of A) through 32-bit buffer ranges.
constexpr int64_t kMaxRange = (int64_t(1) << 32) - 1;
bool scales_fit(int fmt, int64_t rows, int64_t K) {
  return ((rows + 31) / 32) * ((K + 255) / 256) * (fmt == FP4_NVFP4 ? 512 : 256) <= kMaxRange;
}

// ---- debug mode (FP4_DEBUG=1 in the environment, or fp4_set_debug(1)) ----
// Checks that need HIP calls and a synchronisation, so they are off by
// default: every buffer a call reads or writes must lie inside one device
// allocation of the current device, large enough for the call; the grouped
// GEMM's group offsets and token indices are copied to the host and checked;
// and every call waits for its kernels, so that a launch or execution error is
// returned by the call that caused it.  -1: the environment not read yet.
std::atomic<int> g_debug{-1};

bool debug_on() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("FP4_DEBUG");
    v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expect = -1;
    g_debug.compare_exchange_strong(expect, v, std::memory_order_relaxed);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v == 1;
}

// Debug mode names every failure on stderr (what failed and HIP's error).
int debug_fail(int status, const char* what, hipError_t e = hipSuccess) {
  if (e != hipSuccess)
    std::fprintf(stderr, "fp4 debug: %s: %s\n", what, hipGetErrorString(e));
  else
    std::fprintf(stderr, "fp4 debug: %s\n", what);
  return status;
}

// A buffer of a call: its first byte and the bytes the call touches.
struct Buf {
  const void* p;
  uint64_t bytes;
};

// Debug mode: FP4_ERR_BOUNDS unless every non-empty buffer lies wholly inside
// one allocation made on the current device (hipMemGetAddressRange; a caching
// allocator's block counts as one allocation, so an overrun is only seen once
// it leaves the block).
int debug_buffers(std::initializer_list<Buf> bufs) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return debug_fail(FP4_ERR_HIP, "hipGetDevice", e);
  int i = 0;
  for (const Buf& b : bufs) {
    ++i;
    if (!b.p || b.bytes == 0) continue;
    void* base = nullptr;
    size_t size = 0;
    if ((e = hipMemGetAddressRange(&base, &size, const_cast<void*>(b.p))) != hipSuccess) {
      (void)hipGetLastError();
      std::fprintf(stderr, "fp4 debug: buffer %d (%p) is not in a device allocation: %s\n", i, b.p,
                   hipGetErrorString(e));
      return FP4_ERR_BOUNDS;
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), at = reinterpret_cast<uintptr_t>(b.p);
    if (at < lo || at - lo > size || size - (at - lo) < b.bytes) {
      std::fprintf(stderr, "fp4 debug: buffer %d (%p): %llu bytes needed, %llu left in its allocation\n", i, b.p,
                   (unsigned long long)b.bytes, (unsigned long long)(at >= lo && at - lo <= size ? size - (at - lo) : 0));
      return FP4_ERR_BOUNDS;
    }
    hipPointerAttribute_t attr;
    if ((e = hipPointerGetAttributes(&attr, b.p)) != hipSuccess) {
      (void)hipGetLastError();
      std::fprintf(stderr, "fp4 debug: buffer %d (%p): no pointer attributes: %s\n", i, b.p, hipGetErrorString(e));
      return FP4_ERR_BOUNDS;
    }
    if (attr.type == hipMemoryTypeDevice && attr.device != dev) {
      std::fprintf(stderr, "fp4 debug: buffer %d (%p) is on device %d, the current device is %d\n", i, b.p,
                   attr.device, dev);
      return FP4_ERR_BOUNDS;
    }
  }
  return FP4_OK;
}

// Debug mode: the grouped GEMM's device-side indices as the header states
// them: group_off[0] = 0, non-decreasing, group_off[E] = total_rows, and every
// row_idx entry in [0, A_rows).  Waits for the stream first (the offsets may
// be produced on it).
int debug_groups(const int32_t* row_idx, const int32_t* group_off, int32_t E, int64_t total_rows, int64_t A_rows,
                 hipStream_t s) {
  hipError_t err = hipStreamSynchronize(s);
  if (err != hipSuccess) return debug_fail(FP4_ERR_HIP, "hipStreamSynchronize before the index check", err);
  std::vector<int32_t> off((size_t)E + 1), idx((size_t)total_rows);
  if ((err = hipMemcpy(off.data(), group_off, off.size() * sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess ||
      (err = hipMemcpy(idx.data(), row_idx, idx.size() * sizeof(int32_t), hipMemcpyDeviceToHost)) != hipSuccess)
    return debug_fail(FP4_ERR_HIP, "copying the group offsets and token indices", err);
  if (off[0] != 0 || off[(size_t)E] != total_rows)
    return debug_fail(FP4_ERR_BOUNDS, "group_off does not run from 0 to total_rows");
  for (int32_t e = 0; e < E; ++e)
    if (off[(size_t)e + 1] < off[(size_t)e]) return debug_fail(FP4_ERR_BOUNDS, "group_off decreases");
  for (int32_t r : idx)
    if (r < 0 || r >= A_rows) return debug_fail(FP4_ERR_BOUNDS, "a row_idx entry is outside [0, A_rows)");
  return FP4_OK;
}

int launched(hipError_t e) {
  if (e == hipSuccess) return FP4_OK;
  return debug_on() ? debug_fail(FP4_ERR_HIP, "kernel launch", e) : FP4_ERR_HIP;
}

// The status of a call whose kernels were enqueued with status rc; debug
// mode waits for them.
int finish(int rc, hipStream_t s) {
  if (rc != FP4_OK || !debug_on()) return rc;
  const hipError_t e = hipStreamSynchronize(s);
  return e == hipSuccess ? FP4_OK : debug_fail(FP4_ERR_HIP, "hipStreamSynchronize after the launch", e);
}

uint64_t elem_bytes(int dt) { return dt == FP4_F32 ? 4u : 2u; }
// Code bytes of a rows x K quantised matrix.
uint64_t code_bytes(int fmt, int64_t rows, int64_t K) {
  return (uint64_t)rows * (uint64_t)K / (is_mx8(fmt) ? 1u : 2u);
}

}  // namespace

extern "C" {

int fp4_set_debug(int on) {
  const int prev = debug_on() ? 1 : 0;
  g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

int64_t fp4_scale_bytes(int fmt, int64_t rows, int64_t K) {
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (rows < 0 || K < 0 || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  // Tiles of 32 rows x 256 K values: 256 bytes (MXFP4, MXFP8) or 512 bytes (NVFP4).
  return ((rows + 31) / 32) * ((K + 255) / 256) * (fmt == FP4_NVFP4 ? 512 : 256);
}

size_t fp4_workspace_size(int op, int fmt, int64_t M, int64_t N, int64_t K, int32_t E) {
  switch (op) {
    case FP4_OP_QUANTIZE:
      return fmt == FP4_NVFP4 ? 16 : 0;
    case FP4_OP_GEMM:
      return 0;
    case FP4_OP_GEMM_GROUPED:
      // Optional: the token rows gathered into expert order.
      if (!fmt_ok(fmt) || M < 0 || K < 0 || K % 32 != 0) return 0;
      return fp4::gemm_grouped_workspace(fmt, M, N, K, E);
    default:
      return 0;
  }
}

// The one-launch NVFP4 quantiser's wait for the other workgroups is bounded;
// FP4_TEST_NV_GRID_SPIN (a positive count of sleeps) cuts it short so that
// tests can run the path a workgroup takes when it stops waiting.  Unset:
// the kernel's default.
static uint32_t nv_grid_spin_limit() {
  const char* e = std::getenv("FP4_TEST_NV_GRID_SPIN");
  if (!e || !*e) return 0u;
  const unsigned long v = std::strtoul(e, nullptr, 10);
  return v == 0ul || v > 0xFFFFFFFFul ? 0u : (uint32_t)v;
}

// ws_is_scratch: the workspace is fp4_quantize_noalloc's static array (not
// an allocation, so debug mode does not range-check it).
static int quantize_impl(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                         int64_t rows, int64_t K, int in_dtype, unsigned flags, void* workspace,
                         size_t workspace_bytes, uint64_t seed, void* stream, bool ws_is_scratch = false) {
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(in_dtype)) return FP4_ERR_DTYPE;
  if (flags & ~(FP4_TS_GIVEN | FP4_Q_SR | FP4_Q_2D)) return FP4_ERR_FLAGS;
  if ((flags & FP4_Q_2D) && fmt != FP4_NVFP4) return FP4_ERR_FMT;
  if ((flags & FP4_Q_SR) && is_mx8(fmt)) return FP4_ERR_FMT;
  const bool sr = (flags & FP4_Q_SR) != 0u, twod = (flags & FP4_Q_2D) != 0u;
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  if (!quantize_grid_fits(rows, K)) return FP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP4_OK;
  if (!x || !codes || !block_scales) return FP4_ERR_NULL;
  const bool nv = fmt == FP4_NVFP4;
  if (nv && !tensor_scale) return FP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, is_mx8(fmt) ? 8 : 4) || !aligned(block_scales, 4)) return FP4_ERR_ALIGN;
  if (nv && !aligned(tensor_scale, 4)) return FP4_ERR_ALIGN;
  const bool compute_ts = nv && !(flags & FP4_TS_GIVEN);
  if (compute_ts) {
    if (!workspace || workspace_bytes < 16) return FP4_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FP4_ERR_ALIGN;
  }
  hipStream_t s = as_stream(stream);
  if (debug_on()) {
    const int rc = debug_buffers({{x, (uint64_t)rows * (uint64_t)K * elem_bytes(in_dtype)},
                                  {codes, code_bytes(fmt, rows, K)},
                                  {block_scales, (uint64_t)fp4_scale_bytes(fmt, rows, K)},
                                  {nv ? tensor_scale : nullptr, 4u},
                                  {compute_ts && !ws_is_scratch ? workspace : nullptr, 16u}});
    if (rc != FP4_OK) return rc;
  }
  if (compute_ts && !twod && fp4::quantize_nv_small_applies(rows, K, in_dtype))
    return finish(launched(fp4::launch_quantize_nv_small(x, in_dtype, codes, block_scales, tensor_scale, rows, K,
                                                         sr, seed, s)),
                  s);
  if (compute_ts && !twod && fp4::quantize_nv_grid_applies(rows, K, in_dtype))
    return finish(launched(fp4::launch_quantize_nv_grid(x, in_dtype, codes, block_scales, tensor_scale,
                                                        static_cast<uint32_t*>(workspace), rows, K, sr, seed,
                                                        nv_grid_spin_limit(), s)),
                  s);
  if (compute_ts) {
    int rc = launched(fp4::launch_tensor_amax(x, in_dtype, rows * K, static_cast<uint32_t*>(workspace), tensor_scale, s));
    if (rc != FP4_OK) return rc;
  }
  if (twod)
    return finish(
        launched(fp4::launch_quantize_nv2d(x, in_dtype, codes, block_scales, tensor_scale, rows, K, sr, seed, s)), s);
  return finish(
      launched(fp4::launch_quantize(x, fmt, in_dtype, codes, block_scales, tensor_scale, rows, K, sr, seed, s)), s);
}

int fp4_quantize(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                 int64_t rows, int64_t K, int in_dtype, unsigned flags, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (flags & ~FP4_TS_GIVEN) return FP4_ERR_FLAGS;
  return quantize_impl(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, workspace,
                       workspace_bytes, 0ull, stream);
}

int fp4_quantize_noalloc(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                         int64_t rows, int64_t K, int in_dtype, unsigned flags, void* stream) {
  if (flags & ~FP4_TS_GIVEN) return FP4_ERR_FLAGS;
  // The same host-side validation as fp4_quantize, before any HIP call.
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(in_dtype)) return FP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  if (!quantize_grid_fits(rows, K)) return FP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP4_OK;
  const size_t need = fp4_workspace_size(FP4_OP_QUANTIZE, fmt, rows, 0, K, 0);
  if (need > fp4::kScratchBytes) return FP4_ERR_WORKSPACE;
  // NVFP4 computing its own tensor scale takes the scratch as its workspace
  // (inputs up to 256 KB reduce the maximum in one launch and leave it
  // untouched).
  const bool uses_ws = fmt == FP4_NVFP4 && !(flags & FP4_TS_GIVEN);
  if (!uses_ws)
    return quantize_impl(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, nullptr, 0, 0ull,
                         stream);
  // Argument errors first, so that a refused call makes no HIP call at all.
  if (!x || !codes || !block_scales || !tensor_scale) return FP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(block_scales, 4) || !aligned(tensor_scale, 4))
    return FP4_ERR_ALIGN;
  void* ws = nullptr;
  if (fp4::scratch_for_current_device(as_stream(stream), &ws) != hipSuccess) return FP4_ERR_HIP;
  return quantize_impl(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, ws, fp4::kScratchBytes,
                       0ull, stream, true);
}

int fp4_quantize_sr(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                    int64_t rows, int64_t K, int in_dtype, unsigned flags, uint64_t seed, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (flags & ~FP4_TS_GIVEN) return FP4_ERR_FLAGS;
  return quantize_impl(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags | FP4_Q_SR, workspace,
                       workspace_bytes, seed, stream);
}

int fp4_quantize_ex(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                    int64_t rows, int64_t K, int in_dtype, unsigned flags, uint64_t seed, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return quantize_impl(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, workspace,
                       workspace_bytes, seed, stream);
}

int fp4_hadamard16(const void* x, int in_dtype, void* y, int out_dtype, int64_t rows, int64_t K, uint64_t seed,
                   void* stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || K % 16 != 0) return FP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP4_OK;
  if (!x || !y) return FP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return FP4_ERR_ALIGN;
  if (debug_on()) {
    const uint64_t n = (uint64_t)rows * (uint64_t)K;
    const int rc = debug_buffers({{x, n * elem_bytes(in_dtype)}, {y, n * elem_bytes(out_dtype)}});
    if (rc != FP4_OK) return rc;
  }
  return finish(launched(fp4::launch_hadamard16(x, in_dtype, y, out_dtype, rows, K, seed, as_stream(stream))),
                as_stream(stream));
}

int fp4_dequantize(const uint8_t* codes, const uint8_t* block_scales, const float* tensor_scale, int fmt, void* out,
                   int out_dtype, int64_t rows, int64_t K, void* stream) {
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  if (!dequantize_grid_fits(rows, K)) return FP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP4_OK;
  if (!codes || !block_scales || !out) return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && !tensor_scale) return FP4_ERR_NULL;
  if (!aligned(codes, is_mx8(fmt) ? 8 : 4) || !aligned(block_scales, 4) || !aligned(out, 16)) return FP4_ERR_ALIGN;
  if (debug_on()) {
    const int rc = debug_buffers({{codes, code_bytes(fmt, rows, K)},
                                  {block_scales, (uint64_t)fp4_scale_bytes(fmt, rows, K)},
                                  {fmt == FP4_NVFP4 ? tensor_scale : nullptr, 4u},
                                  {out, (uint64_t)rows * (uint64_t)K * elem_bytes(out_dtype)}});
    if (rc != FP4_OK) return rc;
  }
  return finish(launched(fp4::launch_dequantize(codes, block_scales, tensor_scale, fmt, out, out_dtype, rows, K,
                                                as_stream(stream))),
                as_stream(stream));
}

int fp4_gemm(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
             const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int fmt, int out_dtype, void* workspace,
             size_t workspace_bytes, void* stream) {
  if (!fmt_ok(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 32 != 0) return FP4_ERR_SHAPE;
  if (K > kMaxGemmK || !scales_fit(fmt, M, K) || !scales_fit(fmt, N, K)) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (!C) return FP4_ERR_NULL;
  if (K > 0 && (!A || !sA || !B || !sB)) return FP4_ERR_NULL;
  const bool nv = fmt == FP4_NVFP4;
  if (nv && (!tsA || !tsB)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sA, 4) || !aligned(sB, 4)) return FP4_ERR_ALIGN;
  if (!aligned(tsA, 4) || !aligned(tsB, 4)) return FP4_ERR_ALIGN;
  if (!aligned(C, out_dtype == FP4_F32 ? 4 : 2)) return FP4_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  if (debug_on()) {
    const int rc = debug_buffers({{A, code_bytes(fmt, M, K)},
                                  {sA, (uint64_t)fp4_scale_bytes(fmt, M, K)},
                                  {B, code_bytes(fmt, N, K)},
                                  {sB, (uint64_t)fp4_scale_bytes(fmt, N, K)},
                                  {nv ? tsA : nullptr, 4u},
                                  {nv ? tsB : nullptr, 4u},
                                  {C, (uint64_t)M * (uint64_t)N * elem_bytes(out_dtype)}});
    if (rc != FP4_OK) return rc;
  }
  if (nv && fp4::gemv_dot_applies(M, N, K)) {
    return finish(launched(fp4::launch_gemv_dot(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s)), s);
  }
  if (nv && fp4::gemv_bs_applies(M, N, K)) {
    return finish(launched(fp4::launch_gemv_bs(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s)), s);
  }
  if (nv && fp4::gemv_nv_applies(M, N, K)) {
    return finish(launched(fp4::launch_gemv_nv(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s)), s);
  }
  return finish(launched(fp4::launch_gemm_tiled(fmt, A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s)), s);
}

int fp4_gemm_ex(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                const float* tsB, const float* bias, int act, void* C, uint8_t* C_scales,
                const float* C_tensor_scale, int64_t M, int64_t N, int64_t K, int fmt, int out, void* stream) {
  if (!fmt_ok(fmt)) return FP4_ERR_FMT;
  if (out < FP4_OUT_F32 || out > FP4_OUT_NVFP4) return FP4_ERR_DTYPE;
  if (act != FP4_ACT_NONE && act != FP4_ACT_RELU) return FP4_ERR_FLAGS;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 32 != 0) return FP4_ERR_SHAPE;
  if (K > kMaxGemmK || !scales_fit(fmt, M, K) || !scales_fit(fmt, N, K)) return FP4_ERR_SHAPE;
  const bool fp4_out = out >= FP4_OUT_MXFP4;
  if (fp4_out && N % 32 != 0) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (!C) return FP4_ERR_NULL;
  if (fp4_out && !C_scales) return FP4_ERR_NULL;
  if (out == FP4_OUT_NVFP4 && !C_tensor_scale) return FP4_ERR_NULL;
  if (K > 0 && (!A || !sA || !B || !sB)) return FP4_ERR_NULL;
  const bool nv = fmt == FP4_NVFP4;
  if (nv && (!tsA || !tsB)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sA, 4) || !aligned(sB, 4)) return FP4_ERR_ALIGN;
  if (!aligned(tsA, 4) || !aligned(tsB, 4) || !aligned(bias, 16)) return FP4_ERR_ALIGN;
  if (out == FP4_OUT_NVFP4 && !aligned(C_tensor_scale, 4)) return FP4_ERR_ALIGN;
  if (fp4_out ? (!aligned(C, 16) || !aligned(C_scales, 4)) : !aligned(C, out == FP4_OUT_F32 ? 4 : 2))
    return FP4_ERR_ALIGN;
  if (debug_on()) {
    const int cfmt = out == FP4_OUT_NVFP4 ? FP4_NVFP4 : FP4_MXFP4;
    const uint64_t cbytes = fp4_out ? code_bytes(cfmt, M, N)
                                    : (uint64_t)M * (uint64_t)N * (out == FP4_OUT_F32 ? 4u : 2u);
    const int rc = debug_buffers({{A, code_bytes(fmt, M, K)},
                                  {sA, (uint64_t)fp4_scale_bytes(fmt, M, K)},
                                  {B, code_bytes(fmt, N, K)},
                                  {sB, (uint64_t)fp4_scale_bytes(fmt, N, K)},
                                  {nv ? tsA : nullptr, 4u},
                                  {nv ? tsB : nullptr, 4u},
                                  {bias, (uint64_t)N * 4u},
                                  {C, cbytes},
                                  {fp4_out ? C_scales : nullptr, (uint64_t)(fp4_out ? fp4_scale_bytes(cfmt, M, N) : 0)},
                                  {out == FP4_OUT_NVFP4 ? C_tensor_scale : nullptr, 4u}});
    if (rc != FP4_OK) return rc;
  }
  return finish(launched(fp4::launch_gemm_ex(nv ? FP4_NVFP4 : FP4_MXFP4, A, sA, B, sB, tsA, tsB, bias, act, C,
                                             C_scales, out == FP4_OUT_NVFP4 ? C_tensor_scale : nullptr, M, N, K,
                                             out, as_stream(stream))),
                as_stream(stream));
}

int fp4_gemm_grouped(const uint8_t* A, const uint8_t* sA, int64_t A_rows, const int32_t* row_idx,
                     const int32_t* group_off, int32_t E, const uint8_t* B, const uint8_t* sB, const float* tsA,
                     const float* tsB, void* C, int64_t total_rows, int64_t N, int64_t K, int fmt, int out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!fmt_ok(fmt) || !fp4::gemm_grouped_supports(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if (E < 0 || A_rows < 0 || total_rows < 0 || N < 0 || K < 0 || A_rows > kMaxDim || total_rows > kMaxDim ||
      N > kMaxDim || K > kMaxGemmK || K % 32 != 0)
    return FP4_ERR_SHAPE;
  if (!scales_fit(fmt, A_rows, K) || !scales_fit(fmt, N, K) || A_rows * (K / 2) > kMaxRange) return FP4_ERR_SHAPE;
  if (total_rows == 0 || N == 0 || E == 0) return FP4_OK;
  if (!C || !row_idx || !group_off) return FP4_ERR_NULL;
  if (K > 0 && (!A || !sA || !B || !sB)) return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && (!tsA || !tsB)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sA, 4) || !aligned(sB, 4) || !aligned(row_idx, 4) ||
      !aligned(group_off, 4) || !aligned(tsA, 4) || !aligned(tsB, 4))
    return FP4_ERR_ALIGN;
  if (!aligned(C, out_dtype == FP4_F32 ? 4 : 2)) return FP4_ERR_ALIGN;
  // The workspace is optional: NULL runs the GEMM on gathered rows; one of at
  // least fp4_workspace_size bytes first copies the rows into expert order.
  const size_t need = fp4::gemm_grouped_workspace(fmt, total_rows, N, K, E);
  if (workspace && workspace_bytes < need) return FP4_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 16)) return FP4_ERR_ALIGN;
  if (workspace && (uint64_t)total_rows * (uint64_t)(K / 2) > (uint64_t)kMaxRange) return FP4_ERR_SHAPE;
  if (debug_on()) {
    int rc = debug_buffers({{A, code_bytes(fmt, A_rows, K)},
                            {sA, (uint64_t)fp4_scale_bytes(fmt, A_rows, K)},
                            {fmt == FP4_NVFP4 ? tsA : nullptr, 4u},
                            {fmt == FP4_NVFP4 ? tsB : nullptr, (uint64_t)E * 4u},
                            {row_idx, (uint64_t)total_rows * 4u},
                            {group_off, ((uint64_t)E + 1u) * 4u},
                            {B, (uint64_t)E * code_bytes(fmt, N, K)},
                            {sB, (uint64_t)E * (uint64_t)fp4_scale_bytes(fmt, N, K)},
                            {C, (uint64_t)total_rows * (uint64_t)N * elem_bytes(out_dtype)},
                            {workspace, need}});
    if (rc == FP4_OK) rc = debug_groups(row_idx, group_off, E, total_rows, A_rows, as_stream(stream));
    if (rc != FP4_OK) return rc;
  }
  return finish(launched(fp4::launch_gemm_grouped(A, sA, A_rows, row_idx, group_off, E, B, sB, tsA, tsB, C,
                                                  total_rows, N, K, fmt, out_dtype, workspace, as_stream(stream))),
                as_stream(stream));
}

int fp4_gemm_nvfp4_act_supported(int64_t M, int64_t N, int64_t K, int x_dtype) {
  if (!dtype_ok(x_dtype) || M < 1 || N < 1 || K < 0 || K % 32 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK)
    return 0;
  return fp4::gemv_dot_applies(M, N, K) || fp4::gemv_bs_applies(M, N, K) ||
                 fp4::gemv_nv_fused_applies(M, N, K, x_dtype)
             ? 1
             : 0;
}

int fp4_gemm_nvfp4_act(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* W,
                       const uint8_t* sW, const float* tsW, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                       void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if ((flags & ~FP4_TS_GIVEN) != 0u) return FP4_ERR_FLAGS;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK || K % 32 != 0) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  const bool dot = fp4::gemv_dot_applies(M, N, K);
  const bool bs = !dot && fp4::gemv_bs_applies(M, N, K);
  if (!dot && !bs && !fp4::gemv_nv_fused_applies(M, N, K, x_dtype)) return FP4_ERR_SHAPE;
  if (!C || !tsW) return FP4_ERR_NULL;
  if (K > 0 && (!X || !W || !sW)) return FP4_ERR_NULL;
  if ((flags & FP4_TS_GIVEN) && !x_tensor_scale) return FP4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(sW, 4) || !aligned(tsW, 4) || !aligned(x_tensor_scale, 4))
    return FP4_ERR_ALIGN;
  if (!aligned(C, out_dtype == FP4_F32 ? 4 : 2)) return FP4_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  if (debug_on()) {
    const int rc = debug_buffers({{X, (uint64_t)M * (uint64_t)K * elem_bytes(x_dtype)},
                                  {x_tensor_scale, 4u},
                                  {W, code_bytes(FP4_NVFP4, N, K)},
                                  {sW, (uint64_t)fp4_scale_bytes(FP4_NVFP4, N, K)},
                                  {tsW, 4u},
                                  {C, (uint64_t)M * (uint64_t)N * elem_bytes(out_dtype)}});
    if (rc != FP4_OK) return rc;
  }
  if (dot)
    return finish(launched(fp4::launch_gemv_dot_fused(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K,
                                                      out_dtype, s)),
                  s);
  if (bs)
    return finish(launched(fp4::launch_gemv_bs_fused(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K,
                                                     out_dtype, s)),
                  s);
  return finish(launched(fp4::launch_gemv_nv_fused(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K,
                                                   out_dtype, s)),
                s);
}

int fp4_gemm_w4a8(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* bias,
                  int act, void* C, int64_t M, int64_t N, int64_t K, int out_dtype, void* stream) {
  if (!dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if (act != FP4_ACT_NONE && act != FP4_ACT_RELU) return FP4_ERR_FLAGS;
  // K <= 2^23 keeps a 256-row tile of FP8 codes inside one 32-bit buffer range.
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > (kMaxGemmK >> 1) || K % 32 != 0)
    return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (!C) return FP4_ERR_NULL;
  if (K > 0 && (!A || !sA || !B || !sB)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sA, 4) || !aligned(sB, 4) || !aligned(bias, 16))
    return FP4_ERR_ALIGN;
  if (!aligned(C, out_dtype == FP4_F32 ? 4 : 2)) return FP4_ERR_ALIGN;
  if (debug_on()) {
    const int rc = debug_buffers({{A, code_bytes(FP4_MXFP8, M, K)},
                                  {sA, (uint64_t)fp4_scale_bytes(FP4_MXFP8, M, K)},
                                  {B, code_bytes(FP4_MXFP4, N, K)},
                                  {sB, (uint64_t)fp4_scale_bytes(FP4_MXFP4, N, K)},
                                  {bias, (uint64_t)N * 4u},
                                  {C, (uint64_t)M * (uint64_t)N * elem_bytes(out_dtype)}});
    if (rc != FP4_OK) return rc;
  }
  return finish(launched(fp4::launch_gemm_w4a8(A, sA, B, sB, bias, act, C, M, N, K, out_dtype, as_stream(stream))),
                as_stream(stream));
}

const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "FP4_OK";
    case FP4_ERR_NULL: return "FP4_ERR_NULL: a required pointer is NULL";
    case FP4_ERR_SHAPE: return "FP4_ERR_SHAPE: invalid size or K not a multiple of the block";
    case FP4_ERR_ALIGN: return "FP4_ERR_ALIGN: pointer not aligned as required";
    case FP4_ERR_FMT: return "FP4_ERR_FMT: unknown or unsupported format";
    case FP4_ERR_DTYPE: return "FP4_ERR_DTYPE: unknown dtype";
    case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE: workspace missing or too small";
    case FP4_ERR_HIP: return "FP4_ERR_HIP: kernel launch failed";
    case FP4_ERR_FLAGS: return "FP4_ERR_FLAGS: unknown flag bits";
    case FP4_ERR_BOUNDS:
      return "FP4_ERR_BOUNDS: debug mode: a buffer is not device memory of the current device or smaller than "
             "the call needs, or a group offset or token index is out of range";
    default: return "unknown fp4 status";
  }
}

}  // extern "C"
