// abi.cpp -- the C ABI of libfp4 (declared in include/fp4.h): argument
// validation, kernel selection and launch on the caller's stream.
//
// Validation runs on the host before any HIP call, so every argument error is
// reported synchronously with a negative status and nothing is enqueued.
#include "../../include/fp4.h"
#include "fp4_launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// A 256-row operand tile must stay within one 32-bit buffer range.
constexpr int64_t kMaxGemmK = int64_t(1) << 24;

int launched(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

// The FP4 GEMM kernels address an operand's scale buffer (and the grouped
// kernel all of A) through 32-bit buffer ranges.
constexpr int64_t kMaxRange = (int64_t(1) << 32) - 1;
bool scales_fit(int fmt, int64_t rows, int64_t K) {
  return ((rows + 31) / 32) * ((K + 255) / 256) * (fmt == FP4_NVFP4 ? 512 : 256) <= kMaxRange;
}

}  // namespace

extern "C" {

int64_t fp4_scale_bytes(int fmt, int64_t rows, int64_t K) {
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (rows < 0 || K < 0 || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  // Tiles of 32 rows x 256 K values: 256 bytes (MXFP4, MXFP8) or 512 bytes (NVFP4).
  return ((rows + 31) / 32) * ((K + 255) / 256) * (fmt == FP4_NVFP4 ? 512 : 256);
}

size_t fp4_workspace_size(int op, int fmt, int64_t M, int64_t N, int64_t K, int32_t E) {
  switch (op) {
    case FP4_OP_QUANTIZE:
      return fmt == FP4_NVFP4 ? 8 : 0;
    case FP4_OP_GEMM:
      return 0;
    case FP4_OP_GEMM_GROUPED:
      return fp4::gemm_grouped_workspace(M, N, K, E);
    default:
      return 0;
  }
}

static int quantize_impl(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                         int64_t rows, int64_t K, int in_dtype, unsigned flags, void* workspace,
                         size_t workspace_bytes, uint64_t seed, void* stream) {
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(in_dtype)) return FP4_ERR_DTYPE;
  if (flags & ~(FP4_TS_GIVEN | FP4_Q_SR | FP4_Q_2D)) return FP4_ERR_FLAGS;
  if ((flags & FP4_Q_2D) && fmt != FP4_NVFP4) return FP4_ERR_FMT;
  if ((flags & FP4_Q_SR) && is_mx8(fmt)) return FP4_ERR_FMT;
  const bool sr = (flags & FP4_Q_SR) != 0u, twod = (flags & FP4_Q_2D) != 0u;
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  if (rows * K > (int64_t(1) << 40)) return FP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP4_OK;
  if (!x || !codes || !block_scales) return FP4_ERR_NULL;
  const bool nv = fmt == FP4_NVFP4;
  if (nv && !tensor_scale) return FP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, is_mx8(fmt) ? 8 : 4) || !aligned(block_scales, 4)) return FP4_ERR_ALIGN;
  if (nv && !aligned(tensor_scale, 4)) return FP4_ERR_ALIGN;
  const bool compute_ts = nv && !(flags & FP4_TS_GIVEN);
  if (compute_ts) {
    if (!workspace || workspace_bytes < 8) return FP4_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return FP4_ERR_ALIGN;
  }
  hipStream_t s = as_stream(stream);
  if (compute_ts && !twod && fp4::quantize_nv_small_applies(rows, K, in_dtype))
    return launched(
        fp4::launch_quantize_nv_small(x, in_dtype, codes, block_scales, tensor_scale, rows, K, sr, seed, s));
  if (compute_ts) {
    int rc = launched(fp4::launch_tensor_amax(x, in_dtype, rows * K, static_cast<uint32_t*>(workspace), tensor_scale, s));
    if (rc != FP4_OK) return rc;
  }
  if (twod)
    return launched(fp4::launch_quantize_nv2d(x, in_dtype, codes, block_scales, tensor_scale, rows, K, sr, seed, s));
  return launched(fp4::launch_quantize(x, fmt, in_dtype, codes, block_scales, tensor_scale, rows, K, sr, seed, s));
}

int fp4_quantize(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                 int64_t rows, int64_t K, int in_dtype, unsigned flags, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (flags & ~FP4_TS_GIVEN) return FP4_ERR_FLAGS;
  return quantize_impl(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, workspace,
                       workspace_bytes, 0ull, stream);
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
  return launched(fp4::launch_hadamard16(x, in_dtype, y, out_dtype, rows, K, seed, as_stream(stream)));
}

int fp4_dequantize(const uint8_t* codes, const uint8_t* block_scales, const float* tensor_scale, int fmt, void* out,
                   int out_dtype, int64_t rows, int64_t K, void* stream) {
  if (!qfmt_ok(fmt)) return FP4_ERR_FMT;
  if (!dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || K % block_of(fmt) != 0) return FP4_ERR_SHAPE;
  if (rows * K > (int64_t(1) << 40)) return FP4_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP4_OK;
  if (!codes || !block_scales || !out) return FP4_ERR_NULL;
  if (fmt == FP4_NVFP4 && !tensor_scale) return FP4_ERR_NULL;
  if (!aligned(codes, is_mx8(fmt) ? 8 : 4) || !aligned(block_scales, 4) || !aligned(out, 16)) return FP4_ERR_ALIGN;
  return launched(fp4::launch_dequantize(codes, block_scales, tensor_scale, fmt, out, out_dtype, rows, K,
                                         as_stream(stream)));
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
  if (nv && fp4::gemv_bs_applies(M, N, K)) {
    return launched(fp4::launch_gemv_bs(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s));
  }
  if (nv && fp4::gemv_nv_applies(M, N, K)) {
    return launched(fp4::launch_gemv_nv(A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s));
  }
  return launched(fp4::launch_gemm_tiled(fmt, A, sA, B, sB, tsA, tsB, C, M, N, K, out_dtype, s));
}

int fp4_gemm_ex(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                const float* tsB, const float* bias, int act, void* C, uint8_t* C_scales, int64_t M, int64_t N,
                int64_t K, int fmt, int out, void* stream) {
  if (!fmt_ok(fmt)) return FP4_ERR_FMT;
  if (out < FP4_OUT_F32 || out > FP4_OUT_MXFP4_OCP) return FP4_ERR_DTYPE;
  if (act != FP4_ACT_NONE && act != FP4_ACT_RELU) return FP4_ERR_FLAGS;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 32 != 0) return FP4_ERR_SHAPE;
  if (K > kMaxGemmK || !scales_fit(fmt, M, K) || !scales_fit(fmt, N, K)) return FP4_ERR_SHAPE;
  const bool fp4_out = out >= FP4_OUT_MXFP4;
  if (fp4_out && N % 32 != 0) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (!C) return FP4_ERR_NULL;
  if (fp4_out && !C_scales) return FP4_ERR_NULL;
  if (K > 0 && (!A || !sA || !B || !sB)) return FP4_ERR_NULL;
  const bool nv = fmt == FP4_NVFP4;
  if (nv && (!tsA || !tsB)) return FP4_ERR_NULL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sA, 4) || !aligned(sB, 4)) return FP4_ERR_ALIGN;
  if (!aligned(tsA, 4) || !aligned(tsB, 4) || !aligned(bias, 16)) return FP4_ERR_ALIGN;
  if (fp4_out ? (!aligned(C, 16) || !aligned(C_scales, 4)) : !aligned(C, out == FP4_OUT_F32 ? 4 : 2))
    return FP4_ERR_ALIGN;
  return launched(fp4::launch_gemm_ex(nv ? FP4_NVFP4 : FP4_MXFP4, A, sA, B, sB, tsA, tsB, bias, act, C, C_scales,
                                      M, N, K, out, as_stream(stream)));
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
  const size_t need = fp4::gemm_grouped_workspace(total_rows, N, K, E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FP4_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return FP4_ERR_ALIGN;
  return launched(fp4::launch_gemm_grouped(A, sA, A_rows, row_idx, group_off, E, B, sB, tsA, tsB, C, total_rows, N,
                                           K, fmt, out_dtype, workspace, as_stream(stream)));
}

int fp4_gemm_nvfp4_act_supported(int64_t M, int64_t N, int64_t K, int x_dtype) {
  if (!dtype_ok(x_dtype) || M < 1 || N < 1 || K < 0 || K % 32 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK)
    return 0;
  return fp4::gemv_bs_applies(M, N, K) || fp4::gemv_nv_fused_applies(M, N, K, x_dtype) ? 1 : 0;
}

int fp4_gemm_nvfp4_act(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* W,
                       const uint8_t* sW, const float* tsW, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                       void* stream) {
  if (!dtype_ok(x_dtype) || !dtype_ok(out_dtype)) return FP4_ERR_DTYPE;
  if ((flags & ~FP4_TS_GIVEN) != 0u) return FP4_ERR_FLAGS;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxGemmK || K % 32 != 0) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  const bool bs = fp4::gemv_bs_applies(M, N, K);
  if (!bs && !fp4::gemv_nv_fused_applies(M, N, K, x_dtype)) return FP4_ERR_SHAPE;
  if (!C || !tsW) return FP4_ERR_NULL;
  if (K > 0 && (!X || !W || !sW)) return FP4_ERR_NULL;
  if ((flags & FP4_TS_GIVEN) && !x_tensor_scale) return FP4_ERR_NULL;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(sW, 4) || !aligned(tsW, 4) || !aligned(x_tensor_scale, 4))
    return FP4_ERR_ALIGN;
  if (!aligned(C, out_dtype == FP4_F32 ? 4 : 2)) return FP4_ERR_ALIGN;
  if (bs)
    return launched(fp4::launch_gemv_bs_fused(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K, out_dtype,
                                              as_stream(stream)));
  return launched(fp4::launch_gemv_nv_fused(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K, out_dtype,
                                            as_stream(stream)));
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
  return launched(fp4::launch_gemm_w4a8(A, sA, B, sB, bias, act, C, M, N, K, out_dtype, as_stream(stream)));
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
    default: return "unknown fp4 status";
  }
}

}  // extern "C"
