// fp4_launch.h -- host-side launch entry points of the libfp4 kernels.
// Internal header shared by the C-ABI layer (abi.cpp) and the kernel files.
// Every function enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

// Scratch held by the library for fp4_quantize_noalloc (quantize.hip): the
// current device's copy of a static device array of kScratchBytes, found
// with hipGetSymbolAddress on the first call per device (which also clears
// it on `stream`).  At most kMaxDevices devices.
constexpr uint32_t kScratchBytes = 256;
constexpr uint32_t kMaxDevices = 64;
hipError_t scratch_for_current_device(hipStream_t stream, void** ptr);

// Quantisation (quantize.hip).
hipError_t launch_tensor_amax(const void* x, int in_dtype, int64_t n, uint32_t* ws, float* tensor_scale,
                              hipStream_t stream);
// NVFP4 with its own tensor scale in one launch, for inputs of at most 256 KB
// (every workgroup reduces the whole maximum itself).
bool quantize_nv_small_applies(int64_t rows, int64_t K, int in_dtype);
hipError_t launch_quantize_nv_small(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales,
                                    float* tensor_scale, int64_t rows, int64_t K, bool sr, uint64_t seed,
                                    hipStream_t stream);
// NVFP4 with its own tensor scale in one launch for inputs above 256 KB and
// at most 1 MB: workgroups exchange the maximum through ws (3 words, zero
// before the call and after it).  spin_limit 0 takes the default wait.
bool quantize_nv_grid_applies(int64_t rows, int64_t K, int in_dtype);
hipError_t launch_quantize_nv_grid(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales,
                                   float* tensor_scale, uint32_t* ws, int64_t rows, int64_t K, bool sr, uint64_t seed,
                                   uint32_t spin_limit, hipStream_t stream);
// NVFP4 with 16 x 16 patch scales (tensor scale already in *tensor_scale).
hipError_t launch_quantize_nv2d(const void* x, int in_dtype, uint8_t* codes, uint8_t* scales,
                                const float* tensor_scale, int64_t rows, int64_t K, bool sr, uint64_t seed,
                                hipStream_t stream);
// y = random Hadamard transform of x on 16-value blocks along K.
hipError_t launch_hadamard16(const void* x, int in_dtype, void* y, int out_dtype, int64_t rows, int64_t K,
                             uint64_t seed, hipStream_t stream);
// sr: round the elements stochastically (Philox4x64-10 words keyed by seed).
hipError_t launch_quantize(const void* x, int fmt, int in_dtype, uint8_t* codes, uint8_t* scales,
                           const float* tensor_scale, int64_t rows, int64_t K, bool sr, uint64_t seed,
                           hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int fmt,
                             void* out, int out_dtype, int64_t rows, int64_t K, hipStream_t stream);

// Tiled GEMM, MXFP4 (block-scaled FP4 matrix core) or NVFP4 (exact FP16
// decode) (gemm.hip).
// Dense GEMM with the full epilogue: + bias[N] (or nullptr), ReLU (act 1),
// output 0 FP32, 1 BF16, 2 MXFP4 (ceil rule) / 3 MXFP4 (OCP rule) / 4 NVFP4
// under the given tensor scale *tsC, along N: codes into C (M x N/2), scale
// tiles into Cs (N % 32 == 0, C 16-byte aligned).
hipError_t launch_gemm_ex(int fmt, const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, const float* bias, int act, void* C, uint8_t* Cs,
                          const float* tsC, int64_t M, int64_t N, int64_t K, int out, hipStream_t stream);
hipError_t launch_gemm_tiled(int fmt, const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                             const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                             int out_dtype, hipStream_t stream);

// Grouped (mixture-of-experts) GEMM over the same tiles (gemm.hip).
bool gemm_grouped_supports(int fmt);
// Bytes of the optional workspace: the token rows gathered into output-row
// order (codes, then scale tiles).
size_t gemm_grouped_workspace(int fmt, int64_t total_rows, int64_t N, int64_t K, int32_t E);
hipError_t launch_gemm_grouped(const uint8_t* A, const uint8_t* sA, int64_t A_rows, const int32_t* row_idx,
                               const int32_t* group_off, int32_t E, const uint8_t* B, const uint8_t* sB,
                               const float* tsA, const float* tsB, void* C, int64_t total_rows, int64_t N,
                               int64_t K, int fmt, int out_dtype, void* workspace, hipStream_t stream);

// NVFP4 decode GEMV / skinny GEMM for M <= 32 (gemv_nv.hip).
bool gemv_nv_applies(int64_t M, int64_t N, int64_t K);
// MXFP8 (A) x MXFP4 (B) tiled GEMM with the bias / ReLU epilogue; out 0 FP32,
// 1 BF16.
hipError_t launch_gemm_w4a8(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                            const float* bias, int act, void* C, int64_t M, int64_t N, int64_t K, int out,
                            hipStream_t stream);

hipError_t launch_gemv_nv(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB,
                          const float* tsA, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                          int out_dtype, hipStream_t stream);

// NVFP4 decode GEMV for M = 1 and K <= 8192 on the vector ALU, weights read
// in whole 1 KB row pieces (gemv_nv_dot.hip); it takes precedence over the
// kernels below and, like them, serves the pre-quantised and the
// fused-activation calls alike, so that the two return the same bits.
bool gemv_dot_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_dot(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                           const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                           hipStream_t stream);
hipError_t launch_gemv_dot_fused(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* B,
                                 const uint8_t* sB, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                                 int out_dtype, hipStream_t stream);

// NVFP4 decode GEMV for M <= 8 on the FP4 x FP4 matrix core with the block
// scales applied to exact block sums (gemv_nv_blocksum.hip); when it applies
// it serves both the pre-quantised and the fused-activation calls, so that
// the two return the same bits.
bool gemv_bs_applies(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_bs(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                          const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                          hipStream_t stream);
hipError_t launch_gemv_bs_fused(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* B,
                                const uint8_t* sB, const float* tsB, void* C, int64_t M, int64_t N, int64_t K,
                                int out_dtype, hipStream_t stream);

// The same with the activation quantised inside the kernel (small M x K).
bool gemv_nv_fused_applies(int64_t M, int64_t N, int64_t K, int x_dtype);
hipError_t launch_gemv_nv_fused(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags,
                                const uint8_t* B, const uint8_t* sB, const float* tsB, void* C, int64_t M,
                                int64_t N, int64_t K, int out_dtype, hipStream_t stream);

}  // namespace fp4
