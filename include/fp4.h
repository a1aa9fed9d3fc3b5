/*
 * fp4.h -- C ABI of libfp4: FP4 (E2M1) block-scaled quantisation and matrix
 * multiply on AMD Instinct MI355X (gfx950).
 *
 * The operation, as the sources state it:
 *   - E2M1 elements {0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6}, one scale per block
 *     chosen so the block's largest magnitude maps to 6 (Ultralytics glossary
 *     "FP4", "How FP4 works");
 *   - MXFP4: 32-value blocks, power-of-two E8M0 scale; NVFP4: 16-value blocks,
 *     E4M3 scale plus one FP32 per-tensor scale (NVFP4 video transcript,
 *     prism.simon-ai.net; glossary "How FP4 works");
 *   - the GEMM accumulates in FP32 and multiplies by the product of the scales,
 *     C = (A_fp4 * B_fp4) * (scaleA * scaleB) ("Rubin FP4 GEMM deep dive",
 *     yfxerp.com, §1.1, §3.1, §4.2);
 *   - two FP4 values per byte with an explicitly fixed order, scales stored in
 *     the order the kernel tiles read them (same page, §4.2, §5.2);
 *   - weights and activations may take different precisions, FP8 activations
 *     beside FP4 weights (same page, §3.4), here MXFP8: E4M3 elements under
 *     the MXFP4 block scales (§3.1 names MXFP8 among the MX formats).
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers (hipMalloc'd or equivalent) unless
 *     stated otherwise; `stream` is a hipStream_t passed as void* (NULL = the
 *     null stream).  Every call is asynchronous on `stream`: it enqueues work
 *     and returns; nothing is copied to or from the host, no call synchronises.
 *   - The caller owns and allocates every buffer, workspace included.  The
 *     library never allocates or frees memory and keeps no global mutable
 *     state, with one exception: fp4_quantize_noalloc's scratch array, a
 *     static device array of 256 bytes on each GPU the library runs on.
 *   - Argument errors return a negative fp4_status before any HIP call is made,
 *     so they are reported synchronously and leave the stream untouched.  A
 *     failed kernel launch returns FP4_ERR_HIP.  Faults inside a kernel surface
 *     at the caller's next synchronisation.  Debug mode (fp4_set_debug,
 *     FP4_DEBUG) adds checks that make HIP calls and synchronise.
 *   - Format, dtype, output, activation and operation arguments are declared
 *     int and take the values of the enums below.  A C enum's underlying type
 *     is up to the compiler (-fshort-enums makes it one byte), while int is the
 *     same for every compiler and for foreign-function callers; any other value
 *     is refused with FP4_ERR_FMT, FP4_ERR_DTYPE or FP4_ERR_FLAGS.
 *   - Matrices are row-major.  A quantised matrix of `rows` x `K` values is
 *       codes:  rows * K/2 bytes; element k of a row is in byte k/2, bits 0-3
 *               for even k and bits 4-7 for odd k; a code is sign<<3 | magnitude
 *               with magnitude 0..7 -> 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 *       scales: fp4_scale_bytes(fmt, rows, K) bytes in the tiled layout below;
 *       tensor scale (NVFP4 only): one FP32 in device memory.
 *     MXFP8 codes are rows * K bytes instead, one E4M3 byte per element
 *     (sign<<7 | exponent<<3 | mantissa, bias 7, largest value 448; the NaN
 *     patterns 0x7F / 0xFF are never written and not supported as input).
 *   - Element value: MXFP4  E2M1(code) * 2^(scale_byte - 127);
 *                    MXFP8  E4M3(code) * 2^(scale_byte - 127);
 *                    NVFP4  E2M1(code) * E4M3(scale_byte) * tensor_scale.
 *
 * Tiled scale layout (identical for A and B operands; both are "rows x K").
 *   Scales are grouped in tiles of 32 rows x 256 K values, stored row-tile
 *   major: tile (rt, kt) starts at byte T * (rt * ceil(K/256) + kt), with tile
 *   size T = 256 (MXFP4 and MXFP8: 8 blocks of 32) or 512 (NVFP4: 16 blocks
 *   of 16).
 *   Inside a tile, row i (0..31) and 32-value K chunk c (0..7) belong to lane
 *   L = 32 * (c % 2) + i and sub-step s = c / 2 -- the lane order of the 32x32
 *   matrix-core operand, where lane 32*j + i carries row i's chunk j of each
 *   64-value K sub-step:
 *     MXFP4, MXFP8: lane L owns bytes 4L..4L+3; byte 4L + s is the chunk's
 *            E8M0 scale;
 *     NVFP4: lane L owns bytes 8L..8L+7; bytes 8L + 2s and 8L + 2s + 1 are the
 *            E4M3 scales of the chunk's first and second 16-value block.
 *   One dword (MXFP4) or two (NVFP4) per lane thus carry a wavefront's scales
 *   for four K sub-steps.  Bytes of rows >= `rows` or of blocks past K are
 *   padding: the quantiser writes them as 0, and the GEMMs rely on that (a
 *   zero scale makes the codes read past the end of K contribute nothing), so
 *   hand-built scale buffers must keep padding bytes 0.  E8M0 byte 0xFF (NaN)
 *   is never produced and not supported as input.
 */
#ifndef FP4_H_
#define FP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block format. */
enum fp4_fmt {
    FP4_MXFP4 = 0,     /* 32-blocks, E8M0; exponent = smallest e with amax <= 6*2^e */
    FP4_NVFP4 = 1,     /* 16-blocks, E4M3 (bias 7, max 448) + FP32 tensor scale      */
    FP4_MXFP4_OCP = 2, /* 32-blocks, E8M0; exponent = floor(log2 amax) - 2, saturate */
    FP4_MXFP8 = 3,     /* 32-blocks, E8M0, E4M3 elements; smallest e with amax <= 448*2^e */
    FP4_MXFP8_OCP = 4  /* 32-blocks, E8M0, E4M3 elements; floor(log2 amax) - 8, saturate */
};

/* Element type of unquantised inputs and of outputs. */
enum fp4_dtype { FP4_F32 = 0, FP4_BF16 = 1 };

/* Operation selector for fp4_workspace_size. */
enum fp4_op { FP4_OP_QUANTIZE = 0, FP4_OP_GEMM = 1, FP4_OP_GEMM_GROUPED = 2 };

/* Output of fp4_gemm_ex: FP32 or BF16 (the fp4_dtype values), or the product
 * quantised again to MXFP4 along N (ceil or OCP exponent rule, as
 * FP4_MXFP4 / FP4_MXFP4_OCP) or to NVFP4 along N under a given tensor scale. */
enum fp4_out { FP4_OUT_F32 = 0, FP4_OUT_BF16 = 1, FP4_OUT_MXFP4 = 2, FP4_OUT_MXFP4_OCP = 3, FP4_OUT_NVFP4 = 4 };

/* Activation of fp4_gemm_ex. */
enum fp4_act { FP4_ACT_NONE = 0, FP4_ACT_RELU = 1 };

/* Flags for fp4_quantize. */
#define FP4_TS_GIVEN 1u /* NVFP4: read the tensor scale from *tensor_scale instead of computing it */
/* More flags for fp4_quantize_ex. */
#define FP4_Q_SR 2u     /* round the elements stochastically (as fp4_quantize_sr)          */
#define FP4_Q_2D 4u     /* NVFP4 only: one block scale per 16 x 16 patch (2-D scaling)      */

enum fp4_status {
    FP4_OK = 0,
    FP4_ERR_NULL = -1,      /* a required pointer is NULL                          */
    FP4_ERR_SHAPE = -2,     /* negative size, K not a multiple of the block, ...   */
    FP4_ERR_ALIGN = -3,     /* a pointer is not aligned as documented              */
    FP4_ERR_FMT = -4,       /* unknown fmt, or fmt not supported by this operation */
    FP4_ERR_DTYPE = -5,     /* unknown dtype                                       */
    FP4_ERR_WORKSPACE = -6, /* workspace missing or smaller than required          */
    FP4_ERR_HIP = -7,       /* a HIP launch failed                                 */
    FP4_ERR_FLAGS = -8,     /* unknown flag bits                                   */
    FP4_ERR_BOUNDS = -9     /* debug mode only: a buffer is not memory of the      */
                            /* current device or smaller than the call needs, or   */
                            /* a group offset or token index is out of range       */
};

/* Debug mode, for callers hunting a fault or a wrong result: on when the
 * environment variable FP4_DEBUG is set to anything but "0" when the library
 * is first used, or after fp4_set_debug(1).  Then every entry point, after its argument checks:
 *   - checks that each buffer it reads or writes lies wholly inside one device
 *     allocation of the current device (hipMemGetAddressRange; a caching
 *     allocator's block counts as one allocation), else FP4_ERR_BOUNDS;
 *   - fp4_gemm_grouped waits for the stream, copies group_off and row_idx to
 *     the host and checks them as documented there, else FP4_ERR_BOUNDS;
 *   - waits for its kernels (hipStreamSynchronize), so that a launch or
 *     execution error is returned by the call that caused it (FP4_ERR_HIP).
 * The checks make HIP calls and synchronise, and the grouped check allocates
 * host memory; none of this happens with debug mode off.  Returns the previous
 * setting (0 or 1).  Host-only; the setting is process-wide. */
int fp4_set_debug(int on);

/* Size in bytes of the tiled scale buffer of a rows x K matrix, or a negative
 * fp4_status for an invalid fmt or shape.  Host-only, no HIP call. */
int64_t fp4_scale_bytes(int fmt, int64_t rows, int64_t K);

/* Workspace bytes an operation needs (0 if none).  For FP4_OP_QUANTIZE, M is
 * the row count; for FP4_OP_GEMM_GROUPED, E is the expert count and M the total
 * routed rows.  NVFP4 quantisation that computes its own tensor scale needs 16
 * bytes (the running amax and two workgroup counters); fp4_gemm returns 0.
 * FP4_OP_GEMM_GROUPED returns the size of an OPTIONAL workspace (MXFP4
 * formats; 0 for NVFP4): given one, fp4_gemm_grouped first copies the routed
 * token rows into expert order there, which makes the GEMM faster; it needs
 * no zero-fill (it holds no control words).  Operations keep their control words at the start of the
 * workspace.  A workspace must be zero-filled once before its first use; every
 * call leaves the control words zero again when its work on the stream
 * completes, so one zero-filled workspace of the largest size needed serves
 * any sequence of calls.  Calls that share one workspace must be ordered (same
 * stream, or events); calls that overlap on one workspace race.  Host-only. */
size_t fp4_workspace_size(int op, int fmt, int64_t M, int64_t N, int64_t K, int32_t E);

/* Quantise a rows x K matrix x (K contiguous) of `in_dtype` (FP32 or BF16).
 *   Per block: MXFP4 picks an E8M0 exponent from the block's largest magnitude
 *   (MXFP8: the same rules with 448 in place of 6, elements y = x * 2^-e
 *   rounded to the nearest E4M3 value, ties to even, saturating at 448);
 *   NVFP4 takes r = (amax_block / 6) / tensor_scale, rounds it to E4M3 (nearest
 *   even, saturating at 448), and divides by d = E4M3(r) * tensor_scale (FP32).
 *   Each element is then rounded to the nearest E2M1 value, ties to even,
 *   saturating at 6; the sign bit is copied (-0 gives code 8).
 *   NVFP4 tensor scale: unless flags has FP4_TS_GIVEN, computed over the whole
 *   matrix as s_t = amax / 2688 (6 * 448), s_t = 1 for an all-zero matrix and
 *   s_t >= FLT_MIN, and written to *tensor_scale.  With FP4_TS_GIVEN the caller's
 *   value is used (it must be a positive, finite, normal FP32).
 *   (Sources: glossary "How FP4 works"; NVFP4 video transcript.)
 * Requirements: K % bs == 0 (32 for MXFP4 and MXFP8, 16 for NVFP4); x 16-byte
 *   aligned; codes 4-byte (MXFP8: 8-byte) and block_scales 4-byte aligned.  tensor_scale must be non-NULL for NVFP4 and
 *   is ignored for MXFP4.  NVFP4 without FP4_TS_GIVEN needs a workspace of
 *   fp4_workspace_size(FP4_OP_QUANTIZE, ...) bytes; otherwise workspace may be NULL.
 *   (Inputs of at most 256 KB take a single launch in which every workgroup
 *   reduces the maximum itself and the workspace is left untouched; up to 1 MB,
 *   a single launch whose workgroups exchange the maximum through the
 *   workspace and wait for each other (a bounded wait, after which a
 *   workgroup reduces the whole maximum itself); larger ones reduce across
 *   workgroups through the workspace, then quantise.  All give the same
 *   bits.  A test hook: the environment variable FP4_TEST_NV_GRID_SPIN, a
 *   positive count, caps that wait, so that tests reach the path of a
 *   workgroup that stops waiting.)
 * rows == 0 or K == 0 is a no-op. */
int fp4_quantize(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                 int64_t rows, int64_t K, int in_dtype, unsigned flags, void* workspace,
                 size_t workspace_bytes, void* stream);

/* fp4_quantize for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, rules, errors and bits as fp4_quantize (flags:
 * FP4_TS_GIVEN only), without the workspace: where fp4_quantize would use one
 * (NVFP4 computing its own tensor scale over more than 256 KB of input), the
 * running maximum and workgroup counters live in a scratch array the library
 * holds, a static device array of 256 bytes on each GPU (held until the
 * process ends).  The call allocates nothing and calls no allocating
 * routine.
 *   The first call on a device looks the array up for that device (which must
 *   be current) and enqueues a one-workgroup kernel on `stream` that clears
 *   it; every later call leaves its control words zero when its work
 *   completes.
 *   All calls on one GPU share that GPU's array: calls that may run at the
 *   same time on one GPU (different streams, no ordering between them) race
 *   and give wrong tensor scales.  Order them, or use fp4_quantize with a
 *   workspace per stream.
 * Errors: as fp4_quantize; FP4_ERR_WORKSPACE if the operation needed more
 * than the array's 256 bytes (no format needs more than 16 today);
 * FP4_ERR_HIP if the array cannot be located on the current device or the
 * clearing kernel fails to launch. */
int fp4_quantize_noalloc(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                         int64_t rows, int64_t K, int in_dtype, unsigned flags, void* stream);

/* fp4_quantize with stochastic rounding of the elements (NVFP4 video
 * transcript, the training recipe's fourth part: a value between two
 * representable points goes up with probability equal to its distance from
 * the lower one, so the expectation is kept -- meant for gradients).  The
 * block and tensor scales are chosen exactly as by fp4_quantize; only the
 * E2M1 rounding of each scaled value y changes:
 *   lo = the largest grid value <= |y| (|y| >= 6 gives 6), hi the next one;
 *   the code is hi iff u * (hi - lo) < |y| - lo, with u = (w >> 8) * 2^-24 and
 *   w the element's 32-bit random word; the sign bit is copied.
 * Random words: Philox4x64-10 (Salmon et al., "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011) with key (seed, 0); element i of the matrix
 * (row-major, i = r * K + k) takes word (i mod 8) / 2 of the block with
 * counter (i / 8, 0, 0, 0), its low 32 bits for even i.  The result is a
 * function of (x, seed) alone.  FP4 formats only (MXFP8: FP4_ERR_FMT).
 * Arguments and errors as fp4_quantize. */
int fp4_quantize_sr(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                    int64_t rows, int64_t K, int in_dtype, unsigned flags, uint64_t seed, void* workspace,
                    size_t workspace_bytes, void* stream);

/* fp4_quantize with options (flags may combine):
 *   FP4_TS_GIVEN: as in fp4_quantize.
 *   FP4_Q_SR: stochastic rounding of the elements with `seed`, exactly as
 *     fp4_quantize_sr.
 *   FP4_Q_2D (NVFP4 only, else FP4_ERR_FMT): 2-D block scaling (NVFP4 video
 *     transcript, the training recipe's second part: a weight matrix is used
 *     as W forward and as W^T backward, so one scale serves a 16 x 16 patch
 *     and both directions quantise alike).  The patch of rows 16p..16p+15
 *     (those inside the matrix) and columns 16b..16b+15 takes the E4M3 scale
 *     of its largest magnitude, written for each of its rows in the usual
 *     layout; rows past the matrix keep scale byte 0.  W and W^T then
 *     dequantise to exact transposes of each other (rows and K multiples of
 *     16).  The tensor scale is the usual one.
 * seed is ignored without FP4_Q_SR.  Arguments and errors otherwise as
 * fp4_quantize. */
int fp4_quantize_ex(const void* x, int fmt, uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                    int64_t rows, int64_t K, int in_dtype, unsigned flags, uint64_t seed, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Random Hadamard transform (NVFP4 video transcript, the training recipe's
 * third part: values are mixed within a block so that an outlier no longer
 * sets the block scale alone; the transform is orthogonal, so norms and dot
 * products survive).  On every 16-value block along K of the rows x K matrix
 * x: y = (1/4) H16 D x, where D holds the signs of the columns (-1 where the
 * top bit of column k's Philox4x64-10 word under `seed` -- the word
 * fp4_quantize_sr gives element k of a one-row matrix -- is set), and H16 is
 * the 16-point Walsh-Hadamard matrix evaluated as FP32 butterflies
 * (a + b, a - b) of distance 1, 2, 4, 8 in that order; the 1/4 is exact.
 * Two matrices transformed with one seed keep their products along K, so
 * transforming both GEMM operands leaves the product unchanged up to
 * rounding.  x: FP32 or BF16 (in_dtype); y: FP32 or BF16 (out_dtype, round to
 * nearest even), may equal x when the dtypes agree.  K % 16 == 0; x and y
 * 16-byte aligned.  rows == 0 or K == 0 is a no-op. */
int fp4_hadamard16(const void* x, int in_dtype, void* y, int out_dtype, int64_t rows, int64_t K, uint64_t seed,
                   void* stream);

/* Dequantise codes + scales (+ NVFP4 tensor scale) to a rows x K matrix of
 * `out_dtype` (value = E2M1 code x block scale, x tensor scale for NVFP4:
 * Ultralytics glossary "FP4", "How FP4 works"; "Rubin FP4 GEMM deep dive"
 * §3.1; NVFP4 video transcript).  MXFP4 values are exact; NVFP4 computes (E2M1 * E4M3), exact,
 * times tensor_scale with one FP32 rounding; BF16 output is the round-to-
 * nearest-even of that FP32 value.  MXFP8 values are exact.  Same alignment
 * rules as fp4_quantize. */
int fp4_dequantize(const uint8_t* codes, const uint8_t* block_scales, const float* tensor_scale, int fmt,
                   void* out, int out_dtype, int64_t rows, int64_t K, void* stream);

/* C[M x N] = (sum_k A[m,k] * B[n,k]) * tsA * tsB, accumulated in FP32
 * ("Rubin FP4 GEMM deep dive" §3.1-§3.2, §4.2: products of the block-scaled
 * FP4 operands, FP32 accumulation, the scales applied to the result; §4.4 the
 * interface; §1.2, §6.2 decode streams the weights).
 *   A: M x K quantised (codes + scales), B: N x K quantised (each row of B is one
 *   output column, i.e. B is the weight matrix stored K-contiguous).
 *   tsA, tsB: device FP32 tensor scales; required for NVFP4, optional (NULL = 1)
 *   for MXFP4.  C: M x N row-major, FP32 or BF16 (round to nearest even).
 *   MXFP4 runs on the gfx950 block-scaled FP4 matrix core with the E8M0 scales
 *   applied inside the instruction; NVFP4 decodes E2M1 * E4M3 exactly to FP16
 *   and runs the FP16 matrix core, with the tensor scales in the epilogue.
 *   NVFP4 with M <= 32 (decode shapes) takes a bandwidth-first path with
 *   sums in a fixed order (results do not depend on timing) and no workspace.
 *   M = 1 with K <= 8192 runs on the vector ALU (16 weight rows per
 *   workgroup, each thread one 32-value chunk of every row, exact block sums
 *   from FP16 dot products); otherwise one workgroup per 32 weight rows, K
 *   split over its wavefronts.  For M <= 8 the FP4 x FP4 matrix core forms each pair of 16-value blocks'
 *   exact dot product and the E4M3 scales multiply those block sums in FP32
 *   (K up to 8192 at M = 5..8, 16384 at M = 2..4, 32768 at M = 1); otherwise
 *   the weights are decoded to FP16 while the activation fits the
 *   workgroup's staging memory (for example M <= 8 with K <= 8960, or any
 *   M <= 32 with K <= 8192); larger shapes take the tiled kernel.
 * Formats: the FP4 ones (MXFP8 operands: fp4_gemm_w4a8).
 * Requirements: K % 32 == 0 (both formats); codes 16-byte aligned; scales
 *   4-byte aligned; C aligned to its element size.  M, N >= 0 arbitrary, as
 *   long as each operand's scale buffer stays below 4 GiB (at K = 8192:
 *   2^24 rows for MXFP4, 2^23 for NVFP4).
 *   workspace: fp4_workspace_size(FP4_OP_GEMM, fmt, M, N, K, 0) bytes,
 *   zero-filled before first use (0 bytes -> NULL is fine).
 * M == 0 or N == 0 is a no-op; K == 0 writes zeros. */
int fp4_gemm(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
             const float* tsB, void* C, int64_t M, int64_t N, int64_t K, int fmt, int out_dtype,
             void* workspace, size_t workspace_bytes, void* stream);

/* Grouped GEMM for mixture-of-experts layers (glossary "Inference and training
 * in FP4": MXFP4 expert weights).
 *   A: A_rows x K quantised token rows.  row_idx[total_rows] (device int32):
 *   output row r reads token row row_idx[r] of A.  group_off[E+1] (device int32,
 *   non-decreasing, group_off[0] = 0, group_off[E] = total_rows): rows
 *   group_off[e] .. group_off[e+1]-1 belong to expert e.  B: E expert matrices,
 *   each N x K quantised, codes N*K/2 bytes apart and scales
 *   fp4_scale_bytes(fmt, N, K) bytes apart.  C: total_rows x N, row r =
 *   (A[row_idx[r]] . B_e^T) * tsA * tsB for its expert e.
 *   Group sizes stay on the device; the kernel builds its own tile list: a
 *   group's last tile is only as high as its rows need (32 to 256 rows, the
 *   rest of the workgroup idles), and tiles of at most 128 rows run after
 *   the others.  Every row_idx entry must lie in [0, A_rows).
 * Formats: FP4_MXFP4, FP4_MXFP4_OCP and FP4_NVFP4.  NVFP4: tsA is the token
 *   matrix's tensor scale (one device FP32) and tsB holds E device FP32
 *   values, expert e's tensor scale at tsB[e] (each expert quantised on its
 *   own); both required (FP4_ERR_NULL).  MXFP4: both ignored, may be NULL.
 * Requirements as fp4_gemm, and A's codes (A_rows * K/2 bytes) below 4 GiB.
 * workspace (optional, MXFP4 formats): NULL, or at least
 *   fp4_workspace_size(FP4_OP_GEMM_GROUPED, fmt, total_rows, N, K, E) bytes,
 *   16-byte aligned (else FP4_ERR_WORKSPACE / FP4_ERR_ALIGN), with the
 *   gathered codes (total_rows * K/2 bytes) below 4 GiB.  With it, the call
 *   first copies row_idx's token rows (codes and scales) into expert order
 *   there and the GEMM reads them as contiguous rows; the result has the same
 *   bits.  Ignored for NVFP4.  Calls sharing one workspace must be ordered. */
int fp4_gemm_grouped(const uint8_t* A, const uint8_t* sA, int64_t A_rows, const int32_t* row_idx,
                     const int32_t* group_off, int32_t E, const uint8_t* B, const uint8_t* sB,
                     const float* tsA, const float* tsB, void* C, int64_t total_rows, int64_t N, int64_t K,
                     int fmt, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Decode-shape NVFP4 GEMM with the activation quantised inside the call (one
 * kernel): C[M x N] = (X^ . W^T) * s_x * tsW, where X^, s_x are what
 * fp4_quantize(X, FP4_NVFP4, ...) would produce -- the tensor scale from X's
 * largest magnitude (s_x = amax / 2688, 1 for an all-zero X, at least FLT_MIN)
 * unless flags has FP4_TS_GIVEN, 16-value blocks with E4M3 scales, E2M1 codes
 * -- and W^ the NVFP4 weights (codes, scales, tensor scale tsW).  Same
 * arithmetic as fp4_quantize followed by fp4_gemm ("Rubin FP4 GEMM deep dive"
 * §1.2, §6.2: decoding moves every weight once per token, so the activation
 * work is folded into the weight stream); the quantised X is not stored.
 *   X: M x K, FP32 or BF16 (x_dtype), K contiguous, 16-byte aligned.
 *   x_tensor_scale: with FP4_TS_GIVEN, the given s_x (device FP32, required);
 *   otherwise, if non-NULL, receives the computed s_x.
 *   W, sW, tsW: as B, sB, tsB of fp4_gemm.  C: M x N, FP32 or BF16.
 * Applies to small activations (each workgroup stages all of X: for example
 * M <= 8 with K = 8192); fp4_gemm_nvfp4_act_supported says whether a shape
 * is; otherwise FP4_ERR_SHAPE (use fp4_quantize + fp4_gemm).  The result has
 * the same bits as fp4_quantize + fp4_gemm (both take the same decode kernel).
 * Each workgroup re-reads and re-quantises all of X, so beyond M = 2 the two
 * calls are faster (measured at 8192 x 8192). 
 * Requirements: K % 32 == 0.  M == 0 or N == 0 is a no-op. */
int fp4_gemm_nvfp4_act(const void* X, int x_dtype, float* x_tensor_scale, unsigned flags, const uint8_t* W,
                       const uint8_t* sW, const float* tsW, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                       void* stream);

/* 1 if fp4_gemm_nvfp4_act takes this shape and X dtype, else 0.  Host-only. */
int fp4_gemm_nvfp4_act_supported(int64_t M, int64_t N, int64_t K, int x_dtype);

/* Dense GEMM with the whole epilogue in the same kernel ("Rubin FP4 GEMM deep
 * dive" §3.2: scale the FP32 result, add bias, apply the activation, convert
 * to FP4 if wanted; §4.2: C = (A.B) * (sA * sB) + bias, fused so that C makes
 * one trip to memory).  Per element, each step one FP32 rounding:
 *   v = acc * tsA * tsB;  v = v + bias[n] (bias != NULL);
 *   v = v > 0 ? v : +0 (act == FP4_ACT_RELU; -0 becomes +0).
 * Output (out):
 *   FP4_OUT_F32 / FP4_OUT_BF16: C is M x N of that type, as fp4_gemm.
 *   FP4_OUT_MXFP4 / FP4_OUT_MXFP4_OCP: v is quantised along N exactly as
 *     fp4_quantize(v, FP4_MXFP4 / FP4_MXFP4_OCP) quantises an M x N matrix
 *     (rows = M, K = N): codes into C (M x N/2 bytes), scale tiles into C_scales
 *     (fp4_scale_bytes(fmt, M, N) bytes, padding included), so the result feeds
 *     the next fp4_gemm as its A operand.  Requires N % 32 == 0 and C 16-byte
 *     aligned.
 *   FP4_OUT_NVFP4: likewise, quantised exactly as fp4_quantize(v, FP4_NVFP4)
 *     with the given tensor scale *C_tensor_scale (flag FP4_TS_GIVEN; NVFP4
 *     video transcript: 16-value blocks, E4M3 block scales, one FP32 tensor
 *     scale).  The scale is the caller's because the one fp4_quantize would
 *     compute needs the maximum of all of C, i.e. a second pass over it.
 *     The result feeds the next fp4_gemm with that tensor scale.
 *   A, sA, B, sB, tsA, tsB, fmt (FP4_MXFP4, FP4_MXFP4_OCP or FP4_NVFP4), K: as
 *   fp4_gemm (always the tiled kernel, any M).  bias: N device FP32 values,
 *   16-byte aligned, or NULL.  C_scales: required (4-byte aligned) for FP4
 *   output, ignored otherwise.  C_tensor_scale: one device FP32 (finite,
 *   > 0), 4-byte aligned, required for FP4_OUT_NVFP4 (FP4_ERR_NULL), ignored
 *   otherwise.  No workspace.
 * M == 0 or N == 0 is a no-op; K == 0 gives v = 0 (+ bias, activation). */
int fp4_gemm_ex(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* tsA,
                const float* tsB, const float* bias, int act, void* C, uint8_t* C_scales,
                const float* C_tensor_scale, int64_t M, int64_t N, int64_t K, int fmt, int out, void* stream);

/* Mixed-format GEMM, W4A8 ("Rubin FP4 GEMM deep dive" §3.4: activations
 * kept in FP8 while the weights go to FP4):
 *   C[m,n] = sum_k A[m,k] * B[n,k], accumulated in FP32, then
 *   v = v + bias[n] (bias != NULL) and v = v > 0 ? v : +0 (act ==
 *   FP4_ACT_RELU), each step one FP32 rounding, stored as FP32 or BF16
 *   (out_dtype, round to nearest even).
 *   A: M x K MXFP8 (codes M * K bytes, scales fp4_scale_bytes(FP4_MXFP8, M, K)
 *   bytes), as fp4_quantize(FP4_MXFP8 or FP4_MXFP8_OCP) writes them.
 *   B: N x K MXFP4 (either exponent rule), as for fp4_gemm.
 * The gfx950 block-scaled matrix core multiplies E4M3 by E2M1 directly, both
 * E8M0 scales applied inside the instruction (at the FP8 rate, half the FP4
 * rate).
 * Requirements: K % 32 == 0, K <= 2^23; codes 16-byte aligned; scales 4-byte
 *   aligned; bias 16-byte aligned or NULL; C aligned to its element size.
 *   M, N >= 0 arbitrary.  No workspace.
 * M == 0 or N == 0 is a no-op; K == 0 gives v = 0 (+ bias, activation). */
int fp4_gemm_w4a8(const uint8_t* A, const uint8_t* sA, const uint8_t* B, const uint8_t* sB, const float* bias,
                  int act, void* C, int64_t M, int64_t N, int64_t K, int out_dtype, void* stream);

/* Static string naming a status code. */
const char* fp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H_ */
