"""CPU oracle for FP4 (E2M1) block-scaled quantisation and matrix multiply.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library: the arithmetic lives in ``fp4_oracle.c`` (plain C, FP64 accumulation,
no fast-math, no FP contraction), compiled here with gcc; this module only
marshals numpy arrays through ctypes.

Definitions follow the pages cited in ``fp4_oracle.c``: the E2M1 grid and the
block-max-to-6 rule (Ultralytics glossary "FP4", "How FP4 works"), MXFP4 and
NVFP4 block formats (NVFP4 video transcript, prism.simon-ai.net), E8M0 scales
and the scaled FP32-accumulated GEMM ("Rubin FP4 GEMM deep dive",
yfxerp.com, §3.1, §4.2), and MXFP8 operands beside MXFP4 ones (same page, §3.4:
activations kept in FP8 while weights go to FP4).

Parity pins: every function here is pinned by a non-GPU test in
``tests/test_oracle_pins.py`` / ``tests/test_codecs.py`` (printed worked example,
printed value set, torch library casts, closed forms, invariants, numpy
matmul on tiny shapes).
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FMT_MXFP4, FMT_NVFP4, FMT_MXFP4_OCP, FMT_MXFP8, FMT_MXFP8_OCP = 0, 1, 2, 3, 4
DT_F32, DT_BF16 = 0, 1

_lib = None


# ORACLE_SANITIZE=1 loads a copy built with AddressSanitizer and
# UndefinedBehaviorSanitizer (clang, no OpenMP) instead; the process must
# preload clang's ASan runtime (tests/test_sanitizers.py does).
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
CLANG = "/opt/rocm/llvm/bin/clang"


def build_sanitized(force=False):
    if force or not os.path.exists(LIB_SAN) or os.path.getmtime(LIB_SAN) < os.path.getmtime(SRC):
        tmp = LIB_SAN + ".tmp%d" % os.getpid()
        subprocess.check_call(
            [CLANG, "-O1", "-g", "-fno-fast-math", "-ffp-contract=off", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared-libsan", "-fPIC", "-shared",
             "-Wall", "-Wno-unknown-pragmas", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB_SAN)
    return LIB_SAN


def build(force=False):
    """Compile fp4_oracle.c with gcc into liboracle.so next to it."""
    if SANITIZE:
        return build_sanitized(force)
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
             "-shared", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB_SAN if SANITIZE else LIB)
        P, I64, I32, D, F = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                             ctypes.c_double, ctypes.c_float)
        sig = {
            "oracle_e2m1_value": (D, [I32]),
            "oracle_e2m1_encode_mag": (I32, [F]),
            "oracle_e8m0_value": (D, [I32]),
            "oracle_mx_exponent": (I32, [F]),
            "oracle_mx_exponent_ocp": (I32, [F]),
            "oracle_mx8_exponent": (I32, [F]),
            "oracle_mx8_exponent_ocp": (I32, [F]),
            "oracle_e4m3_value": (D, [I32]),
            "oracle_e4m3_encode": (I32, [F]),
            "oracle_f32_to_bf16": (ctypes.c_uint16, [F]),
            "oracle_bf16_to_f32": (F, [ctypes.c_uint16]),
            "oracle_scale_bytes": (I64, [I32, I64, I64]),
            "oracle_scale_offset": (I64, [I32, I64, I64, I64, I64]),
            "oracle_nvfp4_tensor_scale": (F, [F]),
            "oracle_tensor_amax": (F, [P, I32, I64]),
            "oracle_quantize": (I32, [P, I32, I32, I64, I64, P, P, P, P, I32]),
            "oracle_quantize_sr": (I32, [P, I32, I32, I64, I64, P, P, P, P, I32, ctypes.c_uint64]),
            "oracle_philox4x64_10": (None, [P, P, P]),
            "oracle_quantize_ex": (I32, [P, I32, I32, I64, I64, P, P, P, P, I32, I32, ctypes.c_uint64, I32]),
            "oracle_rht16": (None, [P, I32, I64, I64, ctypes.c_uint64, P]),
            "oracle_sr_word": (ctypes.c_uint32, [ctypes.c_uint64, ctypes.c_uint64]),
            "oracle_e2m1_sr_mag": (I32, [F, ctypes.c_uint32]),
            "oracle_dequantize": (None, [P, P, P, I32, P, I32, I64, I64]),
            "oracle_gemm": (None, [P, P, P, P, D, D, I64, I64, I64, I32, P, P]),
            "oracle_gemm_mixed": (None, [P, P, I32, P, P, I32, D, D, I64, I64, I64, P, P]),
            "oracle_gemm_mixed_sampled": (None, [P, P, I32, P, P, I32, D, D, I64, I64, I64, P, P, I64, P, P]),
            "oracle_epilogue": (None, [P, P, I32, I64, I64, P]),
            "oracle_gemm_sampled": (None, [P, P, P, P, D, D, I64, I64, I64, I32, P, P, I64, P, P]),
            "oracle_gemm_grouped_sampled": (None, [P, P, I64, P, P, I32, P, P, D, D, I64, I64, I32,
                                                   P, P, I64, P, P]),
            "oracle_block_mae": (D, [P, I64, I64, I32]),
            "oracle_e2m1_encode_mag_batch": (None, [P, I64, P]),
            "oracle_e4m3_encode_batch": (None, [P, I64, P]),
            "oracle_mx_exponent_batch": (None, [P, I64, I32, P]),
            "oracle_f32_to_bf16_batch": (None, [P, I64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def block_size(fmt):
    return 16 if fmt == FMT_NVFP4 else 32


def is_fp8(fmt):
    """MXFP8 formats store one E4M3 byte per element (FP4: two per byte)."""
    return fmt in (FMT_MXFP8, FMT_MXFP8_OCP)


def code_bytes(fmt, rows, K):
    return rows * K if is_fp8(fmt) else rows * K // 2


# ---- scalar codecs -------------------------------------------------------
def e2m1_value(code):
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(byte):
    return lib().oracle_e4m3_value(int(byte))


def e8m0_value(byte):
    return lib().oracle_e8m0_value(int(byte))


def e2m1_encode_mag(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().oracle_e2m1_encode_mag_batch(_p(y), y.size, _p(out))
    return out


def e4m3_encode(r):
    r = np.ascontiguousarray(r, dtype=np.float32)
    out = np.empty(r.shape, np.uint8)
    lib().oracle_e4m3_encode_batch(_p(r), r.size, _p(out))
    return out


def mx_exponent(amax, ocp=False):
    a = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(a.shape, np.int32)
    lib().oracle_mx_exponent_batch(_p(a), a.size, int(ocp), _p(out))
    return out


def mx8_exponent(amax, ocp=False):
    """MXFP8 block exponent of each amax (scalar loop over the C function)."""
    a = np.ascontiguousarray(amax, dtype=np.float32).ravel()
    fn = lib().oracle_mx8_exponent_ocp if ocp else lib().oracle_mx8_exponent
    return np.array([fn(float(v)) for v in a], np.int32).reshape(np.shape(amax))


def f32_to_bf16_bits(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().oracle_f32_to_bf16_batch(_p(f), f.size, _p(out))
    return out


def nvfp4_tensor_scale(amax_t):
    return lib().oracle_nvfp4_tensor_scale(float(amax_t))


def scale_bytes(fmt, rows, K):
    return lib().oracle_scale_bytes(fmt, rows, K)


def scale_offset(fmt, rows, K, r, b):
    return lib().oracle_scale_offset(fmt, rows, K, r, b)


# ---- quantise / dequantise -------------------------------------------------
def quantize(x, fmt, tensor_scale=None, sr_seed=None, two_d=False):
    """x: (rows, K) float32, or uint16 holding BF16 bit patterns.

    Returns (codes[rows, K//2] u8 (MXFP8: [rows, K]), scales[tiled] u8,
    scales_canon[rows, K//bs] u8, tensor_scale float) -- tensor_scale is 1.0 for
    the MX formats.  sr_seed: round the
    elements stochastically with that seed (scales unchanged).  two_d: NVFP4
    block scales shared by 16 x 16 patches."""
    x = np.ascontiguousarray(x)
    dt = DT_BF16 if x.dtype == np.uint16 else DT_F32
    if dt == DT_F32:
        x = x.astype(np.float32, copy=False)
    rows, K = x.shape
    bs = block_size(fmt)
    codes = np.zeros((rows, K if is_fp8(fmt) else K // 2), np.uint8)
    scales = np.zeros(scale_bytes(fmt, rows, K), np.uint8)
    canon = np.zeros((rows, K // bs), np.uint8)
    ts = np.array([1.0 if tensor_scale is None else tensor_scale], np.float32)
    if sr_seed is None and not two_d:
        rc = lib().oracle_quantize(_p(x), dt, fmt, rows, K, _p(codes), _p(scales), _p(canon), _p(ts),
                                   int(tensor_scale is not None))
    else:
        rc = lib().oracle_quantize_ex(_p(x), dt, fmt, rows, K, _p(codes), _p(scales), _p(canon), _p(ts),
                                      int(tensor_scale is not None), int(sr_seed is not None),
                                      0 if sr_seed is None else int(sr_seed) & 0xFFFFFFFFFFFFFFFF, int(bool(two_d)))
    if rc != 0:
        raise ValueError("oracle_quantize: unsupported shape")
    return codes, scales, canon, float(ts[0])


def philox4x64_10(counter, key):
    """Philox4x64-10 block: counter (4 uint64), key (2 uint64) -> 4 uint64."""
    c = np.array([np.uint64(int(v) & 0xFFFFFFFFFFFFFFFF) for v in counter], dtype=np.uint64)
    k = np.array([np.uint64(int(v) & 0xFFFFFFFFFFFFFFFF) for v in key], dtype=np.uint64)
    out = np.zeros(4, np.uint64)
    lib().oracle_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def rht16(x, seed):
    """Random Hadamard transform on 16-value blocks along K (float32 out)."""
    x = np.ascontiguousarray(x)
    dt = DT_BF16 if x.dtype == np.uint16 else DT_F32
    if dt == DT_F32:
        x = x.astype(np.float32, copy=False)
    rows, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    y = np.empty((rows, K), np.float32)
    lib().oracle_rht16(_p(x), dt, rows, K, int(seed) & 0xFFFFFFFFFFFFFFFF, _p(y))
    return y


def sr_word(seed, i):
    return int(lib().oracle_sr_word(int(seed) & 0xFFFFFFFFFFFFFFFF, int(i)))


def e2m1_sr_mag(y, r):
    return int(lib().oracle_e2m1_sr_mag(float(y), int(r) & 0xFFFFFFFF))


def dequantize(codes, scales, tensor_scale, fmt, rows, K, out_bf16=False):
    ts = np.array([tensor_scale], np.float32)
    if out_bf16:
        out = np.empty((rows, K), np.uint16)
    else:
        out = np.empty((rows, K), np.float32)
    lib().oracle_dequantize(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)), _p(ts),
                            fmt, _p(out), DT_BF16 if out_bf16 else DT_F32, rows, K)
    return out


def tensor_amax(x):
    x = np.ascontiguousarray(x)
    dt = DT_BF16 if x.dtype == np.uint16 else DT_F32
    return lib().oracle_tensor_amax(_p(x), dt, x.size)


# ---- matrix products -------------------------------------------------------
def gemm(A, sA, B, sB, M, N, K, fmt, tsA=1.0, tsB=1.0):
    """Returns (Cref, T) float64 (M, N): FP64 product of dequantised operands
    times tsA*tsB, and the magnitude bound sum|a*b|*|tsA*tsB|."""
    C = np.empty((M, N), np.float64)
    T = np.empty((M, N), np.float64)
    lib().oracle_gemm(_p(A), _p(sA), _p(B), _p(sB), float(tsA), float(tsB), M, N, K, fmt, _p(C), _p(T))
    return C, T


ACT_NONE, ACT_RELU = 0, 1


def epilogue(C, bias=None, act=ACT_NONE):
    """Epilogue of the scaled product C (float64, M x N): C + bias[n] summed in
    FP64 and rounded once to FP32, then ReLU (v > 0 ? v : +0) if act.  Returns
    float32 (M, N); quantise it with quantize(...) for an FP4 output."""
    C = np.ascontiguousarray(C, np.float64)
    M, N = C.shape
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    if b is not None and b.shape != (N,):
        raise ValueError("bias must have N entries")
    out = np.empty((M, N), np.float32)
    lib().oracle_epilogue(_p(C), _p(b), int(act), M, N, _p(out))
    return out


def gemm_mixed(A, sA, fmtA, B, sB, fmtB, M, N, K, tsA=1.0, tsB=1.0):
    """As gemm, with A in format fmtA and B in fmtB (e.g. MXFP8 x MXFP4)."""
    C = np.empty((M, N), np.float64)
    T = np.empty((M, N), np.float64)
    lib().oracle_gemm_mixed(_p(np.ascontiguousarray(A)), _p(np.ascontiguousarray(sA)), fmtA,
                            _p(np.ascontiguousarray(B)), _p(np.ascontiguousarray(sB)), fmtB,
                            float(tsA), float(tsB), M, N, K, _p(C), _p(T))
    return C, T


def gemm_mixed_sampled(A, sA, fmtA, B, sB, fmtB, M, N, K, rows, cols, tsA=1.0, tsB=1.0):
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    C = np.empty(rows.size, np.float64)
    T = np.empty(rows.size, np.float64)
    lib().oracle_gemm_mixed_sampled(_p(np.ascontiguousarray(A)), _p(np.ascontiguousarray(sA)), fmtA,
                                    _p(np.ascontiguousarray(B)), _p(np.ascontiguousarray(sB)), fmtB,
                                    float(tsA), float(tsB), M, N, K, _p(rows), _p(cols), rows.size, _p(C), _p(T))
    return C, T


def gemm_sampled(A, sA, B, sB, M, N, K, fmt, rows, cols, tsA=1.0, tsB=1.0):
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    C = np.empty(rows.size, np.float64)
    T = np.empty(rows.size, np.float64)
    lib().oracle_gemm_sampled(_p(A), _p(sA), _p(B), _p(sB), float(tsA), float(tsB), M, N, K, fmt,
                              _p(rows), _p(cols), rows.size, _p(C), _p(T))
    return C, T


def gemm_grouped_sampled(A, sA, T_rows, row_idx, group_off, B, sB, N, K, fmt, out_rows, cols,
                         tsA=1.0, tsB=1.0):
    row_idx = np.ascontiguousarray(row_idx, np.int32)
    group_off = np.ascontiguousarray(group_off, np.int32)
    out_rows = np.ascontiguousarray(out_rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    E = group_off.size - 1
    C = np.empty(out_rows.size, np.float64)
    T = np.empty(out_rows.size, np.float64)
    lib().oracle_gemm_grouped_sampled(_p(A), _p(sA), T_rows, _p(row_idx), _p(group_off), E, _p(B), _p(sB),
                                      float(tsA), float(tsB), N, K, fmt, _p(out_rows), _p(cols),
                                      out_rows.size, _p(C), _p(T))
    return C, T


MAE_PAGE, MAE_MXFP4, MAE_MXFP4_OCP, MAE_NVFP4 = 0, 1, 2, 3


def block_mae(x, block, mode):
    x = np.ascontiguousarray(x, np.float32)
    return lib().oracle_block_mae(_p(x), x.size, int(block), int(mode))


# ---- acceptance test for matrix-product outputs ----------------------------
REL_TOL = 1e-5  # per element, times sum|a*b| (FP32 accumulation order)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def gemm_within_tolerance(C, Cref, T, out_bf16=False, rel=REL_TOL):
    """Element-wise acceptance mask.

    FP32 output:  |C - Cref| <= rel * T.
    BF16 output:  C (bits) lies in [bf16(Cref - rel*T), bf16(Cref + rel*T)],
                  i.e. the correctly rounded ends of the FP32 acceptance interval.
    T == 0 requires C == 0."""
    Cref = np.asarray(Cref, np.float64)
    T = np.asarray(T, np.float64)
    if out_bf16:
        c = bf16_bits_to_f32(C).astype(np.float64)
        lo = bf16_bits_to_f32(f32_to_bf16_bits((Cref - rel * T).astype(np.float32))).astype(np.float64)
        hi = bf16_bits_to_f32(f32_to_bf16_bits((Cref + rel * T).astype(np.float32))).astype(np.float64)
        ok = (c >= lo) & (c <= hi)
    else:
        c = np.asarray(C, np.float64)
        ok = np.abs(c - Cref) <= rel * T
    return ok | ((T == 0) & (c == 0))
