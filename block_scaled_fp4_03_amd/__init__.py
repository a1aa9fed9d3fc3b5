"""Python binding of libfp4 -- FP4 (E2M1) block-scaled quantisation and GEMM
for AMD Instinct MI355X (gfx950).

The C ABI (include/fp4.h) is exposed under the same names (``fp4_quantize``,
``fp4_dequantize``, ``fp4_gemm``, ``fp4_gemm_ex``, ``fp4_gemm_grouped``, ``fp4_gemm_w4a8``, ``fp4_scale_bytes``,
``fp4_workspace_size``, ``fp4_status_string``), taking raw device pointers as
integers.  The tensor helpers below only allocate outputs with torch and
marshal ``data_ptr()`` / the current stream into those calls: every step of the
computation runs in the HIP kernels of libfp4.so.  There is no fallback -- if
the library is not built, or no GPU is present, the calls fail loudly.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# FP4_LIB_PATH selects another build of the same library (the tests use it
# for the host-sanitized build); the default is the in-tree libfp4.so.
LIB_PATH = os.environ.get("FP4_LIB_PATH") or os.path.join(HERE, "libfp4.so")

# enum fp4_fmt / fp4_dtype / fp4_op, flags
MXFP4, NVFP4, MXFP4_OCP, MXFP8, MXFP8_OCP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
OP_QUANTIZE, OP_GEMM, OP_GEMM_GROUPED = 0, 1, 2
TS_GIVEN = 1
Q_SR, Q_2D = 2, 4
# enum fp4_out / fp4_act (fp4_gemm_ex)
OUT_F32, OUT_BF16, OUT_MXFP4, OUT_MXFP4_OCP, OUT_NVFP4 = 0, 1, 2, 3, 4
ACT_NONE, ACT_RELU = 0, 1

FUNCTIONS = ("fp4_scale_bytes", "fp4_workspace_size", "fp4_quantize", "fp4_quantize_noalloc", "fp4_quantize_sr",
             "fp4_quantize_ex",
             "fp4_hadamard16", "fp4_dequantize", "fp4_gemm", "fp4_gemm_ex",
             "fp4_gemm_grouped", "fp4_gemm_nvfp4_act", "fp4_gemm_nvfp4_act_supported", "fp4_gemm_w4a8",
             "fp4_status_string", "fp4_set_debug")


class Fp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, fp4_status_string(status), status))


_lib = None


def lib():
    """Load libfp4.so (built in-tree by block_scaled_fp4_03_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4.so is not built (run python -m block_scaled_fp4_03_amd.build)")
        # torch first: its HIP runtime then satisfies the library's
        # libamdhip64.so.7, so both share one runtime (streams, allocations).
        # Loaded the other way round, torch loads a second copy of the
        # runtime under another name, and the library's own HIP calls do not
        # see torch's device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        sig = {
            "fp4_scale_bytes": (I64, [I32, I64, I64]),
            "fp4_workspace_size": (SZ, [I32, I32, I64, I64, I64, I32]),
            "fp4_quantize": (I32, [P, I32, P, P, P, I64, I64, I32, U32, P, SZ, P]),
            "fp4_quantize_noalloc": (I32, [P, I32, P, P, P, I64, I64, I32, U32, P]),
            "fp4_quantize_sr": (I32, [P, I32, P, P, P, I64, I64, I32, U32, ctypes.c_uint64, P, SZ, P]),
            "fp4_quantize_ex": (I32, [P, I32, P, P, P, I64, I64, I32, U32, ctypes.c_uint64, P, SZ, P]),
            "fp4_hadamard16": (I32, [P, I32, P, I32, I64, I64, ctypes.c_uint64, P]),
            "fp4_dequantize": (I32, [P, P, P, I32, P, I32, I64, I64, P]),
            "fp4_gemm": (I32, [P, P, P, P, P, P, P, I64, I64, I64, I32, I32, P, SZ, P]),
            "fp4_gemm_ex": (I32, [P, P, P, P, P, P, P, I32, P, P, P, I64, I64, I64, I32, I32, P]),
            "fp4_gemm_grouped": (I32, [P, P, I64, P, P, I32, P, P, P, P, P, I64, I64, I64, I32, I32, P, SZ, P]),
            "fp4_gemm_nvfp4_act": (I32, [P, I32, P, U32, P, P, P, P, I64, I64, I64, I32, P]),
            "fp4_gemm_nvfp4_act_supported": (I32, [I64, I64, I64, I32]),
            "fp4_gemm_w4a8": (I32, [P, P, P, P, P, I32, P, I64, I64, I64, I32, P]),
            "fp4_status_string": (ctypes.c_char_p, [I32]),
            "fp4_set_debug": (I32, [I32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ---- raw C-ABI calls (integers for pointers) --------------------------------
def fp4_set_debug(on):
    """Debug mode on (1) or off (0); returns the previous setting."""
    return lib().fp4_set_debug(1 if on else 0)


def fp4_status_string(status):
    return lib().fp4_status_string(int(status)).decode()


def fp4_scale_bytes(fmt, rows, K):
    return lib().fp4_scale_bytes(fmt, rows, K)


def fp4_workspace_size(op, fmt, M, N, K, E=0):
    return lib().fp4_workspace_size(op, fmt, M, N, K, E)


def fp4_quantize(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, workspace, workspace_bytes,
                 stream):
    return lib().fp4_quantize(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, workspace,
                              workspace_bytes, stream)


def fp4_quantize_noalloc(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, stream):
    return lib().fp4_quantize_noalloc(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, stream)


def fp4_quantize_sr(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, seed, workspace,
                    workspace_bytes, stream):
    return lib().fp4_quantize_sr(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags,
                                 int(seed) & 0xFFFFFFFFFFFFFFFF, workspace, workspace_bytes, stream)


def fp4_quantize_ex(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags, seed, workspace,
                    workspace_bytes, stream):
    return lib().fp4_quantize_ex(x, fmt, codes, block_scales, tensor_scale, rows, K, in_dtype, flags,
                                 int(seed) & 0xFFFFFFFFFFFFFFFF, workspace, workspace_bytes, stream)


def fp4_hadamard16(x, in_dtype, y, out_dtype, rows, K, seed, stream):
    return lib().fp4_hadamard16(x, in_dtype, y, out_dtype, rows, K, int(seed) & 0xFFFFFFFFFFFFFFFF, stream)


def fp4_dequantize(codes, block_scales, tensor_scale, fmt, out, out_dtype, rows, K, stream):
    return lib().fp4_dequantize(codes, block_scales, tensor_scale, fmt, out, out_dtype, rows, K, stream)


def fp4_gemm(A, sA, B, sB, tsA, tsB, C, M, N, K, fmt, out_dtype, workspace, workspace_bytes, stream):
    return lib().fp4_gemm(A, sA, B, sB, tsA, tsB, C, M, N, K, fmt, out_dtype, workspace, workspace_bytes, stream)


def fp4_gemm_ex(A, sA, B, sB, tsA, tsB, bias, act, C, C_scales, C_tensor_scale, M, N, K, fmt, out, stream):
    return lib().fp4_gemm_ex(A, sA, B, sB, tsA, tsB, bias, act, C, C_scales, C_tensor_scale, M, N, K, fmt, out,
                             stream)


def fp4_gemm_grouped(A, sA, A_rows, row_idx, group_off, E, B, sB, tsA, tsB, C, total_rows, N, K, fmt, out_dtype,
                     workspace, workspace_bytes, stream):
    return lib().fp4_gemm_grouped(A, sA, A_rows, row_idx, group_off, E, B, sB, tsA, tsB, C, total_rows, N, K, fmt,
                                  out_dtype, workspace, workspace_bytes, stream)


def fp4_gemm_nvfp4_act(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K, out_dtype, stream):
    return lib().fp4_gemm_nvfp4_act(X, x_dtype, x_tensor_scale, flags, W, sW, tsW, C, M, N, K, out_dtype, stream)


def fp4_gemm_nvfp4_act_supported(M, N, K, x_dtype):
    return lib().fp4_gemm_nvfp4_act_supported(M, N, K, x_dtype)


def fp4_gemm_w4a8(A, sA, B, sB, bias, act, C, M, N, K, out_dtype, stream):
    return lib().fp4_gemm_w4a8(A, sA, B, sB, bias, act, C, M, N, K, out_dtype, stream)


# ---- torch helpers: allocation + pointer/stream marshalling only -------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(rc, where):
    if rc != 0:
        raise Fp4Error(rc, where)


def _need(t, name, dtypes=None, numel=None, device=None, ndim=None):
    """Reject, before any library call, an argument the C ABI would misread:
    not a tensor, not on a GPU, not contiguous (the kernels take a raw
    pointer and assume the documented dense layout), of another dtype (an
    int64 index read as int32 halves), too small, or on another device than
    the call's first operand.  Returns t."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, %d needed" % (name, t.numel(), numel))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor, got device %s" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, the call's operands on %s" % (name, t.device, device))
    return t


def _need_q(q, name, device=None):
    """Check a Quantized operand: codes, scales (and the NVFP4 tensor scale)
    contiguous uint8 / float32 GPU tensors of the sizes its format needs."""
    if not isinstance(q, Quantized):
        raise TypeError("%s must be a Quantized, got %s" % (name, type(q).__name__))
    torch = _torch()
    if q.fmt == NVFP4 and q.tensor_scale is None:
        raise ValueError("%s: an NVFP4 operand needs its tensor scale" % name)
    ncodes = q.rows * (q.K if is_fp8(q.fmt) else q.K // 2)
    _need(q.codes, name + ".codes", (torch.uint8,), ncodes, device)
    nbytes = fp4_scale_bytes(q.fmt, q.rows, q.K)
    if nbytes < 0:
        raise Fp4Error(int(nbytes), "fp4_scale_bytes")
    _need(q.scales, name + ".scales", (torch.uint8,), nbytes, device)
    if q.tensor_scale is not None:
        _need(q.tensor_scale, name + ".tensor_scale", (torch.float32,), 1, device)
    return q


def _need_out(t, name, shape, dtypes, device):
    _need(t, name, dtypes, None, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def workspace(op, fmt, M, N, K, E=0, device="cuda"):
    """A zero-filled workspace tensor of the size the operation needs (or None)."""
    torch = _torch()
    n = fp4_workspace_size(op, fmt, M, N, K, E)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def is_fp8(fmt):
    """MXFP8 formats hold one E4M3 byte per element (the FP4 ones two codes per byte)."""
    return fmt in (MXFP8, MXFP8_OCP)


class Quantized:
    """codes (rows x K/2 uint8; MXFP8 rows x K), scales (tiled uint8), tensor_scale (1 float32 or None)."""

    def __init__(self, codes, scales, tensor_scale, fmt, rows, K):
        self.codes, self.scales, self.tensor_scale = codes, scales, tensor_scale
        self.fmt, self.rows, self.K = fmt, rows, K


def quantize(x, fmt, tensor_scale=None, ws=None, out=None, stream=None, sr_seed=None, two_d=False):
    """Quantise a 2-D float32/bfloat16 CUDA tensor along its last dimension.

    NVFP4: pass `tensor_scale` (a 1-element float32 tensor) to use a given
    scale; otherwise one is computed and returned in the result.  MXFP8 /
    MXFP8_OCP: E4M3 codes, one byte per element.  sr_seed:
    round the elements stochastically with that seed (fp4_quantize_sr).
    two_d: NVFP4 scales per 16 x 16 patch (fp4_quantize_ex, FP4_Q_2D)."""
    torch = _torch()
    _need(x, "x", (torch.float32, torch.bfloat16), ndim=2)
    rows, K = x.shape
    dev = x.device
    if tensor_scale is not None:
        _need(tensor_scale, "tensor_scale", (torch.float32,), 1, dev)
    if ws is not None:
        _need(ws, "ws", (torch.uint8,), None, dev)
    if out is not None:
        if (out.rows, out.K, out.fmt) != (rows, K, fmt):
            raise ValueError("out is a %d x %d matrix of format %d, x needs %d x %d of format %d"
                             % (out.rows, out.K, out.fmt, rows, K, fmt))
        if fmt == NVFP4 and out.tensor_scale is None:
            raise ValueError("out: an NVFP4 result needs a tensor-scale tensor")
        _need_q(out, "out", dev)
    if out is None:
        codes = torch.empty((rows, K if is_fp8(fmt) else K // 2), dtype=torch.uint8, device=dev)
        nbytes = fp4_scale_bytes(fmt, rows, K)
        if nbytes < 0:
            raise Fp4Error(int(nbytes), "fp4_scale_bytes")
        scales = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ts = None
        if fmt == NVFP4:
            ts = tensor_scale if tensor_scale is not None else torch.empty(1, dtype=torch.float32, device=dev)
        out = Quantized(codes, scales, ts, fmt, rows, K)
    flags = TS_GIVEN if (fmt == NVFP4 and tensor_scale is not None) else 0
    if fmt == NVFP4 and not flags and ws is None:
        ws = workspace(OP_QUANTIZE, fmt, rows, 0, K, device=dev)
    if two_d:
        rc = fp4_quantize_ex(_ptr(x), fmt, _ptr(out.codes), _ptr(out.scales), _ptr(out.tensor_scale), rows, K,
                             _dtype_code(x), flags | Q_2D | (Q_SR if sr_seed is not None else 0),
                             0 if sr_seed is None else sr_seed, _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream))
    elif sr_seed is None:
        rc = fp4_quantize(_ptr(x), fmt, _ptr(out.codes), _ptr(out.scales), _ptr(out.tensor_scale), rows, K,
                          _dtype_code(x), flags, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    else:
        rc = fp4_quantize_sr(_ptr(x), fmt, _ptr(out.codes), _ptr(out.scales), _ptr(out.tensor_scale), rows, K,
                             _dtype_code(x), flags, sr_seed, _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream))
    _check(rc, "fp4_quantize_sr" if sr_seed is not None else "fp4_quantize")
    return out


def hadamard16(x, seed, out_dtype=None, out=None, stream=None):
    """Random Hadamard transform of a 2-D float32/bfloat16 CUDA tensor on
    16-value blocks along its last dimension (fp4_hadamard16)."""
    torch = _torch()
    _need(x, "x", (torch.float32, torch.bfloat16), ndim=2)
    rows, K = x.shape
    if out is None:
        out = torch.empty((rows, K), dtype=x.dtype if out_dtype is None else out_dtype, device=x.device)
    _need_out(out, "out", (rows, K), (torch.float32, torch.bfloat16), x.device)
    rc = fp4_hadamard16(_ptr(x), _dtype_code(x), _ptr(out), _dtype_code(out), rows, K, seed, _stream(stream))
    _check(rc, "fp4_hadamard16")
    return out


def dequantize(q, out_dtype=None, stream=None):
    torch = _torch()
    _need_q(q, "q")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    out = torch.empty((q.rows, q.K), dtype=out_dtype, device=q.codes.device)
    rc = fp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), q.fmt, _ptr(out), _dtype_code(out),
                        q.rows, q.K, _stream(stream))
    _check(rc, "fp4_dequantize")
    return out


def gemm(a, b, out_dtype=None, out=None, ws=None, stream=None):
    """C = A . B^T for quantised A (M x K) and B (N x K) of the same format."""
    torch = _torch()
    dev = _need_q(a, "a").codes.device
    _need_q(b, "b", dev)
    M, N, K = a.rows, b.rows, a.K
    if b.K != K or a.fmt != b.fmt:
        raise ValueError("operands disagree on K or format")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype is None else out_dtype, device=dev)
    _need_out(out, "out", (M, N), (torch.float32, torch.bfloat16), dev)
    if ws is None:
        ws = workspace(OP_GEMM, a.fmt, M, N, K, device=dev)
    else:
        _need(ws, "ws", (torch.uint8,), None, dev)
    rc = fp4_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), _ptr(a.tensor_scale),
                  _ptr(b.tensor_scale), _ptr(out), M, N, K, a.fmt, _dtype_code(out), _ptr(ws),
                  0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "fp4_gemm")
    return out


def gemm_ex(a, b, bias=None, act=ACT_NONE, out=OUT_BF16, C=None, c_tensor_scale=None, stream=None):
    """C = act((A . B^T) * tsA * tsB + bias) in one kernel (see fp4_gemm_ex in
    include/fp4.h).  out: OUT_F32 / OUT_BF16 -> an M x N tensor; OUT_MXFP4 /
    OUT_MXFP4_OCP -> a Quantized M x N MXFP4 matrix (the next GEMM's A);
    OUT_NVFP4 -> a Quantized M x N NVFP4 matrix under c_tensor_scale (a
    1-element float32 CUDA tensor, required).  bias: N float32 CUDA tensor or
    None.  C: optional preallocated output (tensor, or Quantized for FP4
    output)."""
    torch = _torch()
    dev = _need_q(a, "a").codes.device
    _need_q(b, "b", dev)
    M, N, K = a.rows, b.rows, a.K
    if b.K != K or a.fmt != b.fmt:
        raise ValueError("operands disagree on K or format")
    if bias is not None:
        _need(bias, "bias", (torch.float32,), N, dev)
    fp4_out = out in (OUT_MXFP4, OUT_MXFP4_OCP, OUT_NVFP4)
    ofmt = {OUT_MXFP4: MXFP4, OUT_MXFP4_OCP: MXFP4_OCP, OUT_NVFP4: NVFP4}.get(out)
    if out == OUT_NVFP4:
        if c_tensor_scale is None:
            raise ValueError("OUT_NVFP4 needs c_tensor_scale (1-element float32 CUDA tensor)")
        _need(c_tensor_scale, "c_tensor_scale", (torch.float32,), 1, dev)
    if C is None:
        if fp4_out:
            nbytes = fp4_scale_bytes(ofmt, M, N)
            if nbytes < 0:
                raise Fp4Error(int(nbytes), "fp4_scale_bytes")
            C = Quantized(torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
                          torch.empty(nbytes, dtype=torch.uint8, device=dev),
                          c_tensor_scale if out == OUT_NVFP4 else None, ofmt, M, N)
        else:
            C = torch.empty((M, N), dtype=torch.float32 if out == OUT_F32 else torch.bfloat16, device=dev)
    if fp4_out:
        if (C.rows, C.K) != (M, N):
            raise ValueError("C is a %d x %d matrix, the product %d x %d" % (C.rows, C.K, M, N))
        _need(C.codes, "C.codes", (torch.uint8,), M * (N // 2), dev)
        _need(C.scales, "C.scales", (torch.uint8,), max(0, fp4_scale_bytes(ofmt, M, N)), dev)
    else:
        _need_out(C, "C", (M, N), (torch.float32 if out == OUT_F32 else torch.bfloat16,), dev)
    cptr, sptr = (_ptr(C.codes), _ptr(C.scales)) if fp4_out else (_ptr(C), None)
    tsc = _ptr(c_tensor_scale) if out == OUT_NVFP4 else None
    rc = fp4_gemm_ex(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), _ptr(a.tensor_scale),
                     _ptr(b.tensor_scale), _ptr(bias), act, cptr, sptr, tsc, M, N, K, a.fmt, out, _stream(stream))
    _check(rc, "fp4_gemm_ex")
    return C


def gemm_w4a8(a, b, bias=None, act=ACT_NONE, out_dtype=None, out=None, stream=None):
    """C = act(A . B^T + bias) for MXFP8 activations A (M x K) and MXFP4
    weights B (N x K), FP32 accumulation (see fp4_gemm_w4a8 in include/fp4.h)."""
    torch = _torch()
    dev = _need_q(a, "a").codes.device
    _need_q(b, "b", dev)
    M, N, K = a.rows, b.rows, a.K
    if b.K != K or not is_fp8(a.fmt) or b.fmt not in (MXFP4, MXFP4_OCP):
        raise ValueError("A must be MXFP8 and B MXFP4 with the same K")
    if bias is not None:
        _need(bias, "bias", (torch.float32,), N, dev)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype is None else out_dtype, device=dev)
    _need_out(out, "out", (M, N), (torch.float32, torch.bfloat16), dev)
    rc = fp4_gemm_w4a8(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), _ptr(bias), act, _ptr(out),
                       M, N, K, _dtype_code(out), _stream(stream))
    _check(rc, "fp4_gemm_w4a8")
    return out


def gemm_grouped(a, row_idx, group_off, b_codes, b_scales, N, K, fmt, b_tensor_scale=None, out_dtype=None,
                 out=None, ws=None, stream=None, pregather=True):
    """Grouped (mixture-of-experts) GEMM; see fp4_gemm_grouped in include/fp4.h.
    NVFP4: b_tensor_scale holds one float32 per expert.  pregather: pass a
    workspace (ws, or one allocated here) so that the call first copies the
    token rows into expert order; False runs the GEMM on the gathered rows."""
    torch = _torch()
    dev = _need_q(a, "a").codes.device
    if a.K != K or a.fmt != fmt:
        raise ValueError("a is %d x %d of format %d, the call K = %d, format %d" % (a.rows, a.K, a.fmt, K, fmt))
    # int32 indices: torch's default int64 (cumsum, argsort) would be read as
    # pairs of int32 halves.
    _need(row_idx, "row_idx", (torch.int32,), None, dev, ndim=1)
    _need(group_off, "group_off", (torch.int32,), 1, dev, ndim=1)
    E = group_off.numel() - 1
    total = row_idx.numel()
    nscale = fp4_scale_bytes(fmt, N, K)
    if nscale < 0:
        raise Fp4Error(int(nscale), "fp4_scale_bytes")
    _need(b_codes, "b_codes", (torch.uint8,), E * N * (K // 2), dev)
    _need(b_scales, "b_scales", (torch.uint8,), E * nscale, dev)
    if fmt == NVFP4 and (a.tensor_scale is None or b_tensor_scale is None):
        raise ValueError("NVFP4 needs a's tensor scale and b_tensor_scale (one float32 per expert)")
    if b_tensor_scale is not None:
        _need(b_tensor_scale, "b_tensor_scale", (torch.float32,), E if fmt == NVFP4 else 1, dev)
    if out is None:
        out = torch.empty((total, N), dtype=torch.bfloat16 if out_dtype is None else out_dtype, device=dev)
    _need_out(out, "out", (total, N), (torch.float32, torch.bfloat16), dev)
    if not pregather:
        ws = None
    elif ws is None:
        n = fp4_workspace_size(OP_GEMM_GROUPED, fmt, total, N, K, E)
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None   # no control words: not zeroed
    else:
        _need(ws, "ws", (torch.uint8,), None, dev)
    rc = fp4_gemm_grouped(_ptr(a.codes), _ptr(a.scales), a.rows, _ptr(row_idx), _ptr(group_off), E, _ptr(b_codes),
                          _ptr(b_scales), _ptr(a.tensor_scale), _ptr(b_tensor_scale), _ptr(out), total, N, K, fmt,
                          _dtype_code(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "fp4_gemm_grouped")
    return out


def gemm_nvfp4_act(x, w, tensor_scale=None, ts_out=None, out_dtype=None, out=None, stream=None):
    """C = quantise_nvfp4(x) . w^T in one call (see fp4_gemm_nvfp4_act in
    include/fp4.h).  x: M x K float32/bfloat16 CUDA tensor; w: NVFP4 Quantized.
    tensor_scale: given activation tensor scale (1-element float32 tensor), or
    None to compute it; ts_out: optional 1-element tensor receiving it."""
    torch = _torch()
    _need(x, "x", (torch.float32, torch.bfloat16), ndim=2)
    _need_q(w, "w", x.device)
    M, K = x.shape
    N = w.rows
    if w.K != K or w.fmt != NVFP4:
        raise ValueError("weights must be NVFP4 with the same K")
    for t, name in ((tensor_scale, "tensor_scale"), (ts_out, "ts_out")):
        if t is not None:
            _need(t, name, (torch.float32,), 1, x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16 if out_dtype is None else out_dtype, device=x.device)
    _need_out(out, "out", (M, N), (torch.float32, torch.bfloat16), x.device)
    flags = TS_GIVEN if tensor_scale is not None else 0
    ts = tensor_scale if tensor_scale is not None else ts_out
    rc = fp4_gemm_nvfp4_act(_ptr(x), _dtype_code(x), _ptr(ts), flags, _ptr(w.codes), _ptr(w.scales),
                            _ptr(w.tensor_scale), _ptr(out), M, N, K, _dtype_code(out), _stream(stream))
    _check(rc, "fp4_gemm_nvfp4_act")
    return out
