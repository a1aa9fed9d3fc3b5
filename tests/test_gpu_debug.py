"""Debug mode (fp4_set_debug / FP4_DEBUG): every entry point gives the same
bits with the checks on, and refuses before any launch a buffer shorter than
the call needs and malformed grouped indices (FP4_ERR_BOUNDS).

The short buffers come from hipMalloc of fewer bytes than the call needs,
short by less than the page the allocation occupies, so even a check that
let the call through could not make the kernel leave mapped memory."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

BOUNDS = -9


@pytest.fixture
def debug():
    import block_scaled_fp4_03_amd as fp4
    prev = fp4.fp4_set_debug(1)
    yield fp4
    fp4.fp4_set_debug(prev)


def _hip():
    # The HIP runtime torch loaded (the library uses the same one).
    h = ctypes.CDLL("libamdhip64.so.7")
    h.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    h.hipMalloc.restype = ctypes.c_int
    h.hipFree.argtypes = [ctypes.c_void_p]
    h.hipFree.restype = ctypes.c_int
    h.hipMemset.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t]
    h.hipMemset.restype = ctypes.c_int
    return h


class _Bufs:
    """hipMalloc'd buffers of exact sizes, zeroed, freed at the end."""

    def __init__(self):
        self.h = _hip()
        self.ptrs = []

    def __call__(self, n):
        p = ctypes.c_void_p()
        assert self.h.hipMalloc(ctypes.byref(p), n) == 0
        assert self.h.hipMemset(p.value, 0, n) == 0
        self.ptrs.append(p.value)
        return p.value

    def free(self):
        import torch
        torch.cuda.synchronize()
        for p in self.ptrs:
            self.h.hipFree(p)


def _bits(t):
    return np.ascontiguousarray(to_host(t)).view(np.uint8)


def test_debug_mode_same_bits(debug):
    """Quantise (MXFP4, NVFP4 small / grid / two-pass paths), dequantise, the
    tiled GEMM and each decode GEMV, the fused epilogue with FP4 output, the
    grouped GEMM, the fused decode call, W4A8 and the Hadamard transform:
    debug on and off give the same bits."""
    import torch
    fp4 = debug

    def run():
        out = []
        x = to_dev(synth.gaussian(31, (96, 512)))
        for fmt in (fp4.MXFP4, fp4.NVFP4):
            q = fp4.quantize(x, fmt)
            out += [q.codes, q.scales] + ([q.tensor_scale] if fmt == fp4.NVFP4 else [])
            out.append(fp4.dequantize(q, out_dtype=torch.float32))
        for rows in (32, 512):    # NVFP4 one-launch grid path, two-pass path (BF16, K = 8192)
            xb = to_dev(synth.to_bf16_bits(synth.gaussian(32 + rows, (rows, 8192))))
            q = fp4.quantize(xb, fp4.NVFP4)
            out += [q.codes, q.scales, q.tensor_scale]
        # fp4_quantize_noalloc: its workspace is the library's static array.
        codes = torch.empty(512 * 4096, dtype=torch.uint8, device="cuda")
        scales = torch.empty(fp4.fp4_scale_bytes(1, 512, 8192), dtype=torch.uint8, device="cuda")
        ts = torch.empty(1, dtype=torch.float32, device="cuda")
        rc = fp4.fp4_quantize_noalloc(xb.data_ptr(), fp4.NVFP4, codes.data_ptr(), scales.data_ptr(), ts.data_ptr(),
                                      512, 8192, 1, 0, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, fp4.fp4_status_string(rc)
        out += [codes, scales, ts]
        a = fp4.quantize(to_dev(synth.gaussian(33, (300, 512))), fp4.MXFP4)
        b = fp4.quantize(to_dev(synth.gaussian(34, (256, 512))), fp4.MXFP4)
        out.append(fp4.gemm(a, b, out_dtype=torch.float32))
        C = fp4.gemm_ex(a, b, bias=torch.linspace(-1, 1, 256, device="cuda"), act=fp4.ACT_RELU, out=fp4.OUT_MXFP4)
        out += [C.codes, C.scales]
        w = fp4.quantize(to_dev(synth.gaussian(35, (512, 1024), std=0.02)), fp4.NVFP4)
        for M in (1, 8, 32):
            xa = fp4.quantize(to_dev(synth.gaussian(36 + M, (M, 1024))), fp4.NVFP4)
            out.append(fp4.gemm(xa, w, out_dtype=torch.bfloat16))
            out.append(fp4.gemm_nvfp4_act(to_dev(synth.to_bf16_bits(synth.gaussian(40 + M, (M, 1024)))), w))
        counts = np.array([40, 0, 300, 1])
        row_idx, off = synth.moe_routing(counts, tokens=300, seed=7)
        t = fp4.quantize(to_dev(synth.gaussian(41, (300, 512))), fp4.MXFP4)
        E, N, K = 4, 96, 512
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((E, fp4.fp4_scale_bytes(0, N, K)), dtype=torch.uint8, device="cuda")
        for e in range(E):
            fp4.quantize(to_dev(synth.gaussian(50 + e, (N, K), std=0.02)), 0,
                         out=fp4.Quantized(codes[e], scales[e], None, 0, N, K))
        out.append(fp4.gemm_grouped(t, torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda(), codes, scales,
                                    N, K, 0, out_dtype=torch.bfloat16))
        a8 = fp4.quantize(to_dev(synth.gaussian(42, (64, 512))), fp4.MXFP8)
        out.append(fp4.gemm_w4a8(a8, b, out_dtype=torch.float32))
        out.append(fp4.hadamard16(to_dev(synth.gaussian(43, (64, 512))), 9))
        torch.cuda.synchronize()
        return [_bits(o) for o in out]

    say("debug mode on: every entry point")
    on = run()
    fp4.fp4_set_debug(0)
    say("debug mode off: every entry point")
    off = run()
    assert len(on) == len(off)
    for i, (p, q) in enumerate(zip(on, off)):
        assert np.array_equal(p, q), "output %d differs with debug mode on" % i


def test_debug_mode_refuses_short_buffers(debug):
    """An output or input buffer a little shorter than the call needs:
    FP4_ERR_BOUNDS before any launch; exact sizes pass."""
    import torch
    fp4 = debug
    bufs = _Bufs()
    s = torch.cuda.current_stream().cuda_stream
    try:
        rows, K = 4, 64                       # MXFP4: x 1024 B, codes 128 B, scales 256 B
        nsc = fp4.fp4_scale_bytes(0, rows, K)
        x, codes, sc = bufs(rows * K * 4), bufs(rows * K // 2), bufs(nsc)
        say("debug: quantise into exact buffers")
        assert fp4.fp4_quantize(x, 0, codes, sc, None, rows, K, 0, 0, None, 0, s) == 0
        say("debug: quantise into short buffers")
        assert fp4.fp4_quantize(x, 0, bufs(rows * K // 2 - 16), sc, None, rows, K, 0, 0, None, 0, s) == BOUNDS
        assert fp4.fp4_quantize(x, 0, codes, bufs(nsc - 4), None, rows, K, 0, 0, None, 0, s) == BOUNDS
        assert fp4.fp4_quantize(bufs(rows * K * 4 - 16), 0, codes, sc, None, rows, K, 0, 0, None, 0, s) == BOUNDS
        # NVFP4: the tensor scale and the workspace.
        nsn = fp4.fp4_scale_bytes(1, rows, K)
        scn, ts, ws = bufs(nsn), bufs(4), bufs(16)
        assert fp4.fp4_quantize(x, 1, codes, scn, ts, rows, K, 0, 0, ws, 16, s) == 0
        assert fp4.fp4_quantize(x, 1, codes, scn, bufs(2), rows, K, 0, 0, ws, 16, s) == BOUNDS
        assert fp4.fp4_quantize(x, 1, codes, scn, ts, rows, K, 0, 0, bufs(8), 16, s) == BOUNDS
        # GEMM: C 4 x 4 FP32 = 64 B.
        say("debug: gemm into exact and short C")
        assert fp4.fp4_gemm(codes, sc, codes, sc, None, None, bufs(64), 4, 4, K, 0, 0, None, 0, s) == 0
        assert fp4.fp4_gemm(codes, sc, codes, sc, None, None, bufs(60), 4, 4, K, 0, 0, None, 0, s) == BOUNDS
        assert fp4.fp4_gemm(codes, bufs(nsc - 64), codes, sc, None, None, bufs(64), 4, 4, K, 0, 0, None, 0,
                            s) == BOUNDS
        # Dequantise: out 4 x 64 FP32.
        assert fp4.fp4_dequantize(codes, sc, None, 0, bufs(1024), 0, rows, K, s) == 0
        assert fp4.fp4_dequantize(codes, sc, None, 0, bufs(1008), 0, rows, K, s) == BOUNDS
        # Hadamard: y 4 x 64 FP32.
        assert fp4.fp4_hadamard16(x, 0, bufs(1024), 0, rows, K, 1, s) == 0
        assert fp4.fp4_hadamard16(x, 0, bufs(1000), 0, rows, K, 1, s) == BOUNDS
        torch.cuda.synchronize()
    finally:
        bufs.free()


@pytest.mark.parametrize("case", ["sum", "decreasing", "first", "token"])
def test_debug_mode_refuses_bad_group_indices(debug, case):
    """Group offsets that do not start at 0, decrease or do not end at
    total_rows, and a token index past A's rows: FP4_ERR_BOUNDS before the
    launch; the well-formed call passes and matches debug mode off."""
    import torch
    fp4 = debug
    E, N, K, T = 3, 64, 256, 40
    t = fp4.quantize(to_dev(synth.gaussian(60, (T, K))), fp4.MXFP4)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, fp4.fp4_scale_bytes(0, N, K)), dtype=torch.uint8, device="cuda")
    for e in range(E):
        fp4.quantize(to_dev(synth.gaussian(61 + e, (N, K), std=0.02)), 0,
                     out=fp4.Quantized(codes[e], scales[e], None, 0, N, K))
    off = np.array([0, 10, 25, 50], dtype=np.int32)
    idx = (np.arange(50) % T).astype(np.int32)
    total = 50
    if case == "sum":
        off[-1] = 49
    elif case == "decreasing":
        off[2] = 5
    elif case == "first":
        off[0] = 1
    else:
        idx[7] = T
    C = torch.empty((total, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    ri, go = torch.from_numpy(idx).cuda(), torch.from_numpy(off).cuda()
    say("debug: grouped indices %s" % case)
    rc = fp4.fp4_gemm_grouped(t.codes.data_ptr(), t.scales.data_ptr(), T, ri.data_ptr(), go.data_ptr(), E,
                              codes.data_ptr(), scales.data_ptr(), None, None, C.data_ptr(), total, N, K, 0, 0,
                              None, 0, s)
    assert rc == BOUNDS
    good_off = torch.tensor([0, 10, 25, 50], dtype=torch.int32, device="cuda")
    good_idx = torch.from_numpy((np.arange(50) % T).astype(np.int32)).cuda()
    rc = fp4.fp4_gemm_grouped(t.codes.data_ptr(), t.scales.data_ptr(), T, good_idx.data_ptr(), good_off.data_ptr(),
                              E, codes.data_ptr(), scales.data_ptr(), None, None, C.data_ptr(), total, N, K, 0, 0,
                              None, 0, s)
    assert rc == 0
    ref = fp4.gemm_grouped(t, good_idx, good_off, codes, scales, N, K, 0, out_dtype=torch.float32)
    assert np.array_equal(to_host(C), to_host(ref))


def test_library_loaded_before_torch_shares_its_runtime():
    """A program that loads the library (here through fp4_set_debug) before
    importing torch: the binding imports torch first, so the library's own
    HIP calls see torch's device (debug mode makes such calls on every entry
    point)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prog = ("import block_scaled_fp4_03_amd as fp4\n"
            "fp4.fp4_set_debug(1)\n"
            "import torch\n"
            "q = fp4.quantize(torch.ones(4, 64, device='cuda'), fp4.NVFP4)\n"
            "torch.cuda.synchronize()\n"
            "import numpy as np\n"
            "assert q.tensor_scale.item() == float(np.float32(1.0) / np.float32(2688.0)), q.tensor_scale.item()\n"
            "print('ok')\n")
    say("library loaded before torch, in a child process")
    env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", prog], capture_output=True, text=True, timeout=120, env=env, cwd=root)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
