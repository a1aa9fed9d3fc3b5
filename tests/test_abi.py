"""The C ABI library loads, exports every entry point include/fp4.h declares,
and rejects bad arguments synchronously, before any HIP call (so these run
without a GPU)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_03_amd as fp4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "fp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(fp4_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fp4.LIB_PATH):
        import block_scaled_fp4_03_amd.build as b
        b.build()
    return fp4.lib()


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert set(names) == set(fp4.FUNCTIONS), names
    for n in names:
        assert hasattr(L, n), n
        assert isinstance(getattr(L, n), ctypes._CFuncPtr)


def test_status_strings(L):
    for s in range(0, -10, -1):
        assert fp4.fp4_status_string(s).startswith("FP4_")
    assert "unknown" in fp4.fp4_status_string(5)
    assert "unknown" in fp4.fp4_status_string(-10)


def test_debug_mode_switch(L):
    """fp4_set_debug is host-only and returns the previous setting; argument
    errors are still reported before any check that would call HIP."""
    prev = fp4.fp4_set_debug(1)
    try:
        assert fp4.fp4_set_debug(1) == 1
        assert fp4.fp4_quantize(FAKE, 7, FAKE, FAKE, None, 4, 64, 0, 0, None, 0, None) == -4
        assert fp4.fp4_gemm(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 4, 48, 0, 1, None, 0, None) == -2
        assert fp4.fp4_set_debug(0) == 1
        assert fp4.fp4_set_debug(0) == 0
    finally:
        fp4.fp4_set_debug(prev)


def test_scale_bytes(L):
    assert fp4.fp4_scale_bytes(fp4.MXFP4, 256, 256) == 8 * 1 * 256
    assert fp4.fp4_scale_bytes(fp4.NVFP4, 8192, 8192) == 256 * 32 * 512
    assert fp4.fp4_scale_bytes(fp4.MXFP4, 5760, 2880) == 180 * 12 * 256
    assert fp4.fp4_scale_bytes(fp4.MXFP4, 17, 96) == 1 * 1 * 256
    assert fp4.fp4_scale_bytes(fp4.MXFP4, 4, 48) == -2  # K % 32
    assert fp4.fp4_scale_bytes(fp4.NVFP4, 4, 48) == 512
    assert fp4.fp4_scale_bytes(7, 4, 64) == -4
    assert fp4.fp4_scale_bytes(fp4.MXFP4, -1, 64) == -2


def test_scale_bytes_agrees_with_oracle(L, orc):
    for fmt in (0, 1, 2):
        for rows, K in [(1, 32), (16, 512), (33, 2880), (100, 4096)]:
            assert fp4.fp4_scale_bytes(fmt, rows, K) == orc.scale_bytes(fmt, rows, K)


def test_workspace_sizes(L):
    assert fp4.fp4_workspace_size(fp4.OP_QUANTIZE, fp4.MXFP4, 10, 0, 64) == 0
    assert fp4.fp4_workspace_size(fp4.OP_QUANTIZE, fp4.NVFP4, 10, 0, 64) == 16
    assert fp4.fp4_workspace_size(fp4.OP_GEMM, fp4.MXFP4, 8192, 8192, 8192) == 0
    assert fp4.fp4_workspace_size(fp4.OP_GEMM, fp4.NVFP4, 1, 8192, 8192) == 0
    assert fp4.fp4_workspace_size(fp4.OP_GEMM, fp4.NVFP4, 32, 8192, 8192) == 0
    # Grouped (optional): the routed token rows in expert order, codes padded
    # to 256 bytes, then their scale tiles.
    assert fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, fp4.MXFP4, 65536, 5760, 2880, 32) == \
        65536 * 1440 + 2048 * 12 * 256
    assert fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, fp4.MXFP4_OCP, 100, 64, 544, 3) == \
        (100 * 272 + 255) // 256 * 256 + 4 * 3 * 256
    assert fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, fp4.NVFP4, 100, 64, 544, 3) == 0   # gathers in the GEMM
    assert fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, fp4.MXFP4, 8, 16, 40, 2) == 0   # K % 32


FAKE = 0x100000  # 16-byte-aligned fake device address: never dereferenced on the error paths
ODD = FAKE + 2


def test_quantize_argument_errors(L):
    q = fp4.fp4_quantize
    # fmt, dtype, flags
    assert q(FAKE, 9, FAKE, FAKE, FAKE, 4, 64, 0, 0, None, 0, None) == -4
    assert q(FAKE, 0, FAKE, FAKE, FAKE, 4, 64, 3, 0, None, 0, None) == -5
    assert q(FAKE, 0, FAKE, FAKE, FAKE, 4, 64, 0, 4, None, 0, None) == -8
    # shapes
    assert q(FAKE, 0, FAKE, FAKE, FAKE, -1, 64, 0, 0, None, 0, None) == -2
    assert q(FAKE, 0, FAKE, FAKE, FAKE, 4, 48, 0, 0, None, 0, None) == -2   # MXFP4 needs K % 32
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 40, 0, 0, None, 0, None) == -2   # NVFP4 needs K % 16
    # empty is a no-op even with NULL pointers
    assert q(None, 0, None, None, None, 0, 64, 0, 0, None, 0, None) == 0
    assert q(None, 1, None, None, None, 5, 0, 0, 0, None, 0, None) == 0
    # NULLs
    assert q(None, 0, FAKE, FAKE, None, 4, 64, 0, 0, None, 0, None) == -1
    assert q(FAKE, 1, FAKE, FAKE, None, 4, 64, 0, 0, FAKE, 8, None) == -1   # NVFP4 needs tensor_scale
    # alignment
    assert q(ODD, 0, FAKE, FAKE, None, 4, 64, 0, 0, None, 0, None) == -3
    assert q(FAKE, 0, ODD, FAKE, None, 4, 64, 0, 0, None, 0, None) == -3
    # NVFP4 computing its tensor scale needs the workspace
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 64, 0, 0, None, 0, None) == -6
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 64, 0, 0, FAKE, 4, None) == -6
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 64, 0, 0, FAKE, 8, None) == -6   # 16 bytes since the one-launch grid path


def test_dequantize_argument_errors(L):
    d = fp4.fp4_dequantize
    assert d(FAKE, FAKE, None, 5, FAKE, 0, 4, 64, None) == -4
    assert d(FAKE, FAKE, None, 0, FAKE, 2, 4, 64, None) == -5
    assert d(FAKE, FAKE, None, 0, FAKE, 0, 4, 50, None) == -2
    assert d(FAKE, FAKE, None, 1, FAKE, 0, 4, 64, None) == -1
    assert d(None, None, None, 0, None, 0, 0, 64, None) == 0
    assert d(FAKE, FAKE, None, 0, ODD, 0, 4, 64, None) == -3


def test_gemm_argument_errors(L):
    g = fp4.fp4_gemm
    args = dict(A=FAKE, sA=FAKE, B=FAKE, sB=FAKE, tsA=None, tsB=None, C=FAKE, M=4, N=4, K=64, fmt=0, out=0)

    def call(**kw):
        a = dict(args, **kw)
        return g(a["A"], a["sA"], a["B"], a["sB"], a["tsA"], a["tsB"], a["C"], a["M"], a["N"], a["K"], a["fmt"],
                 a["out"], None, 0, None)

    assert call(fmt=4) == -4
    assert call(out=7) == -5
    assert call(K=48) == -2            # K % 32 for the GEMM
    assert call(M=-1) == -2
    assert call(M=0, C=None) == 0      # empty output: no-op
    assert call(C=None) == -1
    assert call(A=None) == -1
    assert call(fmt=1) == -1           # NVFP4 needs both tensor scales
    assert call(A=ODD) == -3
    assert call(C=FAKE + 1, out=1) == -3


def test_grouped_argument_errors(L):
    g = fp4.fp4_gemm_grouped

    def call(**kw):
        a = dict(A=FAKE, sA=FAKE, A_rows=8, row_idx=FAKE, off=FAKE, E=2, B=FAKE, sB=FAKE, tsA=None, tsB=None, C=FAKE,
                 total=8, N=16, K=64, fmt=0, out=1, ws=None, wsb=0)
        a.update(kw)
        return g(a["A"], a["sA"], a["A_rows"], a["row_idx"], a["off"], a["E"], a["B"], a["sB"], a["tsA"], a["tsB"],
                 a["C"], a["total"], a["N"], a["K"], a["fmt"], a["out"], a["ws"], a["wsb"], None)

    assert call(fmt=3) == -4
    assert call(fmt=1) == -1                    # NVFP4 without tensor scales
    assert call(fmt=1, tsA=FAKE, tsB=FAKE + 2) == -3
    assert call(K=40) == -2
    assert call(E=-1) == -2
    assert call(total=0) == 0
    assert call(row_idx=None) == -1
    assert call(off=FAKE + 2) == -3
    # The optional workspace: too small, misaligned.
    need = fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, 0, 8, 16, 64, 2)
    assert need > 0
    assert call(ws=FAKE, wsb=need - 1) == -6
    assert call(ws=FAKE + 8, wsb=need) == -3


def test_fused_decode_argument_errors(L):
    g = fp4.fp4_gemm_nvfp4_act

    def call(**kw):
        a = dict(X=FAKE, xdt=1, ts=None, flags=0, W=FAKE, sW=FAKE, tsW=FAKE, C=FAKE, M=1, N=64, K=8192, out=1)
        a.update(kw)
        return g(a["X"], a["xdt"], a["ts"], a["flags"], a["W"], a["sW"], a["tsW"], a["C"], a["M"], a["N"], a["K"],
                 a["out"], None)

    assert call(xdt=2) == -5
    assert call(out=3) == -5
    assert call(flags=2) == -8
    assert call(K=8176) == -2          # K % 32
    assert call(M=-1) == -2
    assert call(M=16) == -2            # 16 x 8192 does not fit the fused staging
    assert call(M=0, C=None) == 0      # empty output: no-op
    assert call(C=None) == -1
    assert call(tsW=None) == -1
    assert call(X=None) == -1
    assert call(flags=1) == -1         # a given tensor scale must be passed
    assert call(X=ODD) == -3
    assert call(C=FAKE + 1, out=1) == -3


def test_fused_decode_supported_shapes(L):
    s = fp4.fp4_gemm_nvfp4_act_supported
    assert s(1, 8192, 8192, fp4.BF16) == 1
    assert s(8, 8192, 8192, fp4.BF16) == 1
    assert s(16, 8192, 8192, fp4.BF16) == 0
    assert s(4, 8192, 8192, fp4.F32) == 1
    assert s(8, 8192, 8192, fp4.F32) == 1     # M <= 8: the block-sum decode kernel stages up to 4096 blocks
    assert s(8, 64, 8704, fp4.F32) == 0       # 4352 blocks: neither decode kernel's staging holds them
    assert s(1, 64, 32768, fp4.BF16) == 1
    assert s(32, 64, 1024, fp4.BF16) == 1
    assert s(33, 64, 1024, fp4.BF16) == 0
    assert s(1, 64, 48, fp4.BF16) == 0  # K % 32
    assert s(0, 64, 1024, fp4.BF16) == 0


def test_gemm_ex_argument_errors(L):
    """fp4_gemm_ex rejects bad arguments before any HIP call (fake pointers)."""
    g = fp4.fp4_gemm_ex

    def call(**kw):
        a = dict(A=FAKE, sA=FAKE, B=FAKE, sB=FAKE, tsA=None, tsB=None, bias=None, act=0, C=FAKE, Cs=FAKE, tsC=None,
                 M=64, N=64, K=256, fmt=0, out=2)
        a.update(kw)
        return g(a["A"], a["sA"], a["B"], a["sB"], a["tsA"], a["tsB"], a["bias"], a["act"], a["C"], a["Cs"],
                 a["tsC"], a["M"], a["N"], a["K"], a["fmt"], a["out"], None)

    assert call(fmt=3) == -4
    assert call(out=5) == -5
    assert call(out=-1) == -5
    assert call(out=4) == -1            # NVFP4 output needs the caller's tensor scale
    assert call(out=4, tsC=FAKE + 2) == -3
    assert call(out=4, tsC=FAKE, N=48) == -2
    assert call(out=4, tsC=FAKE, Cs=None) == -1
    assert call(act=2) == -8
    assert call(K=48) == -2             # K % 32
    assert call(N=48) == -2             # FP4 output needs N % 32 == 0
    assert call(M=-1) == -2
    assert call(M=0) == 0 and call(N=0) == 0
    assert call(C=None) == -1
    assert call(Cs=None) == -1          # FP4 output needs the scale buffer
    assert call(fmt=1) == -1            # NVFP4 needs both tensor scales
    assert call(bias=FAKE + 4) == -3    # bias 16-byte aligned
    assert call(C=FAKE + 4) == -3       # FP4 output codes 16-byte aligned
    assert call(Cs=FAKE + 2) == -3
    assert call(A=FAKE + 8) == -3


def test_quantize_ex_and_hadamard_argument_errors(L):
    q = fp4.fp4_quantize_ex
    assert q(FAKE, 0, FAKE, FAKE, None, 4, 64, 0, fp4.Q_2D, 0, None, 0, None) == -4     # 2-D needs NVFP4
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 64, 0, 16, 0, None, 0, None) == -8           # unknown flag
    assert fp4.fp4_quantize(FAKE, 0, FAKE, FAKE, None, 4, 64, 0, fp4.Q_SR, None, 0, None) == -8  # not a quantize flag
    h = fp4.fp4_hadamard16
    assert h(FAKE, 0, FAKE, 0, 4, 40, 0, None) == -2       # K % 16
    assert h(FAKE, 2, FAKE, 0, 4, 64, 0, None) == -5
    assert h(FAKE, 0, FAKE, 3, 4, 64, 0, None) == -5
    assert h(None, 0, FAKE, 0, 4, 64, 0, None) == -1
    assert h(FAKE + 8, 0, FAKE, 0, 4, 64, 0, None) == -3
    assert h(FAKE, 0, FAKE, 0, 0, 64, 0, None) == 0


def test_w4a8_and_mxfp8_argument_errors(L):
    """fp4_gemm_w4a8 and the MXFP8 formats reject bad arguments before any HIP
    call (fake pointers)."""
    g = fp4.fp4_gemm_w4a8

    def call(**kw):
        a = dict(A=FAKE, sA=FAKE, B=FAKE, sB=FAKE, bias=None, act=0, C=FAKE, M=64, N=64, K=256, out=1)
        a.update(kw)
        return g(a["A"], a["sA"], a["B"], a["sB"], a["bias"], a["act"], a["C"], a["M"], a["N"], a["K"], a["out"],
                 None)

    assert call(out=2) == -5
    assert call(act=2) == -8
    assert call(K=48) == -2
    assert call(K=1 << 24) == -2        # an FP8 tile of 256 rows must stay inside 32-bit ranges
    assert call(M=-1) == -2
    assert call(M=0) == 0 and call(N=0) == 0
    assert call(C=None) == -1
    assert call(A=None) == -1
    assert call(A=FAKE + 8) == -3
    assert call(bias=FAKE + 4) == -3
    assert call(out=0, C=FAKE + 2) == -3
    # MXFP8 quantise: no stochastic rounding, codes 8-byte aligned; FP4 GEMMs refuse it
    assert fp4.fp4_quantize_sr(FAKE, 3, FAKE, FAKE, None, 4, 64, 0, 0, 1, None, 0, None) == -4
    assert fp4.fp4_quantize(FAKE, 4, FAKE + 4, FAKE, None, 4, 64, 0, 0, None, 0, None) == -3
    assert fp4.fp4_quantize(FAKE, 5, FAKE, FAKE, None, 4, 64, 0, 0, None, 0, None) == -4
    assert fp4.fp4_quantize(FAKE, 3, FAKE, FAKE, None, 4, 48, 0, 0, None, 0, None) == -2
    assert fp4.fp4_dequantize(FAKE + 4, FAKE, None, 3, FAKE, 0, 4, 64, None) == -3   # MXFP8 codes 8-byte aligned
    assert fp4.fp4_scale_bytes(3, 33, 288) == 2 * 2 * 256
    assert fp4.fp4_gemm(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 64, 64, 256, 3, 1, None, 0, None) == -4


def test_gemm_scale_ranges_are_checked(L):
    """Shapes whose scale buffers would not fit the kernels' 32-bit ranges are
    refused on the host."""
    big = 1 << 25      # rows: (2^25 / 32) tiles * 32 K-tiles * 256 B = 2^33 bytes of scales at K = 8192
    assert fp4.fp4_gemm(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, big, 64, 8192, 0, 1, None, 0, None) == -2
    assert fp4.fp4_gemm(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 64, big, 8192, 0, 1, None, 0, None) == -2
    assert fp4.fp4_gemm_ex(FAKE, FAKE, FAKE, FAKE, None, None, None, 0, FAKE, None, None, big, 64, 8192, 0, 1,
                           None) == -2
    assert fp4.fp4_gemm_grouped(FAKE, FAKE, big, FAKE, FAKE, 4, FAKE, FAKE, None, None, FAKE, 64, 64, 8192, 0, 1,
                                None, 0, None) == -2


def test_quantize_and_dequantize_grid_limits(L):
    """The element-wise kernels index their waves and threads in 32 bits and
    a launch counts its work-items in 32 bits: shapes past that are refused on
    the host (one 64-lane wave per 32-row-padded row and 512-value slice for
    the quantisers, one thread per 8 values for dequantisation)."""
    q, d = fp4.fp4_quantize, fp4.fp4_dequantize
    # 2^26 waves = 2^32 work-items: refused; one slice fewer fits.
    assert q(FAKE, 0, FAKE, FAKE, None, 1 << 20, 1 << 15, 0, 0, None, 0, None) == -2   # 2^20 rows x 64 slices
    assert q(FAKE, 0, FAKE, FAKE, None, 32, 1 << 30, 0, 0, None, 0, None) == -2        # padding rows count too
    # Shapes inside the limit pass the size check and stop at the next one
    # (a NULL output), so nothing is launched on these fake pointers.
    assert q(FAKE, 0, None, FAKE, None, 1, (1 << 29), 0, 0, None, 0, None) == -1       # 32 x 2^20 x 64 < 2^32
    assert q(FAKE, 0, None, FAKE, None, 1 << 20, (1 << 15) - 512, 0, 0, None, 0, None) == -1
    assert d(FAKE, FAKE, None, 0, FAKE, 0, 1 << 20, 1 << 15, None) == -2              # 2^32 threads
    assert d(FAKE, FAKE, None, 0, None, 0, 1 << 19, 1 << 15, None) == -1


def test_wrappers_reject_bad_tensors_before_the_library():
    """The Python wrappers refuse, before any library call, tensors the C ABI
    would misread: int64 indices (read as int32 halves), non-contiguous views
    (silently wrong layout), host tensors (a host pointer handed to a kernel),
    wrong shapes and short buffers."""
    import torch
    need = fp4._need
    ok = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(TypeError):
        need(torch.zeros(8, dtype=torch.int64), "row_idx", (torch.int32,))
    with pytest.raises(ValueError, match="contiguous"):
        need(torch.zeros((8, 8), dtype=torch.float32).t(), "x", (torch.float32,))
    with pytest.raises(ValueError, match="contiguous"):
        need(torch.zeros((8, 16), dtype=torch.float32)[:, :8], "x", (torch.float32,))
    with pytest.raises(ValueError, match="dimensions"):
        need(torch.zeros((2, 4), dtype=torch.int32), "row_idx", (torch.int32,), ndim=1)
    with pytest.raises(ValueError, match="elements"):
        need(ok, "group_off", (torch.int32,), 9)
    with pytest.raises(ValueError, match="GPU"):
        need(ok, "group_off", (torch.int32,), 8)
    with pytest.raises(TypeError):
        need(np_array := [1, 2], "x")  # noqa: F841
    # Whole calls with host tensors stop in the wrapper, not in a kernel.
    x = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        fp4.quantize(x, fp4.MXFP4)
    with pytest.raises(TypeError):
        fp4.quantize(x.to(torch.float64), fp4.MXFP4)
    with pytest.raises(ValueError, match="contiguous"):
        fp4.quantize(torch.zeros((64, 4), dtype=torch.float32).t(), fp4.MXFP4)
    with pytest.raises(ValueError, match="dimensions"):
        fp4.quantize(torch.zeros(64, dtype=torch.float32), fp4.MXFP4)
    with pytest.raises(ValueError, match="GPU"):
        fp4.hadamard16(x, seed=1)
    q = fp4.Quantized(torch.zeros((4, 32), dtype=torch.uint8), torch.zeros(256, dtype=torch.uint8), None,
                      fp4.MXFP4, 4, 64)
    with pytest.raises(ValueError, match="GPU"):
        fp4.gemm(q, q)
    with pytest.raises(ValueError, match="GPU"):
        fp4.dequantize(q)
    with pytest.raises(ValueError, match="GPU"):
        fp4.gemm_ex(q, q)
    short = fp4.Quantized(torch.zeros((4, 16), dtype=torch.uint8), torch.zeros(256, dtype=torch.uint8), None,
                          fp4.MXFP4, 4, 64)
    with pytest.raises(ValueError, match="elements"):
        fp4.gemm(short, q)
    nv = fp4.Quantized(torch.zeros((4, 32), dtype=torch.uint8), torch.zeros(512, dtype=torch.uint8), None,
                       fp4.NVFP4, 4, 64)
    with pytest.raises(ValueError, match="tensor scale"):
        fp4.gemm(nv, nv)
    with pytest.raises(TypeError):
        fp4.gemm("a", q)
    with pytest.raises(ValueError, match="GPU"):
        fp4.gemm_grouped(q, ok, ok, torch.zeros(64, dtype=torch.uint8), torch.zeros(256, dtype=torch.uint8),
                         16, 64, fp4.MXFP4)
    with pytest.raises(ValueError, match="GPU"):
        fp4.gemm_nvfp4_act(x, nv)


def test_quantize_noalloc_argument_errors(L):
    """fp4_quantize_noalloc validates like fp4_quantize, before any HIP call
    (the scratch lookup included)."""
    q = fp4.fp4_quantize_noalloc
    assert q(FAKE, 9, FAKE, FAKE, FAKE, 4, 64, 0, 0, None) == -4
    assert q(FAKE, 0, FAKE, FAKE, FAKE, 4, 64, 3, 0, None) == -5
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 64, 0, fp4.Q_SR, None) == -8      # only FP4_TS_GIVEN
    assert q(FAKE, 1, FAKE, FAKE, FAKE, 4, 40, 0, 0, None) == -2
    assert q(FAKE, 0, FAKE, FAKE, None, 1 << 20, 1 << 15, 0, 0, None) == -2
    assert q(None, 1, None, None, None, 0, 64, 0, 0, None) == 0
    # NVFP4 above 256 KB: argument errors come before the scratch lookup.
    assert q(FAKE, 1, FAKE, FAKE, None, 1024, 1024, 0, 0, None) == -1
    assert q(None, 1, FAKE, FAKE, FAKE, 1024, 1024, 0, 0, None) == -1
    assert q(ODD, 1, FAKE, FAKE, FAKE, 1024, 1024, 0, 0, None) == -3
    # Paths without scratch validate as fp4_quantize does.
    assert q(FAKE, 0, None, FAKE, None, 4, 64, 0, 0, None) == -1
    assert q(FAKE, 1, FAKE, FAKE, None, 4, 64, 0, 0, None) == -1
