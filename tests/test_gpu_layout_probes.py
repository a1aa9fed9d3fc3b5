"""Layout probes through the public GEMM calls: one operand is the identity
matrix, so every output element is a single product and exact.  C[m, n] =
A^[m, n] (B identity) or B^[n, m] (A identity), each value times the scales
of its K block.  Every K position of a 512-value K (both halves of each
64-value step, both 256-value scale tiles), every scale block and both
operands' scale-lane mappings are checked bit for bit, for MXFP4, NVFP4 (tiled
kernel and, at M <= 32, both decode kernels) and W4A8 ("Rubin FP4 GEMM deep
dive" §5.2: nibble order and scale layout must match what the kernel reads)."""
import numpy as np
import pytest

from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

K = 512


def _pack(c):
    c = np.asarray(c, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _scales(orc, fmt, rows, byte_of):
    bs = orc.block_size(fmt)
    s = np.zeros(orc.scale_bytes(fmt, rows, K), np.uint8)
    for r in range(rows):
        for b in range(K // bs):
            s[orc.scale_offset(fmt, rows, K, r, b)] = byte_of(r, b)
    return s


def _scale_value(orc, fmt, byte):
    return orc.e4m3_value(byte) if fmt == 1 else 2.0 ** (byte - 127)


def _gemm(fmt, A, sA, B, sB, M, N, fp8=False):
    import block_scaled_fp4_03_amd as fp4
    import torch
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    dA, dsA, dB, dsB = to_dev(A), to_dev(sA), to_dev(B), to_dev(sB)
    s = torch.cuda.current_stream().cuda_stream
    if fp8:
        rc = fp4.fp4_gemm_w4a8(dA.data_ptr(), dsA.data_ptr(), dB.data_ptr(), dsB.data_ptr(), None, 0, C.data_ptr(),
                               M, N, K, fp4.F32, s)
    else:
        rc = fp4.fp4_gemm(dA.data_ptr(), dsA.data_ptr(), dB.data_ptr(), dsB.data_ptr(), one.data_ptr(),
                          one.data_ptr(), C.data_ptr(), M, N, K, fmt, fp4.F32, None, 0, s)
    assert rc == 0, fp4.fp4_status_string(rc)
    return to_host(C).astype(np.float64)


def _scale_rules(fmt):
    """Distinct scale bytes per (row, block): powers of two 2^-2..2^2 (E8M0) or
    a spread of E4M3 values (NVFP4)."""
    if fmt == 1:
        bytes_ = [0x30, 0x33, 0x38, 0x3B, 0x3E, 0x41, 0x44]
        return (lambda r, b: bytes_[(r + 3 * b) % 7]), (lambda r, b: bytes_[(2 * r + b) % 5])
    return (lambda r, b: 127 + (r + 3 * b) % 5 - 2), (lambda r, b: 127 + (2 * r + b) % 3 - 1)


@pytest.mark.parametrize("fmt", [0, 1])
def test_identity_a_pins_b_layout(orc, fmt):
    """A = identity (512 x 512), B random: C[m, n] = sA(m) * B^[n, m]."""
    M, N = K, 40
    g = np.random.default_rng(31)
    ra, rb = _scale_rules(fmt)
    bs = orc.block_size(fmt)
    A = np.zeros((M, K), np.uint8)
    A[np.arange(M), np.arange(M)] = 2                  # 1.0
    Bc = g.integers(0, 16, (N, K)).astype(np.uint8)
    say("layout: identity A, fmt=%d" % fmt)
    C = _gemm(fmt, _pack(A), _scales(orc, fmt, M, ra), _pack(Bc), _scales(orc, fmt, N, rb), M, N)
    want = np.array([[_scale_value(orc, fmt, ra(m, m // bs)) * orc.e2m1_value(int(Bc[n, m]))
                      * _scale_value(orc, fmt, rb(n, m // bs)) for n in range(N)] for m in range(M)])
    np.testing.assert_array_equal(C, want)


@pytest.mark.parametrize("fmt,M", [(0, 40), (1, 40), (1, 1), (1, 2), (1, 3), (1, 8), (1, 32)])
def test_identity_b_pins_a_layout(orc, fmt, M):
    """B = identity (512 x 512), A random: C[m, n] = A^[m, n] * sB(n).  NVFP4
    with M <= 8 takes the block-sum decode kernel (M = 1, 2, 3, 8: one, two,
    four and eight activation rows per operand), M = 32 the FP16-decode kernel."""
    N = K
    g = np.random.default_rng(32 + M)
    ra, rb = _scale_rules(fmt)
    bs = orc.block_size(fmt)
    Ac = g.integers(0, 16, (M, K)).astype(np.uint8)
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), np.arange(N)] = 2
    say("layout: identity B, fmt=%d M=%d" % (fmt, M))
    C = _gemm(fmt, _pack(Ac), _scales(orc, fmt, M, ra), _pack(B), _scales(orc, fmt, N, rb), M, N)
    want = np.array([[_scale_value(orc, fmt, ra(m, n // bs)) * orc.e2m1_value(int(Ac[m, n]))
                      * _scale_value(orc, fmt, rb(n, n // bs)) for n in range(N)] for m in range(M)])
    np.testing.assert_array_equal(C, want)


def test_w4a8_identity_a_pins_b_layout(orc):
    """A = identity in E4M3 (0x38 = 1.0) with per-block scales, B random
    MXFP4: C[m, n] = sA(m) * B^[n, m]."""
    M, N = K, 40
    g = np.random.default_rng(41)
    ra, rb = _scale_rules(0)
    A = np.zeros((M, K), np.uint8)
    A[np.arange(M), np.arange(M)] = 0x38
    Bc = g.integers(0, 16, (N, K)).astype(np.uint8)
    say("layout: w4a8 identity A")
    C = _gemm(0, A, _scales(orc, 3, M, ra), _pack(Bc), _scales(orc, 0, N, rb), M, N, fp8=True)
    want = np.array([[2.0 ** (ra(m, m // 32) - 127) * orc.e2m1_value(int(Bc[n, m])) * 2.0 ** (rb(n, m // 32) - 127)
                      for n in range(N)] for m in range(M)])
    np.testing.assert_array_equal(C, want)


def test_w4a8_identity_b_pins_fp8_layout(orc):
    """B = identity (1.0), A random E4M3 bytes: C[m, n] = E4M3(A[m, n]) *
    sA(m) * sB(n); pins the FP8 operand's lane layout (K [16j, 16j + 16) and
    [32 + 16j, 32 + 16j + 16) per half j).  The codes keep exponent fields
    5..11 (all mantissas, both signs), a range the matrix core's 16-value
    window always holds exactly."""
    M, N = 40, K
    g = np.random.default_rng(42)
    ra, rb = _scale_rules(0)
    Ac = ((g.integers(0, 2, (M, K)) << 7) | (g.integers(5, 12, (M, K)) << 3) | g.integers(0, 8, (M, K))).astype(np.uint8)
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), np.arange(N)] = 2
    say("layout: w4a8 identity B")
    C = _gemm(0, Ac, _scales(orc, 3, M, ra), _pack(B), _scales(orc, 0, N, rb), M, N, fp8=True)
    want = np.array([[orc.e4m3_value(int(Ac[m, n])) * 2.0 ** (ra(m, n // 32) - 127) * 2.0 ** (rb(n, n // 32) - 127)
                      for n in range(N)] for m in range(M)])
    np.testing.assert_array_equal(C, want)
