"""GPU MXFP8 quantiser and W4A8 GEMM (MXFP8 activations x MXFP4 weights;
"Rubin FP4 GEMM deep dive" §3.4) against the oracle.

- Quantiser: codes (one E4M3 byte per element) and tiled scale bytes equal the
  oracle's bit for bit, both scale rules, FP32 and BF16 inputs, ragged rows,
  K not a multiple of 256, edge values; dequantisation bit-exact.
- GEMM: every output element within 1e-5 * sum |a * b| of the oracle's FP64
  product (FP32 output), or inside the BF16-rounded interval of that bound --
  the tolerance every FP4 GEMM here meets; bit-exact on data whose partial
  sums are exact in FP32; the bias / ReLU epilogue; K of one partial stage;
  the full 8192^3 size on sampled rows and columns.

Why no wider bound is needed.  The gfx950 FP8 x FP4 block-scaled matrix
instruction sums the products of each 16-value K group in a fixed-point
window anchored at the group's largest E4M3 exponent plus its largest E2M1
exponent, truncating each product to a multiple of 2^(anchor - 13)
(measured on the device: 448 * 4 next to a small value v keeps only the part
of 4v above 2^-3).  The kernel runs every step twice, once on the A elements
of magnitude >= 2 (before the block scale) and once on the others, so that
within either part every element is within 7 binades of the part's largest
and no product is cut; test_w4a8_exact_where_one_instruction_truncates pins
that on the very data a single instruction truncates."""
import numpy as np
import pytest

import synth
from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

F8, F8O, F4 = 3, 4, 0


def w4a8_bound(T):
    """The GEMM tolerance of every FP4 GEMM here: 1e-5 * sum |a * b|."""
    return 1e-5 * T


def assert_w4a8_close(orc, C, Cref, bound, out_bf16, what):
    lo, hi = Cref - bound, Cref + bound
    if out_bf16:
        c = orc.bf16_bits_to_f32(C).astype(np.float64)
        lo = orc.bf16_bits_to_f32(orc.f32_to_bf16_bits(lo.astype(np.float32))).astype(np.float64)
        hi = orc.bf16_bits_to_f32(orc.f32_to_bf16_bits(hi.astype(np.float32))).astype(np.float64)
    else:
        c = C.astype(np.float64)
    ok = (c >= lo) & (c <= hi)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d / %d outside 1e-5 * sum|ab|; at %s got %r ref %r bound %r"
                             % (what, (~ok).sum(), ok.size, i, float(c[i]), float(Cref[i]), float(bound[i])))


def _q(orc, x, fmt):
    import block_scaled_fp4_03_amd as fp4
    q = fp4.quantize(to_dev(x), fmt)
    ref = orc.quantize(x, fmt)
    np.testing.assert_array_equal(to_host(q.codes), ref[0])
    np.testing.assert_array_equal(to_host(q.scales), ref[1])
    return q, ref


@pytest.mark.parametrize("fmt", [F8, F8O])
@pytest.mark.parametrize("rows,K", [(1, 32), (17, 96), (33, 2880), (64, 4096), (300, 544), (3, 8192)])
@pytest.mark.parametrize("bf16", [False, True])
def test_mxfp8_quantize_bit_exact(orc, fmt, rows, K, bf16):
    x = synth.gaussian(rows * 13 + K, (rows, K), every=101, bernoulli=0.002)
    if bf16:
        x = synth.to_bf16_bits(x)
    say("mxfp8 quantize fmt=%d rows=%d K=%d bf16=%s" % (fmt, rows, K, bf16))
    _q(orc, x, fmt)


@pytest.mark.parametrize("fmt", [F8, F8O])
def test_mxfp8_edge_values(orc, fmt):
    """Zeros and -0, values far below the block maximum (E4M3 subnormals and
    underflow to zero), exact ties between E4M3 neighbours, a block at the top
    of the FP32 range, FP32 subnormals, and maxima just above 448 * 2^k (the
    OCP rule saturates those)."""
    g = synth.rng(91)
    rows, K = 10, 512
    x = synth.gaussian(91, (rows, K))
    x[0] = 0.0
    x[1] = -0.0
    x[2, ::2] *= np.float32(1e-5)
    x[3] = 0.0
    x[3, ::32] = 448.0
    m = g.integers(0, 7, K).astype(np.float32)
    x[3, 1::2] = ((1.0 + m / 8.0 + 1.0 / 16.0) * np.ldexp(1.0, g.integers(-9, 8, K)))[1::2]
    x[4] = np.float32(3e38) * (g.random(K) - 0.5)
    x[5] = np.float32(1e-40) * g.standard_normal(K)
    x[6] = np.nextafter(np.float32(448.0), np.float32(1e3)) * np.ldexp(1.0, g.integers(-5, 5, K))
    x[7, :] = np.float32(460.0)
    say("mxfp8 edge values fmt=%d" % fmt)
    _q(orc, x.astype(np.float32), fmt)


@pytest.mark.parametrize("fmt", [F8, F8O])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_mxfp8_dequantize_bit_exact(orc, fmt, bf16_out):
    import block_scaled_fp4_03_amd as fp4
    import torch
    rows, K = 70, 1056
    x = synth.gaussian(92, (rows, K), bernoulli=0.01)
    say("mxfp8 dequantize fmt=%d bf16=%s" % (fmt, bf16_out))
    q, ref = _q(orc, x, fmt)
    got = to_host(fp4.dequantize(q, torch.bfloat16 if bf16_out else torch.float32))
    want = orc.dequantize(ref[0], ref[1], 1.0, fmt, rows, K, out_bf16=bf16_out)
    np.testing.assert_array_equal(got, want)


def _w4a8_case(orc, M, N, K, bf16_out, seed, fmtA=F8, with_bias=False, act=0):
    import block_scaled_fp4_03_amd as fp4
    import torch
    a = synth.gaussian(seed, (M, K), every=509 if M * K >= 509 else None, bernoulli=0.002)
    b = synth.gaussian(seed + 1, (N, K), std=0.05, bernoulli=0.002)
    say("w4a8 M=%d N=%d K=%d bf16=%s fmtA=%d bias=%s act=%d" % (M, N, K, bf16_out, fmtA, with_bias, act))
    qa, ra = _q(orc, a, fmtA)
    qb, rb = _q(orc, b, F4)
    bias = (0.5 * synth.gaussian(seed + 2, (N,))).astype(np.float32) if with_bias else None
    C = fp4.gemm_w4a8(qa, qb, bias=None if bias is None else to_dev(bias), act=act,
                      out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    Cref, T = orc.gemm_mixed(ra[0], ra[1], fmtA, rb[0], rb[1], F4, M, N, K)
    bound = w4a8_bound(T)
    if bias is None and not act:
        assert_w4a8_close(orc, to_host(C), Cref, bound, bf16_out, "w4a8 M=%d N=%d K=%d" % (M, N, K))
        return
    # epilogue: the product within the bound, + bias (one FP32 rounding), ReLU
    lo, hi = Cref - bound, Cref + bound
    if bias is not None:
        lo, hi = lo + bias.astype(np.float64), hi + bias.astype(np.float64)
    lo, hi = lo - np.abs(lo) * 2.0 ** -23, hi + np.abs(hi) * 2.0 ** -23
    if act:
        lo, hi = np.maximum(lo, 0.0), np.maximum(hi, 0.0)
    c = to_host(C)
    c = orc.bf16_bits_to_f32(c).astype(np.float64) if bf16_out else c.astype(np.float64)
    if bf16_out:
        lo, hi = lo - np.abs(lo) * 2.0 ** -8, hi + np.abs(hi) * 2.0 ** -8
    ok = (c >= lo) & (c <= hi)
    assert ok.all(), "%d / %d outside the epilogue interval" % ((~ok).sum(), ok.size)
    if act:
        assert not np.signbit(c).any()


SHAPES = [(256, 256, 256), (1, 1, 32), (17, 33, 96), (300, 260, 544), (512, 512, 1024), (257, 513, 2880),
          (64, 640, 128), (520, 16, 4096), (40, 100, 160)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("bf16_out", [False, True])
def test_w4a8_gemm(orc, M, N, K, bf16_out):
    _w4a8_case(orc, M, N, K, bf16_out, seed=M * 7 + N * 3 + K)


def test_w4a8_gemm_ocp_activations(orc):
    _w4a8_case(orc, 129, 255, 640, False, seed=12, fmtA=F8O)


@pytest.mark.parametrize("with_bias,act", [(True, 0), (True, 1), (False, 1)])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_w4a8_epilogue(orc, with_bias, act, bf16_out):
    _w4a8_case(orc, 300, 288, 1024, bf16_out, seed=21, with_bias=with_bias, act=act)


def _grid8(seed, rows, K):
    """Values k / 4 (k = 0..15) with random signs, each 32-block holding a
    +-3.75, so the MXFP8 scale is 2^-6 and the E4M3 codes hold 16 k exactly
    (exponents 4..7: with E2M1 every product lies well inside the matrix
    core's 14-bit window)."""
    g = synth.rng(seed)
    x = (g.integers(0, 16, (rows, K)) * 0.25).astype(np.float32) * np.where(g.random((rows, K)) < 0.5, -1, 1)
    x[:, ::32] = np.float32(3.75) * np.where(g.random((rows, K // 32)) < 0.5, -1, 1)
    return x.astype(np.float32)


def _grid4(seed, rows, K):
    g = synth.rng(seed)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = grid[g.integers(0, 8, (rows, K))] * np.where(g.random((rows, K)) < 0.5, -1, 1).astype(np.float32)
    x[:, ::32] = np.float32(6.0) * np.where(g.random((rows, K // 32)) < 0.5, -1, 1)
    return x.astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(300, 288, 512), (256, 512, 256), (33, 96, 1056)])
def test_w4a8_exact_on_grid(orc, M, N, K):
    """Every product is a multiple of 1/8, no product is cut by the matrix
    core's window, and every partial sum stays below 2^21 eighths, exact in
    FP32 in any order: the result equals the oracle's bit for bit (FP32
    output)."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    say("w4a8 exact M=%d N=%d K=%d" % (M, N, K))
    qa, ra = _q(orc, _grid8(1, M, K), F8)
    qb, rb = _q(orc, _grid4(2, N, K), F4)
    C = to_host(fp4.gemm_w4a8(qa, qb, out_dtype=torch.float32))
    Cref, _ = orc.gemm_mixed(ra[0], ra[1], F8, rb[0], rb[1], F4, M, N, K)
    np.testing.assert_array_equal(C.astype(np.float64), Cref)


def test_w4a8_k_zero_gives_bias(orc):
    import block_scaled_fp4_03_amd as fp4
    import torch
    M, N = 5, 64
    a = fp4.Quantized(torch.zeros((M, 0), dtype=torch.uint8, device="cuda"),
                      torch.zeros(0, dtype=torch.uint8, device="cuda"), None, F8, M, 0)
    b = fp4.Quantized(torch.zeros((N, 0), dtype=torch.uint8, device="cuda"),
                      torch.zeros(0, dtype=torch.uint8, device="cuda"), None, F4, N, 0)
    bias = (synth.gaussian(5, (N,))).astype(np.float32)
    say("w4a8 K=0")
    C = to_host(fp4.gemm_w4a8(a, b, bias=to_dev(bias), act=1, out_dtype=torch.float32))
    np.testing.assert_array_equal(C, np.tile(np.maximum(bias, 0.0), (M, 1)))


def test_w4a8_full_size_8192(orc):
    """The 8192^3 W4A8 workload (the MXFP4 headline's inputs, A quantised to
    MXFP8): 4 sampled rows, every column, against the oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    n = 8192
    a, b = synth.mxfp4_8192(n)
    say("w4a8 8192^3")
    qa = fp4.quantize(to_dev(a), F8)
    qb = fp4.quantize(to_dev(b), F4)
    C = to_host(fp4.gemm_w4a8(qa, qb, out_dtype=torch.bfloat16))
    rows = np.array([0, 1, 4097, 8191])
    ra = orc.quantize(a[rows], F8)
    np.testing.assert_array_equal(to_host(qa.codes)[rows], ra[0])
    rb = orc.quantize(b, F4)
    np.testing.assert_array_equal(to_host(qb.scales), rb[1])
    rr = np.repeat(np.arange(len(rows)), n)
    cc = np.tile(np.arange(n), len(rows))
    Cref, T = orc.gemm_mixed_sampled(ra[0], ra[1], F8, rb[0], rb[1], F4, len(rows), n, n, rr, cc)
    bound = w4a8_bound(T.reshape(len(rows), n))
    assert_w4a8_close(orc, C[rows], Cref.reshape(len(rows), n), bound, True, "w4a8 8192^3 sampled rows")


def test_w4a8_exact_where_one_instruction_truncates(orc):
    """Data on which one FP8 x FP4 instruction loses bits, multiplied exactly.
    B is all 4.0 (E2M1 exponent 2 everywhere, block scale 1); row r of A holds
    448 at the start of each 16-value group and, two positions on, a small
    value v_r of either sign (E4M3 subnormals up to 16, across the split's
    exponent-field boundary at 2); every other element is 0.  A single
    instruction would truncate each product to a multiple of 2^(8 + 2 - 13)
    and drop the low bits of 4 v_r; the kernel's two-part product gives
    4 * (448 * 4 + 4 v_r), exact in FP32, bit for bit."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    M, N, K = 32, 32, 64
    smalls = [0x01, 0x07, 0x08, 0x0F, 0x10, 0x17, 0x18, 0x1F, 0x20, 0x28, 0x30, 0x38, 0x3F, 0x40, 0x48, 0x58]
    codes = np.zeros((M, K), np.uint8)
    for r in range(M):
        c = smalls[r % 16] | (0x80 if r >= 16 else 0)
        for g in range(K // 16):
            codes[r, 16 * g] = 0x7E
            codes[r, 16 * g + 2] = c
    bcodes = np.full((N, K // 2), 0x66, np.uint8)         # every nibble 6 -> 4.0
    sA = np.zeros(orc.scale_bytes(F8, M, K), np.uint8)
    sB = np.zeros(orc.scale_bytes(F4, N, K), np.uint8)
    for r in range(M):
        for b in range(K // 32):
            sA[orc.scale_offset(F8, M, K, r, b)] = 127
            sB[orc.scale_offset(F4, N, K, r, b)] = 127
    qa = fp4.Quantized(to_dev(codes), to_dev(sA), None, F8, M, K)
    qb = fp4.Quantized(to_dev(bcodes), to_dev(sB), None, F4, N, K)
    say("w4a8 exact where one instruction truncates")
    C = to_host(fp4.gemm_w4a8(qa, qb, out_dtype=torch.float32))
    lsb = 2.0 ** (8 + 2 - 13)
    exact = np.zeros((M, N))
    truncated = np.zeros(M)
    for r in range(M):
        v = orc.e4m3_value(int(codes[r, 2]))
        exact[r, :] = (K // 16) * (448.0 * 4.0 + v * 4.0)
        truncated[r] = (K // 16) * (448.0 * 4.0 + np.trunc(v * 4.0 / lsb) * lsb)
    np.testing.assert_array_equal(C.astype(np.float64), exact)
    Cref, _ = orc.gemm_mixed(codes, sA, F8, bcodes, sB, F4, M, N, K)
    np.testing.assert_array_equal(C.astype(np.float64), Cref)
    # The data does reach the truncation a single instruction applies.
    assert (truncated != exact[:, 0]).sum() == 12      # v below 2^-1 in magnitude, both signs
