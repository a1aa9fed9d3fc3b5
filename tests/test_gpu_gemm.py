"""GPU GEMM parity against the oracle's FP64 product of the oracle-quantised
operands: every output element within 1e-5 * sum|a*b| (FP32 outputs) or inside
the BF16-rounded acceptance interval (BF16 outputs); closed forms bit-exact."""
import numpy as np
import pytest

import synth
from gpu_helpers import assert_gemm_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _quant_both(orc, x, fmt):
    """Quantise on the GPU and in the oracle; the bits must agree."""
    import block_scaled_fp4_03_amd as fp4
    q = fp4.quantize(to_dev(x), fmt)
    ref = orc.quantize(x, fmt)
    np.testing.assert_array_equal(to_host(q.codes), ref[0])
    np.testing.assert_array_equal(to_host(q.scales), ref[1])
    return q, ref


def _gemm_case(orc, fmt, M, N, K, bf16_out, seed, a_std=1.0, b_std=1.0):
    import block_scaled_fp4_03_amd as fp4
    import torch
    a = synth.gaussian(seed, (M, K), std=a_std, every=512 if M * K >= 512 else None)
    b = synth.gaussian(seed + 1, (N, K), std=b_std, bernoulli=0.002)
    say("gemm fmt=%d M=%d N=%d K=%d bf16=%s" % (fmt, M, N, K, bf16_out))
    qa, ra = _quant_both(orc, a, fmt)
    qb, rb = _quant_both(orc, b, fmt)
    C = fp4.gemm(qa, qb, out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    Cref, T = orc.gemm(ra[0], ra[1], rb[0], rb[1], M, N, K, fmt, tsA=ra[3], tsB=rb[3])
    assert_gemm_close(orc, to_host(C), Cref, T, bf16_out, "fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))


MX_SHAPES = [(256, 256, 256), (1, 1, 32), (17, 33, 96), (300, 260, 544), (512, 512, 1024), (257, 513, 2880),
             (64, 640, 128), (520, 16, 4096)]


@pytest.mark.parametrize("M,N,K", MX_SHAPES)
@pytest.mark.parametrize("bf16_out", [False, True])
def test_mxfp4_gemm(orc, M, N, K, bf16_out):
    _gemm_case(orc, 0, M, N, K, bf16_out, seed=M * 7 + N * 3 + K)


@pytest.mark.parametrize("M,N,K", [(129, 255, 640)])
def test_mxfp4_ocp_gemm(orc, M, N, K):
    _gemm_case(orc, 2, M, N, K, False, seed=11)


NV_SHAPES = [(256, 256, 256), (1, 1, 32), (17, 33, 96), (300, 260, 544), (512, 512, 1024), (257, 513, 2880),
             (64, 640, 128), (520, 16, 4096)]


@pytest.mark.parametrize("M,N,K", NV_SHAPES)
@pytest.mark.parametrize("bf16_out", [False, True])
def test_nvfp4_gemm(orc, M, N, K, bf16_out):
    _gemm_case(orc, 1, M, N, K, bf16_out, seed=M * 5 + N * 11 + K, a_std=3.0, b_std=0.05)


def test_nvfp4_gemm_row_scaled(orc):
    """Rows with standard deviations spread log-uniformly over [0.01, 1] (the
    MLP workload's law), BF16 activations quantised on the GPU."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    M, N, K = 384, 320, 1024
    a = synth.to_bf16_bits(synth.row_scaled_gaussian(61, M, K))
    w = synth.row_scaled_gaussian(62, N, K)
    say("gemm nvfp4 row-scaled")
    qa, ra = _quant_both(orc, a, 1)
    qb, rb = _quant_both(orc, w, 1)
    assert to_host(qa.tensor_scale)[0] == np.float32(ra[3])
    C = fp4.gemm(qa, qb, out_dtype=torch.bfloat16)
    Cref, T = orc.gemm(ra[0], ra[1], rb[0], rb[1], M, N, K, 1, tsA=ra[3], tsB=rb[3])
    assert_gemm_close(orc, to_host(C), Cref, T, True, "nvfp4 row-scaled")


def test_mxfp4_256_config_fp32_out(orc):
    """The 256^3 MXFP4 workload: FP32 A, B with every 512th element x20."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    a, b = synth.mxfp4_256()
    qa, ra = _quant_both(orc, a, 0)
    qb, rb = _quant_both(orc, b, 0)
    say("gemm mxfp4_256")
    C = to_host(fp4.gemm(qa, qb, out_dtype=torch.float32))
    Cref, T = orc.gemm(ra[0], ra[1], rb[0], rb[1], 256, 256, 256, 0)
    assert_gemm_close(orc, C, Cref, T, False, "mxfp4_256")


def _pack(c):
    c = np.asarray(c, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _scales(orc, fmt, rows, K, byte_of):
    s = np.zeros(orc.scale_bytes(fmt, rows, K), np.uint8)
    for r in range(rows):
        for b in range(K // orc.block_size(fmt)):
            s[orc.scale_offset(fmt, rows, K, r, b)] = byte_of(r, b)
    return s


def _run_raw(fmt, A, sA, B, sB, M, N, K, tsA=None, tsB=None):
    import block_scaled_fp4_03_amd as fp4
    import torch
    Cd = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dA, dsA, dB, dsB = to_dev(A), to_dev(sA), to_dev(B), to_dev(sB)
    tA = None if tsA is None else torch.tensor([tsA], dtype=torch.float32, device="cuda")
    tB = None if tsB is None else torch.tensor([tsB], dtype=torch.float32, device="cuda")
    ws = fp4.workspace(fp4.OP_GEMM, fmt, M, N, K)
    rc = fp4.fp4_gemm(dA.data_ptr(), dsA.data_ptr(), dB.data_ptr(), dsB.data_ptr(),
                      None if tA is None else tA.data_ptr(), None if tB is None else tB.data_ptr(), Cd.data_ptr(),
                      M, N, K, fmt, fp4.F32, None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
                      torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fp4.fp4_status_string(rc)
    return to_host(Cd)


@pytest.mark.parametrize("fmt", [0, 1])
def test_closed_forms_bit_exact(orc, fmt):
    """All-6 operands with unit scales give 36*K; one-hot operands pin the
    row/column/K and nibble mapping; alternating signs cancel exactly."""
    M, N, K = 40, 24, 512
    unit = 127 if fmt != 1 else 0x38
    s1a = _scales(orc, fmt, M, K, lambda r, b: unit)
    s1b = _scales(orc, fmt, N, K, lambda r, b: unit)
    say("closed form all-6")
    C = _run_raw(fmt, _pack(np.full((M, K), 7)), s1a, _pack(np.full((N, K), 7)), s1b, M, N, K, 1.0, 1.0)
    np.testing.assert_array_equal(C, np.full((M, N), 36.0 * K, np.float32))
    alt = np.tile(np.array([7, 15], np.uint8), (N, K // 2))
    say("closed form alternating")
    C = _run_raw(fmt, _pack(np.full((M, K), 7)), s1a, _pack(alt), s1b, M, N, K, 1.0, 1.0)
    np.testing.assert_array_equal(C, np.zeros((M, N), np.float32))
    g = np.random.default_rng(5)
    for trial in range(6):
        m, n, k = int(g.integers(M)), int(g.integers(N)), int(g.integers(K))
        a1 = np.zeros((M, K), np.uint8)
        b1 = np.zeros((N, K), np.uint8)
        ca, cb = int(g.integers(1, 16)), int(g.integers(1, 16))
        a1[m, k] = ca
        b1[n, k] = cb
        if fmt == 1:  # E4M3 scales, any byte (normal or subnormal)
            ea, eb = int(g.integers(1, 127)), int(g.integers(1, 127))
            sa = _scales(orc, fmt, M, K, lambda r, b: ea)
            sb = _scales(orc, fmt, N, K, lambda r, b: eb)
            want = orc.e2m1_value(ca) * orc.e2m1_value(cb) * orc.e4m3_value(ea) * orc.e4m3_value(eb)
        else:
            ea, eb = int(g.integers(-5, 6)), int(g.integers(-5, 6))
            sa = _scales(orc, fmt, M, K, lambda r, b: 127 + ea)
            sb = _scales(orc, fmt, N, K, lambda r, b: 127 + eb)
            want = orc.e2m1_value(ca) * orc.e2m1_value(cb) * 2.0 ** (ea + eb)
        say("closed form one-hot m=%d n=%d k=%d" % (m, n, k))
        C = _run_raw(fmt, _pack(a1), sa, _pack(b1), sb, M, N, K, 1.0, 1.0)
        ref = np.zeros((M, N), np.float32)
        ref[m, n] = want
        np.testing.assert_array_equal(C, ref)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 20, 40])
def test_nvfp4_every_e4m3_scale_byte(orc, M):
    """Every finite E4M3 byte as a block scale of A and of B, exactly: W row n
    holds 1.0 codes only in block n, with scale byte n; A row m holds 1.0 codes
    with scale byte (7m + 13b) mod 127 in block b; so C[m, n] = 16 * e4m3(sA) *
    e4m3(n), a product exact in FP32.  M = 1, 2, 3, 5 take the block-sum decode
    kernel (1, 2, 4 and 8 activation rows per operand), M = 20 the FP16 decode
    kernel, M = 40 the tiled GEMM."""
    fmt, N, K = 1, 127, 2048
    A = np.full((M, K), 2, np.uint8)
    B = np.zeros((N, K), np.uint8)
    for n in range(N):
        B[n, 16 * n:16 * n + 16] = 2
    sa = lambda r, b: (7 * r + 13 * b) % 127
    sA = _scales(orc, fmt, M, K, sa)
    sB = _scales(orc, fmt, N, K, lambda r, b: r if b == r else 0x38)
    say("every e4m3 byte M=%d" % M)
    C = _run_raw(fmt, _pack(A), sA, _pack(B), sB, M, N, K, 1.0, 1.0)
    want = np.array([[16.0 * orc.e4m3_value(sa(m, n)) * orc.e4m3_value(n) for n in range(N)] for m in range(M)],
                    np.float32)
    np.testing.assert_array_equal(C, want)


def test_exact_small_exponent_range_bit_exact(orc):
    """Scale exponents within a range of 4 and K <= 256 keep every partial sum
    exact in FP32, so any accumulation order gives the oracle's value."""
    fmt, M, N, K = 0, 48, 80, 256
    g = np.random.default_rng(9)
    A = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    B = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sA = _scales(orc, fmt, M, K, lambda r, b: int(125 + g.integers(0, 3)))
    sB = _scales(orc, fmt, N, K, lambda r, b: int(126 + g.integers(0, 2)))
    say("exact small range")
    C = _run_raw(fmt, A, sA, B, sB, M, N, K)
    Cref, _ = orc.gemm(A, sA, B, sB, M, N, K, fmt)
    np.testing.assert_array_equal(C.astype(np.float64), Cref)


def _band_picks(n, band, seed):
    """One index in each `band`-wide band of range(n) (the first band's is 0,
    the last band's n - 1): with band = 256, one row (or column) in every
    output tile row (or column)."""
    g = np.random.default_rng(seed)
    starts = np.arange(0, n, band)
    picks = starts + g.integers(0, band, starts.size)
    picks = np.minimum(picks, n - 1)
    picks[0], picks[-1] = 0, n - 1
    return picks


def test_mxfp4_8192_every_tile(orc):
    """The 8192^3 MXFP4 workload in the benchmark's launch configuration,
    every 256 x 256 output tile checked: one row in each 256-row band against
    all 8192 columns, and one column in each 256-column band against all 8192
    rows, each against the oracle (which quantises the operands itself)."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    n = 8192
    a, b = synth.mxfp4_8192()
    say("gemm mxfp4_8192 full size")
    qa = fp4.quantize(to_dev(a), 0)
    qb = fp4.quantize(to_dev(b), 0)
    C = to_host(fp4.gemm(qa, qb, out_dtype=torch.bfloat16))
    rows, cols = _band_picks(n, 256, 3), _band_picks(n, 256, 33)
    ra, rb_all = orc.quantize(a[rows], 0), orc.quantize(b, 0)
    Cref, T = orc.gemm(ra[0], ra[1], rb_all[0], rb_all[1], rows.size, n, n, 0)
    assert_gemm_close(orc, C[rows], Cref, T, True, "mxfp4_8192 one row per 256-row band")
    del rb_all
    ra_all, rb = orc.quantize(a, 0), orc.quantize(b[cols], 0)
    Cref, T = orc.gemm(ra_all[0], ra_all[1], rb[0], rb[1], n, cols.size, n, 0)
    assert_gemm_close(orc, C[:, cols], Cref, T, True, "mxfp4_8192 one column per 256-column band")


def test_nvfp4_mlp_every_tile(orc):
    """The 4096 x 14336 x 4096 NVFP4 workload (BF16 activations quantised on
    the fly, weights pre-quantised) in the benchmark's launch configuration,
    every output tile checked: one row per 256-row band x all columns, one
    column per 256-column band x all rows, against the oracle, which
    quantises with the tensor scales it computes from the whole operands."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    M, N, K = 4096, 14336, 4096
    a, w = synth.nvfp4_mlp()
    say("gemm nvfp4_mlp full size")
    qa = fp4.quantize(to_dev(a), 1)
    qw = fp4.quantize(to_dev(w), 1)
    C = to_host(fp4.gemm(qa, qw, out_dtype=torch.bfloat16))
    ts_a = orc.nvfp4_tensor_scale(orc.tensor_amax(a))
    ts_w = orc.nvfp4_tensor_scale(orc.tensor_amax(w))
    assert to_host(qa.tensor_scale)[0] == np.float32(ts_a) and to_host(qw.tensor_scale)[0] == np.float32(ts_w)
    rows, cols = _band_picks(M, 256, 4), _band_picks(N, 256, 44)
    ra = orc.quantize(a[rows], 1, tensor_scale=ts_a)
    rw = orc.quantize(w, 1, tensor_scale=ts_w)
    Cref, T = orc.gemm(ra[0], ra[1], rw[0], rw[1], rows.size, N, K, 1, tsA=ts_a, tsB=ts_w)
    assert_gemm_close(orc, C[rows], Cref, T, True, "nvfp4_mlp one row per 256-row band")
    del rw
    ra = orc.quantize(a, 1, tensor_scale=ts_a)
    rw = orc.quantize(w[cols], 1, tensor_scale=ts_w)
    Cref, T = orc.gemm(ra[0], ra[1], rw[0], rw[1], M, cols.size, K, 1, tsA=ts_a, tsB=ts_w)
    assert_gemm_close(orc, C[:, cols], Cref, T, True, "nvfp4_mlp one column per 256-column band")


# M = 1 with K <= 8192 takes the vector-ALU decode kernel, other M <= 8
# within its K reach the block-sum decode kernel; otherwise the
# FP16-decode kernel stages the activation as FP16 (M x K small), as codes
# (larger), or it is too large for either (the tiled GEMM takes it):
# (8, 100, 8960) is the largest FP16 staging at M = 8 (past the block-sum
# kernel's K = 8192 at M = 8), (32, 130, 8192) the largest code staging,
# (2, 64, 40000) small M past both decode kernels' K reach.
@pytest.mark.parametrize("M,N,K", [(1, 96, 512), (3, 1000, 2880), (8, 333, 1024), (17, 256, 4096), (32, 130, 8192),
                                   (1, 8192, 256), (32, 64, 96), (8, 100, 8960), (9, 100, 8192), (32, 64, 8448),
                                   (2, 64, 40000)])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_nvfp4_decode_gemv(orc, M, N, K, bf16_out):
    """M <= 32 rows take a decode kernel (K split over the workgroup's
    waves, reduced in LDS); checked in full against the oracle."""
    _gemm_case(orc, 1, M, N, K, bf16_out, seed=M * 13 + N + K, a_std=1.0, b_std=0.02)


# The block-sum decode kernel (M <= 8): every operand packing (M = 1, 2,
# 3-4, 5-8), K tails that end inside a 512-value unit and inside a 256-value
# scale tile (K = 96, 288, 800, 4128), several units per wave (K = 17440 at
# M = 1: 35 units; 12320 at M = 2: 25 units), ragged N.
@pytest.mark.parametrize("M,N,K", [(1, 200, 17440), (2, 130, 12320), (4, 96, 4128), (5, 64, 800), (6, 300, 96),
                                   (7, 40, 288), (8, 257, 8192)])
def test_nvfp4_decode_blocksum_shapes(orc, M, N, K):
    _gemm_case(orc, 1, M, N, K, False, seed=M * 7 + N + K, a_std=1.0, b_std=0.02)


# The vector-ALU decode kernel (M = 1, K <= 8192): 16 weight rows per
# workgroup, so ragged N ends inside a workgroup (17, 9, 1000, 33) and inside
# a 32-row scale tile (40); K from one chunk (32) to the maximum (8192), with
# threads past the row's chunks (K = 8160: 255 of 256 chunks; 2880: 90) and
# many tiny workgroups (N = 300, K = 256).  M = 2 takes the block-sum kernel.
@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (1, 17, 64), (1, 9, 8192), (1, 1000, 2880), (1, 33, 8160),
                                   (1, 40, 4096), (1, 300, 256), (1, 48, 8192), (2, 40, 8192)])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_nvfp4_decode_vector_kernel_shapes(orc, M, N, K, bf16_out):
    _gemm_case(orc, 1, M, N, K, bf16_out, seed=M * 5 + N + K, a_std=1.0, b_std=0.02)


def test_nvfp4_decode_gemv_repeated_calls(orc):
    """The decode kernel keeps no state and needs no workspace: several calls
    in a row (a smaller problem after a larger one) all agree with the oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    K = 2048
    assert fp4.fp4_workspace_size(fp4.OP_GEMM, fp4.NVFP4, 32, 1024, K) == 0
    w = synth.gaussian(71, (1024, K), std=0.02, bernoulli=0.001)
    qw, rw = _quant_both(orc, w, 1)
    for M in (32, 8, 1, 32):
        x = synth.to_bf16_bits(synth.gaussian(72 + M, (M, K)))
        qx, rx = _quant_both(orc, x, 1)
        say("gemv repeated M=%d" % M)
        C = fp4.gemm(qx, qw, out_dtype=torch.float32)
        Cref, T = orc.gemm(rx[0], rx[1], rw[0], rw[1], M, 1024, K, 1, tsA=rx[3], tsB=rw[3])
        assert_gemm_close(orc, to_host(C), Cref, T, False, "gemv repeated M=%d" % M)


@pytest.mark.parametrize("M,N,K", [(3, 1024 * 32 + 40, 288), (20, 1024 * 32 + 40, 288), (32, 300 * 32 + 8, 4352)])
def test_nvfp4_decode_many_row_blocks(orc, M, N, K):
    """More 32-row weight blocks than the decode grid holds (grid-stride loop),
    a ragged last block and a ragged K tail.  M <= 8 reduces in one round
    everywhere; larger M in three rounds except in a workgroup's last row
    block, so both reductions run in one launch."""
    import torch
    a = synth.gaussian(81 + M, (M, K))
    b = synth.gaussian(82, (N, K), std=0.02, bernoulli=0.002)
    say("gemv many row blocks M=%d N=%d K=%d" % (M, N, K))
    qa, ra = _quant_both(orc, a, 1)
    qb, rb = _quant_both(orc, b, 1)
    import block_scaled_fp4_03_amd as fp4
    C = fp4.gemm(qa, qb, out_dtype=torch.float32)
    Cref, T = orc.gemm(ra[0], ra[1], rb[0], rb[1], M, N, K, 1, tsA=ra[3], tsB=rb[3])
    assert_gemm_close(orc, to_host(C), Cref, T, False, "gemv many row blocks")


@pytest.mark.parametrize("fmt,M", [(1, 1), (1, 32), (0, 4), (0, 300)])
def test_gemm_k_zero(fmt, M):
    """K == 0: the product is empty and C is all zeros."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    N = 70
    say("gemm K=0 fmt=%d M=%d" % (fmt, M))
    ts = torch.ones(1, dtype=torch.float32, device="cuda") if fmt == 1 else None
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    qa = fp4.Quantized(e, e, ts, fmt, M, 0)
    qb = fp4.Quantized(e, e, ts, fmt, N, 0)
    C = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    fp4.gemm(qa, qb, out=C)
    assert (to_host(C) == 0).all()


@pytest.mark.parametrize("M", [1, 8, 32])
def test_nvfp4_decode_8192_sampled(orc, M):
    """The decode workload: W 8192 x 8192 N(0, 0.02^2) with 0.1% outliers x20
    (NVFP4, pre-quantised), X M x 8192 BF16 N(0,1) quantised on the fly; all
    rows x 48 sampled columns against the oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    w = synth.nvfp4_decode_weight()
    x = synth.nvfp4_decode_act(M)
    say("decode 8192 M=%d" % M)
    qw = fp4.quantize(to_dev(w), 1)
    qx = fp4.quantize(to_dev(x), 1)
    C = to_host(fp4.gemm(qx, qw, out_dtype=torch.bfloat16))
    g = np.random.default_rng(M)
    cols = np.sort(np.concatenate([[0, 8191], g.choice(8192, 46, replace=False)]))
    ts_w = orc.nvfp4_tensor_scale(orc.tensor_amax(w))
    rx = orc.quantize(x, 1)
    rw = orc.quantize(w[cols], 1, tensor_scale=ts_w)
    assert to_host(qw.tensor_scale)[0] == np.float32(ts_w)
    Cref, T = orc.gemm(rx[0], rx[1], rw[0], rw[1], M, cols.size, 8192, 1, tsA=rx[3], tsB=ts_w)
    assert_gemm_close(orc, C[:, cols], Cref, T, True, "decode M=%d" % M)


# ---- grouped (mixture-of-experts) GEMM ----------------------------------------
def _quant_experts(orc, ws, fmt):
    """Quantise each expert on the GPU into one stacked buffer (codes, scales)
    and check each against the oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    E = len(ws)
    N, K = ws[0].shape
    sbytes = fp4.fp4_scale_bytes(fmt, N, K)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, sbytes), dtype=torch.uint8, device="cuda")
    refs = []
    for e, w in enumerate(ws):
        q = fp4.Quantized(codes[e], scales[e], None, fmt, N, K)
        fp4.quantize(to_dev(w), fmt, out=q)
        r = orc.quantize(w, fmt)
        np.testing.assert_array_equal(to_host(codes[e]), r[0])
        np.testing.assert_array_equal(to_host(scales[e]), r[1])
        refs.append(r)
    return codes, scales, refs


# Group sizes that reach every per-group M-tile: last m-tiles of 1-32, 33-64,
# 65-128 rows (light: half the waves idle), 129-160, 161-192, 193-255 rows and
# whole 256-row tiles, with K of one, two and 11.25 stages.
_EVERY_MTILE = [140, 170, 200, 250, 64, 65, 32, 33, 128, 129, 0, 256, 385, 16]


@pytest.mark.parametrize("counts,N,K", [([5, 0, 33, 2], 96, 128), ([300, 1, 0, 257, 17], 160, 544),
                                        ([0, 0, 0], 64, 64), ([600], 300, 2880), ([1, 1, 1, 1, 1, 1, 1, 1], 520, 256),
                                        (_EVERY_MTILE, 520, 2880), (_EVERY_MTILE, 264, 512),
                                        (_EVERY_MTILE, 96, 256)])
@pytest.mark.parametrize("bf16_out", [False, True])
@pytest.mark.parametrize("pregather", [True, False])
def test_grouped_gemm(orc, counts, N, K, bf16_out, pregather):
    import block_scaled_fp4_03_amd as fp4
    import torch
    fmt = 0
    counts = np.array(counts)
    T_rows = max(64, int(counts.max()) if counts.size else 1)
    row_idx, off = synth.moe_routing(counts, tokens=T_rows, seed=int(counts.sum()) + N)
    x = synth.to_bf16_bits(synth.gaussian(80 + N, (T_rows, K)))
    ws = [synth.gaussian(90 + e, (N, K), std=0.02) for e in range(counts.size)]
    say("grouped counts=%s N=%d K=%d pregather=%s" % (counts.tolist(), N, K, pregather))
    qa, ra = _quant_both(orc, x, fmt)
    codes, scales, _ = _quant_experts(orc, ws, fmt)
    total = int(off[-1])
    C = fp4.gemm_grouped(qa, torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda(), codes, scales, N, K,
                         fmt, out_dtype=torch.bfloat16 if bf16_out else torch.float32, pregather=pregather)
    if total == 0:
        assert C.numel() == 0
        return
    Cg = to_host(C)
    B = to_host(codes).reshape(-1)
    sB = to_host(scales).reshape(-1)
    rows = np.repeat(np.arange(total), N)
    cols = np.tile(np.arange(N), total)
    Cref, T = orc.gemm_grouped_sampled(ra[0], ra[1], T_rows, row_idx, off, B, sB, N, K, fmt, rows, cols)
    assert_gemm_close(orc, Cg.reshape(-1), Cref, T, bf16_out, "grouped")


@pytest.mark.parametrize("counts,N,K", [([5, 0, 33, 2], 96, 128), ([300, 1, 0, 257, 17], 160, 544),
                                        (_EVERY_MTILE, 264, 512), ([600], 300, 2880)])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_grouped_gemm_nvfp4(orc, counts, N, K, bf16_out):
    """NVFP4 experts, each quantised on its own (its own tensor scale, tsB[e]),
    against NVFP4 tokens: every output element against the oracle, expert by
    expert with that expert's tensor scale.  Weights of each expert have a
    different spread, so the tensor scales differ."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    fmt = fp4.NVFP4
    counts = np.array(counts)
    E = counts.size
    T_rows = max(64, int(counts.max()))
    row_idx, off = synth.moe_routing(counts, tokens=T_rows, seed=int(counts.sum()) + N + 1)
    x = synth.to_bf16_bits(synth.gaussian(70 + N, (T_rows, K)))
    say("grouped nvfp4 counts=%s N=%d K=%d" % (counts.tolist(), N, K))
    qa, ra = _quant_both(orc, x, fmt)
    assert to_host(qa.tensor_scale)[0] == np.float32(ra[3])
    sbytes = fp4.fp4_scale_bytes(fmt, N, K)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, sbytes), dtype=torch.uint8, device="cuda")
    ts = torch.empty(E, dtype=torch.float32, device="cuda")
    ref_ts = []
    for e in range(E):
        w = synth.gaussian(95 + e, (N, K), std=0.02 * (1 + e), bernoulli=0.001)
        fp4.quantize(to_dev(w), fmt, out=fp4.Quantized(codes[e], scales[e], ts[e:e + 1], fmt, N, K))
        r = orc.quantize(w, fmt)
        np.testing.assert_array_equal(to_host(codes[e]), r[0])
        np.testing.assert_array_equal(to_host(scales[e]), r[1])
        assert to_host(ts[e:e + 1])[0] == np.float32(r[3])
        ref_ts.append(r[3])
    C = fp4.gemm_grouped(qa, torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda(), codes, scales, N, K,
                         fmt, b_tensor_scale=ts, out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    Cg = to_host(C)
    B = to_host(codes).reshape(-1)
    sB = to_host(scales).reshape(-1)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.repeat(np.arange(lo, hi), N)
        cols = np.tile(np.arange(N), hi - lo)
        Cref, T = orc.gemm_grouped_sampled(ra[0], ra[1], T_rows, row_idx, off, B, sB, N, K, fmt, rows, cols,
                                           tsA=ra[3], tsB=ref_ts[e])
        assert_gemm_close(orc, Cg[lo:hi].reshape(-1), Cref, T, bf16_out, "grouped nvfp4 expert %d" % e)


@pytest.mark.parametrize("fmt", [0, 2])
def test_grouped_pregather_bit_equal(orc, fmt):
    """The two MXFP4 grouped paths -- token rows copied into expert order in
    the workspace first, or gathered by the GEMM itself -- return the same bits
    (same products in the same order), also with padding rows past the end
    of the 32-row scale tiles and a token matrix smaller than the routed
    rows."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    counts = np.array([70, 0, 257, 3, 33, 129])
    E, N, K = counts.size, 264, 544
    T_rows = 100
    row_idx, off = synth.moe_routing(counts, tokens=T_rows, seed=11)
    x = synth.to_bf16_bits(synth.gaussian(12, (T_rows, K)))
    qa = fp4.quantize(to_dev(x), fmt)
    sbytes = fp4.fp4_scale_bytes(fmt, N, K)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, sbytes), dtype=torch.uint8, device="cuda")
    ts = torch.empty(E, dtype=torch.float32, device="cuda") if fmt == 1 else None
    for e in range(E):
        w = synth.gaussian(13 + e, (N, K), std=0.02)
        fp4.quantize(to_dev(w), fmt, out=fp4.Quantized(codes[e], scales[e], ts[e:e + 1] if fmt == 1 else None,
                                                       fmt, N, K))
    ri, go = torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda()
    say("grouped pregather vs gather fmt=%d" % fmt)
    for dt in (torch.float32, torch.bfloat16):
        c1 = fp4.gemm_grouped(qa, ri, go, codes, scales, N, K, fmt, b_tensor_scale=ts, out_dtype=dt, pregather=True)
        c0 = fp4.gemm_grouped(qa, ri, go, codes, scales, N, K, fmt, b_tensor_scale=ts, out_dtype=dt, pregather=False)
        assert np.array_equal(to_host(c1).view(np.uint8), to_host(c0).view(np.uint8))


def test_grouped_moe_full_size(orc):
    """The MoE workload: 32 experts (5760 x 2880 MXFP4 weights N(0, 0.02^2)),
    16384 BF16 tokens quantised once, Zipf(1.2) routing with top-4.  Every
    row of each expert with at most 256 rows, a whole 256-row band of each
    larger expert (at a random offset) and the rows of its last, partial
    tile, against one column in each 256-column band, checked against the
    oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    E, N, K, T_rows = 32, 5760, 2880, 16384
    counts = synth.zipf_counts()
    row_idx, off = synth.moe_routing(counts)
    x = synth.mxfp4_moe_act()
    say("grouped moe full size: quantise")
    qa = fp4.quantize(to_dev(x), 0)
    sbytes = fp4.fp4_scale_bytes(0, N, K)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, sbytes), dtype=torch.uint8, device="cuda")
    for e in range(E):
        w = synth.mxfp4_moe_weights(E, N, K, experts=[e])[0]
        fp4.quantize(to_dev(w), 0, out=fp4.Quantized(codes[e], scales[e], None, 0, N, K))
    say("grouped moe full size: gemm")
    C = fp4.gemm_grouped(qa, torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda(), codes, scales, N, K, 0,
                         out_dtype=torch.bfloat16)
    Ch = to_host(C)
    g = np.random.default_rng(5)
    cols = _band_picks(N, 256, 55)
    checked = 0
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        if hi - lo <= 256:
            rs = np.arange(lo, hi)
        else:
            start = lo + int(g.integers(0, hi - lo - 256 + 1))
            tail = np.arange(lo + (hi - lo) // 256 * 256, hi)     # the last, partial tile
            rs = np.union1d(np.arange(start, start + 256), tail)
        w = synth.mxfp4_moe_weights(E, N, K, experts=[e])[0]
        rw = orc.quantize(w[cols], 0)
        rx = orc.quantize(x[row_idx[rs]], 0)
        Cref, T = orc.gemm(rx[0], rx[1], rw[0], rw[1], rs.size, cols.size, K, 0)
        assert_gemm_close(orc, Ch[np.ix_(rs, cols)], Cref, T, True, "moe expert %d" % e)
        checked += rs.size
    assert checked > 2000


@pytest.mark.parametrize("offsets", [[0, 60, 40, 130], [0, -10, 50, 100], [0, 30, 30, 2 ** 31 - 1]])
@pytest.mark.parametrize("with_ws", [False, True])
def test_grouped_malformed_offsets_stay_in_bounds(orc, offsets, with_ws):
    """group_off that decreases, goes negative or runs past total_rows: the
    kernel clamps every group to [0, total_rows], so nothing past C's
    total_rows rows is written.  C and row_idx are allocated with guard rows
    beyond what the call is told, so a wrong clamp would show as a changed
    guard, not as an access outside the allocation.  Rows that only a
    well-formed, clamped group covers equal the oracle's."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    E, total, N, K, T_rows, guard = 3, 100, 64, 64, 64, 300
    x = synth.gaussian(501, (T_rows, K))
    ws = [synth.gaussian(510 + e, (N, K), std=0.05) for e in range(E)]
    qa, ra = _quant_both(orc, x, 0)
    codes, scales, refs = _quant_experts(orc, ws, 0)
    ri = np.random.default_rng(7).integers(0, T_rows, total + guard).astype(np.int32)
    off = np.array(offsets, np.int64).astype(np.int32)
    ri_d, off_d = to_dev(ri), to_dev(off)
    C = torch.full((total + guard, N), 1234.5, dtype=torch.float32, device="cuda")
    nws = fp4.fp4_workspace_size(fp4.OP_GEMM_GROUPED, 0, total, N, K, E) if with_ws else 0
    wsp = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    say("grouped malformed offsets %s workspace %d" % (offsets, nws))
    rc = fp4.fp4_gemm_grouped(qa.codes.data_ptr(), qa.scales.data_ptr(), T_rows, ri_d.data_ptr(), off_d.data_ptr(),
                              E, codes.data_ptr(), scales.data_ptr(), None, None, C.data_ptr(), total, N, K, 0,
                              fp4.F32, wsp.data_ptr() if with_ws else None, nws,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    Ch = to_host(C)
    assert (Ch[total:] == np.float32(1234.5)).all(), "rows past total_rows were written"
    # the clamped groups: [lo, hi) with 0 <= lo <= hi <= total
    cl = [min(max(int(v), 0), total) for v in offsets]
    spans = []
    for e in range(E):
        lo, hi = cl[e], max(cl[e + 1], cl[e])
        spans.append((lo, hi))
    for e, (lo, hi) in enumerate(spans):
        rows = [r for r in range(lo, hi) if all(not (l2 <= r < h2) for j, (l2, h2) in enumerate(spans) if j != e)]
        if not rows:
            continue
        rows = np.array(rows)
        rx = orc.quantize(x[ri[rows]], 0)
        Cref, T = orc.gemm(rx[0], rx[1], refs[e][0], refs[e][1], rows.size, N, K, 0)
        assert_gemm_close(orc, Ch[rows], Cref, T, False, "malformed offsets expert %d" % e)


def test_wrapper_rejects_int64_group_offsets():
    """int64 indices (torch's default from cumsum / argsort) are refused before
    the library is called: read as int32 halves they would make group sizes
    wrap."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    qa = fp4.quantize(x, 0)
    codes = torch.zeros((2, 64, 32), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((2, fp4.fp4_scale_bytes(0, 64, 64)), dtype=torch.uint8, device="cuda")
    ri = torch.arange(10, device="cuda")                       # int64
    off = torch.tensor([0, 4, 10], device="cuda")              # int64
    with pytest.raises(TypeError):
        fp4.gemm_grouped(qa, ri, off.int(), codes, scales, 64, 64, 0)
    with pytest.raises(TypeError):
        fp4.gemm_grouped(qa, ri.int(), off, codes, scales, 64, 64, 0)
    with pytest.raises(ValueError, match="contiguous"):
        fp4.gemm_grouped(qa, torch.arange(20, device="cuda", dtype=torch.int32)[::2], off.int(), codes, scales,
                         64, 64, 0)


def _rne_bf16_of(c32):
    """torch's (CPU) round-to-nearest-even of FP32 values to BF16, as bits."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(c32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("path", ["dense_mx", "dense_nv", "grouped", "grouped_partial"])
def test_bf16_output_is_rne_of_fp32_output(orc, path):
    """The same call with BF16 and with FP32 output forms the same FP32 sums,
    so every BF16 element must be the round-to-nearest-even of the FP32 one,
    bit for bit: this pins each epilogue's BF16 rounding (through LDS in the
    one-tile-per-workgroup kernel, from registers in the persistent ones, on
    their unmasked whole-tile path and their masked partial-tile path)."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    if path in ("dense_mx", "dense_nv"):
        fmt = 0 if path == "dense_mx" else 1
        M, N, K = (520, 512, 1024) if fmt == 0 else (600, 520, 1024)
        say("bf16 rne %s M=%d N=%d K=%d" % (path, M, N, K))
        qa = fp4.quantize(to_dev(synth.gaussian(301 + fmt, (M, K))), fmt)
        qb = fp4.quantize(to_dev(synth.gaussian(311 + fmt, (N, K), std=0.05)), fmt)
        c32 = to_host(fp4.gemm(qa, qb, out_dtype=torch.float32))
        c16 = to_host(fp4.gemm(qa, qb, out_dtype=torch.bfloat16))
    else:
        counts = np.array([512, 3, 260, 0, 256] if path == "grouped" else [40, 300, 1])
        N, K = (512, 1024) if path == "grouped" else (300, 544)
        T_rows = 600
        row_idx, off = synth.moe_routing(counts, tokens=T_rows, seed=int(counts.sum()) + N)
        say("bf16 rne %s counts=%s N=%d K=%d" % (path, counts.tolist(), N, K))
        qa = fp4.quantize(to_dev(synth.to_bf16_bits(synth.gaussian(321, (T_rows, K)))), 0)
        ws = [synth.gaussian(330 + e, (N, K), std=0.02) for e in range(counts.size)]
        codes, scales, _ = _quant_experts(orc, ws, 0)
        ri, go = torch.from_numpy(row_idx).cuda(), torch.from_numpy(off).cuda()
        c32 = to_host(fp4.gemm_grouped(qa, ri, go, codes, scales, N, K, 0, out_dtype=torch.float32))
        c16 = to_host(fp4.gemm_grouped(qa, ri, go, codes, scales, N, K, 0, out_dtype=torch.bfloat16))
    assert np.isfinite(c32).all() and np.abs(c32).max() > 0
    np.testing.assert_array_equal(c16.view(np.uint16), _rne_bf16_of(c32))


def test_nvfp4_persistent_tail_runs_as_half_tiles(orc):
    """4096 x 4352 x 256 NVFP4 is 16 x 17 = 272 tiles: on 256 resident
    workgroups the last 16 tiles (the last tile group: rows 3072-4095,
    columns 3328-4351) run as 128-row halves, each by a workgroup whose other
    four waves only copy.  Every element of those 1024 rows, and rows picked
    from every other 256-row band, against the oracle."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    M, N, K = 4096, 4352, 256
    a = synth.gaussian(601, (M, K))
    w = synth.gaussian(602, (N, K), std=0.05)
    say("nvfp4 persistent tail halves M=%d N=%d K=%d" % (M, N, K))
    qa, ra_full = _quant_both(orc, a, 1)
    qw, rw = _quant_both(orc, w, 1)
    C = to_host(fp4.gemm(qa, qw, out_dtype=torch.bfloat16))
    rows = np.concatenate([_band_picks(3072, 256, 6), np.arange(3072, 4096)])
    rr = orc.quantize(a[rows], 1, tensor_scale=ra_full[3])   # the picked rows, under the whole operand's s_t
    Cref, T = orc.gemm(rr[0], rr[1], rw[0], rw[1], rows.size, N, K, 1, tsA=ra_full[3], tsB=rw[3])
    assert_gemm_close(orc, C[rows], Cref, T, True, "nvfp4 tail half tiles")
