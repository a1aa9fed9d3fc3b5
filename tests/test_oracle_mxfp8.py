"""The oracle's MXFP8 operand and mixed MXFP8 x MXFP4 product, pinned to what
the pages and library routines fix.

"Rubin FP4 GEMM deep dive" §3.4: weights and activations can take different
precisions, activations kept in FP8 while the weights go to FP4; §3.1 names
MXFP8 beside MXFP4 among the microscaling formats (one power-of-two E8M0 scale
per block).  Readings (E4M3 elements, 32-blocks, the MXFP4 scale rules with
448 in place of 6) are the oracle's; these tests pin it against:

  * the scale rules' defining invariants (power of two, no clipping,
    minimality; the OCP exponent from frexp);
  * torch's float8_e4m3fn cast (round to nearest even) of the scaled values,
    for every element, and its decode for dequantisation;
  * closed forms of the product on hand-built operands, and numpy's FP64
    matmul of operands decoded through torch on small shapes.
"""
import numpy as np
import pytest
import torch

import synth


def _amax_sample():
    g = synth.rng(7)
    bits = g.integers(0, 0x7F800000, 200000, dtype=np.int64).astype(np.uint32)
    a = bits.view(np.float32)
    j = np.arange(-126, 120)
    edge = np.concatenate([np.ldexp(np.float32(448.0), j), np.ldexp(np.float32(1.0), j),
                           np.nextafter(np.ldexp(np.float32(448.0), j), np.float32(np.inf))])
    return np.concatenate([np.zeros(1, np.float32), a, edge.astype(np.float32)])


def test_mx8_exponent_invariants(orc):
    """Smallest e with amax <= 448 * 2^e: no element clips, and e is minimal."""
    a = _amax_sample()
    e = orc.mx8_exponent(a).astype(np.int64)
    assert e.min() >= -127 and e.max() <= 127
    a64 = a.astype(np.float64)
    assert np.all(a64 <= 448.0 * np.ldexp(1.0, e))
    assert np.all((e == -127) | (a64 > 448.0 * np.ldexp(1.0, e - 1)))
    # amax exactly 448 * 2^j lands on E4M3's largest value: e = j.
    j = np.arange(-100, 100)
    np.testing.assert_array_equal(orc.mx8_exponent(np.ldexp(np.float32(448.0), j).astype(np.float32)), j)


def test_mx8_exponent_ocp_rule(orc):
    a = _amax_sample()
    a = a[a > 0]
    e = orc.mx8_exponent(a, ocp=True).astype(np.int64)
    _, ex = np.frexp(a.astype(np.float64))
    np.testing.assert_array_equal(e, np.clip(ex - 1 - 8, -127, 127))
    assert orc.mx8_exponent(np.zeros(1, np.float32), ocp=True)[0] == -127


def _torch_codes(x, fmt, orc):
    """MXFP8 codes and scale exponents built from torch's E4M3 cast: per
    32-block e from the (separately pinned) exponent rule, y = x * 2^-e exact
    in FP32, saturated to +-448 (the OCP rule's elements may exceed it), then
    float8_e4m3fn round to nearest even."""
    rows, K = x.shape
    xb = x.reshape(rows, K // 32, 32)
    amax = np.abs(xb).max(axis=2)
    e = orc.mx8_exponent(amax, ocp=(fmt == orc.FMT_MXFP8_OCP)).astype(np.int64)
    y = np.ldexp(xb, -e[:, :, None]).astype(np.float32)
    y = np.clip(y, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y.reshape(rows, K)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, e


def _mixed_data(seed, rows, K):
    """N(0,1) with outliers, some tiny values (E4M3 subnormals after scaling),
    exact ties between E4M3 neighbours, zeros and -0."""
    x = synth.gaussian(seed, (rows, K), bernoulli=0.01)
    g = synth.rng(seed + 1)
    x[:, 5::32] *= np.float32(1e-3)
    # ties: (1 + m/8 + 1/16) * 2^k lies halfway between two E4M3 values; the
    # block holds a 448 * 2^k' maximum so that the scale is known exactly.
    if rows > 2:
        x[2] = 0.0
        x[2, ::32] = 448.0
        m = g.integers(0, 7, K).astype(np.float32)
        x[2, 1::2] = ((1.0 + m / 8.0 + 1.0 / 16.0) * np.ldexp(1.0, g.integers(-6, 8, K)))[1::2]
    if rows > 3:
        x[3, :32] = 0.0
        x[3, 32:64] = -0.0
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", [3, 4])
@pytest.mark.parametrize("rows,K", [(1, 32), (5, 96), (33, 512)])
def test_mxfp8_codes_equal_torch_e4m3_cast(orc, fmt, rows, K):
    x = _mixed_data(rows + K, rows, K)
    codes, scales, canon, ts = orc.quantize(x, fmt)
    assert codes.shape == (rows, K) and ts == 1.0
    want, e = _torch_codes(x, fmt, orc)
    np.testing.assert_array_equal(canon, (e + 127).astype(np.uint8))
    np.testing.assert_array_equal(codes, want)
    # tiled scale bytes sit where the shared layout puts them
    for r in range(rows):
        for b in range(K // 32):
            assert scales[orc.scale_offset(fmt, rows, K, r, b)] == canon[r, b]


def test_mxfp8_negative_zero_and_zero_block(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, :32] = -0.0
    x[1, 32] = 1.0
    codes, _, canon, _ = orc.quantize(x, orc.FMT_MXFP8)
    assert canon[0, 0] == 0 and canon[0, 1] == 0 and canon[1, 0] == 0
    assert np.all(codes[0] == 0)
    assert np.all(codes[1, :32] == 0x80)


def test_mxfp8_stochastic_rounding_rejected(orc):
    with pytest.raises(ValueError):
        orc.quantize(np.ones((1, 32), np.float32), orc.FMT_MXFP8, sr_seed=1)


@pytest.mark.parametrize("fmt", [3, 4])
def test_mxfp8_dequantize_is_torch_e4m3_value_times_scale(orc, fmt):
    rows, K = 9, 256
    x = _mixed_data(41, rows, K)
    codes, scales, canon, _ = orc.quantize(x, fmt)
    e4 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    want = e4 * np.repeat(np.ldexp(1.0, canon.astype(np.int64) - 127), 32, axis=1)
    got = orc.dequantize(codes, scales, 1.0, fmt, rows, K)
    np.testing.assert_array_equal(got.astype(np.float64), want)
    bf = orc.dequantize(codes, scales, 1.0, fmt, rows, K, out_bf16=True)
    np.testing.assert_array_equal(bf, orc.f32_to_bf16_bits(want.astype(np.float32)))


def _scales_const(orc, fmt, rows, K, byte):
    s = np.zeros(orc.scale_bytes(fmt, rows, K), np.uint8)
    for r in range(rows):
        for b in range(K // 32):
            s[orc.scale_offset(fmt, rows, K, r, b)] = byte
    return s


def _pack4(c):
    c = np.asarray(c, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def test_mixed_gemm_closed_forms(orc):
    M, N, K = 3, 5, 256
    F8, F4 = orc.FMT_MXFP8, orc.FMT_MXFP4
    A = np.full((M, K), 0x7E, np.uint8)              # 448
    B = _pack4(np.full((N, K), 7))                   # 6
    sA = _scales_const(orc, F8, M, K, 127)
    sB = _scales_const(orc, F4, N, K, 127)
    C, T = orc.gemm_mixed(A, sA, F8, B, sB, F4, M, N, K)
    np.testing.assert_array_equal(C, np.full((M, N), 448.0 * 6.0 * K))
    np.testing.assert_array_equal(T, C)
    # alternating signs of A along K cancel exactly
    alt = np.tile(np.array([0x7E, 0xFE], np.uint8), (M, K // 2))
    C2, T2 = orc.gemm_mixed(alt, sA, F8, B, sB, F4, M, N, K)
    np.testing.assert_array_equal(C2, 0.0)
    np.testing.assert_array_equal(T2, 448.0 * 6.0 * K)
    # one-hot: A[1, 70] = 0x3B (1.375) at 2^3, B[4, 70] = -4 (code 14) at 2^-2
    a1 = np.zeros((M, K), np.uint8)
    b1 = np.zeros((N, K), np.uint8)
    a1[1, 70] = 0x3B
    b1[4, 70] = 14
    C3, _ = orc.gemm_mixed(a1, _scales_const(orc, F8, M, K, 130), F8, _pack4(b1),
                           _scales_const(orc, F4, N, K, 125), F4, M, N, K)
    ref = np.zeros((M, N))
    ref[1, 4] = 1.375 * -4.0 * 8.0 * 0.25
    np.testing.assert_array_equal(C3, ref)


@pytest.mark.parametrize("fmtA", [3, 4])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 7, 64), (16, 9, 256)])
def test_mixed_gemm_equals_numpy_of_torch_decoded(orc, fmtA, M, N, K):
    x = _mixed_data(60 + M, M, K)
    w = synth.gaussian(70 + N, (N, K), std=0.05, bernoulli=0.01)
    A, sA, cA, _ = orc.quantize(x, fmtA)
    B, sB, _, _ = orc.quantize(w, orc.FMT_MXFP4)
    C, T = orc.gemm_mixed(A, sA, fmtA, B, sB, orc.FMT_MXFP4, M, N, K)
    dA = torch.from_numpy(A).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dA = dA * np.repeat(np.ldexp(1.0, cA.astype(np.int64) - 127), 32, axis=1)
    dB = orc.dequantize(B, sB, 1.0, orc.FMT_MXFP4, N, K).astype(np.float64)   # exact
    np.testing.assert_allclose(C, dA @ dB.T, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(T, np.abs(dA) @ np.abs(dB).T, rtol=1e-12, atol=1e-300)
    rows = np.array([0, M - 1, M // 2])
    cols = np.array([N - 1, 0, N // 2])
    Cs, Ts = orc.gemm_mixed_sampled(A, sA, fmtA, B, sB, orc.FMT_MXFP4, M, N, K, rows, cols)
    np.testing.assert_array_equal(Cs, C[rows, cols])
    np.testing.assert_array_equal(Ts, T[rows, cols])
