"""GPU quantiser and dequantiser parity: codes, tiled scale bytes (padding
included) and the NVFP4 tensor scale must equal the oracle's bit for bit."""
import numpy as np
import pytest

import synth
from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

SHAPES = [(1, 32), (16, 512), (17, 96), (33, 2880), (64, 4096), (3, 544), (40, 1056)]


def _special(rows, K, seed):
    """Edge values: zeros, -0, grid midpoints at several scales, subnormals,
    huge magnitudes, one all-zero row and a row of one repeated value."""
    g = synth.rng(seed)
    x = synth.gaussian(seed, (rows, K), every=7)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    n = x.size
    sel = g.random(n) < 0.2
    e = g.integers(-20, 20, n)
    x.reshape(-1)[sel] = (mids[g.integers(0, 8, n)] * np.ldexp(np.float32(1), e))[sel].astype(np.float32)
    x.reshape(-1)[g.random(n) < 0.02] = -0.0
    x.reshape(-1)[g.random(n) < 0.01] = np.float32(1e-40) * g.integers(1, 100, n)[0]
    if rows > 2:
        x[1] = 0.0
        x[2] = np.float32(3.0e38) * (g.random(K) < 0.1) + g.standard_normal(K).astype(np.float32)
    if rows > 3:
        x[3] = np.float32(0.7)
    return x


def _run(orc, fmt, x, ts=None):
    import block_scaled_fp4_03_amd as fp4
    import torch
    rows, K = x.shape
    codes, scales, canon, ts_ref = orc.quantize(x, fmt, tensor_scale=ts)
    xd = to_dev(x)
    say("quantize fmt=%d shape=%s dtype=%s ts=%s" % (fmt, x.shape, x.dtype, ts))
    tsd = None if ts is None else torch.tensor([ts], dtype=torch.float32, device="cuda")
    q = fp4.quantize(xd, fmt, tensor_scale=tsd)
    np.testing.assert_array_equal(to_host(q.codes), codes)
    np.testing.assert_array_equal(to_host(q.scales), scales)
    if fmt == 1:
        assert to_host(q.tensor_scale)[0] == np.float32(ts_ref)
    return q, (codes, scales, ts_ref)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("rows,K", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_bit_exact(orc, fmt, rows, K, bf16):
    x = synth.gaussian(100 + rows + K, (rows, K), every=97, std=0.5)
    if bf16:
        x = synth.to_bf16_bits(x)
    _run(orc, fmt, x)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("rows,K", [(16, 512), (33, 2880)])
def test_quantize_edge_values_bit_exact(orc, fmt, rows, K):
    _run(orc, fmt, _special(rows, K, 7 + fmt))


@pytest.mark.parametrize("ts", [1.0, 0.001, 3.5e-3, 1.1754944e-38, 1e10])
def test_nvfp4_given_tensor_scale(orc, ts):
    x = synth.row_scaled_gaussian(9, 20, 256)
    x[0, :5] = [1e-30, -1e-20, 5e6, -3e3, 0.0]
    _run(orc, 1, x, ts=ts)


def test_nvfp4_all_zero_tensor(orc):
    q, (codes, scales, ts) = _run(orc, 1, np.zeros((5, 64), np.float32))
    assert ts == 1.0


@pytest.mark.parametrize("rows,K,bf16", [(8, 8192, True), (32, 2048, False), (32, 2064, False), (1, 16, True)])
def test_nvfp4_single_launch_threshold(orc, rows, K, bf16):
    """Inputs of at most 256 KB take the one-launch quantiser (each workgroup
    reduces the whole maximum), larger ones the two-launch path: (32, 2048)
    FP32 is exactly 256 KB, (32, 2064) FP32 one block more.  The maximum sits
    in the last element, so a workgroup that skipped any part would get s_t
    wrong."""
    x = synth.gaussian(23 + rows, (rows, K))
    x[-1, -1] = 777.0
    if bf16:
        x = synth.to_bf16_bits(x)
    _run(orc, 1, x)


def test_nvfp4_tensor_scale_on_large_tensor(orc):
    # many workgroups contribute to the amax; the maximum sits in the last row
    x = synth.gaussian(21, (4096, 1024), every=4099)
    x[-1, -1] = 1234.5
    _run(orc, 1, x)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_dequantize_matches_oracle(orc, fmt, bf16_out):
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = _special(33, 2880, 40 + fmt)
    q, (codes, scales, ts) = _run(orc, fmt, x)
    say("dequantize fmt=%d bf16=%s" % (fmt, bf16_out))
    out = fp4.dequantize(q, out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    ref = orc.dequantize(codes, scales, ts, fmt, 33, 2880, out_bf16=bf16_out)
    got = to_host(out)
    np.testing.assert_array_equal(got.view(np.uint32 if not bf16_out else np.uint16),
                                  ref.view(np.uint32 if not bf16_out else np.uint16))


def test_full_size_operands_bit_exact(orc):
    """The 8192 x 8192 MXFP4 operand (0.2% outliers) and the 14336 x 4096 NVFP4
    weight, compared in full."""
    a, _ = synth.mxfp4_8192()
    _run(orc, 0, a)
    _, w = synth.nvfp4_mlp()
    _run(orc, 1, w)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_large_bf16_multi_item_path(orc, fmt):
    """BF16 inputs large enough (at least 32768 row slices of 512 values) for
    the quantisers to give each wave four slices: 4100 x 4000 (padding rows
    and a ragged last slice), with edge values; bit-exact, all formats."""
    x = synth.to_bf16_bits(_special(4100, 4000, 97 + fmt))
    _run(orc, fmt, x)
