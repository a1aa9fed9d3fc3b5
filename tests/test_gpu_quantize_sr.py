"""GPU stochastic-rounding quantiser (fp4_quantize_sr) against the oracle:
codes, tiled scale bytes and the NVFP4 tensor scale equal bit for bit for the
same seed (both sides draw the element words from Philox4x64-10 by the
element's index), and the scales equal the deterministic quantiser's."""
import numpy as np
import pytest

import synth
from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu

SHAPES = [(1, 32), (17, 96), (33, 2880), (64, 4096), (3, 544), (300, 1056)]


def _run(orc, fmt, x, seed, ts=None):
    import block_scaled_fp4_03_amd as fp4
    import torch
    say("quantize_sr fmt=%d shape=%s dtype=%s seed=%d ts=%s" % (fmt, x.shape, x.dtype, seed, ts))
    codes, scales, _, ts_ref = orc.quantize(x, fmt, tensor_scale=ts, sr_seed=seed)
    tsd = None if ts is None else torch.tensor([ts], dtype=torch.float32, device="cuda")
    q = fp4.quantize(to_dev(x), fmt, tensor_scale=tsd, sr_seed=seed)
    np.testing.assert_array_equal(to_host(q.codes), codes)
    np.testing.assert_array_equal(to_host(q.scales), scales)
    if fmt == fp4.NVFP4:
        assert to_host(q.tensor_scale)[0] == np.float32(ts_ref)
    return q


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("rows,K", SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
def test_sr_bit_exact(orc, fmt, rows, K, bf16):
    x = synth.gaussian(rows * 31 + K, (rows, K), every=101)
    if bf16:
        x = synth.to_bf16_bits(x)
    _run(orc, fmt, x, seed=rows * 1000003 + K)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_sr_edge_values(orc, fmt):
    """Grid points at several scales (no randomness), midpoints, values far
    below the block maximum, zeros and -0, a saturating row."""
    g = synth.rng(77)
    rows, K = 12, 512
    x = synth.gaussian(77, (rows, K))
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x[0] = grid[g.integers(0, 8, K)] * np.float32(2.0) ** g.integers(-3, 3)
    x[1] = (grid[g.integers(0, 7, K)] + grid[g.integers(1, 8, K)]) / 2
    x[2, :] = 0.0
    x[3, :] = -0.0
    x[4, ::2] *= np.float32(1e-7)
    x[5] = np.float32(1e30) * (g.random(K) < 0.05)
    _run(orc, fmt, x.astype(np.float32), seed=2 ** 63 + 12345)


def test_sr_given_tensor_scale(orc):
    x = synth.to_bf16_bits(synth.gaussian(78, (64, 1024)))
    _run(orc, 1, x, seed=9, ts=0.0011)


def test_sr_seeds(orc):
    """Same seed, same bits; another seed changes codes but never scales; the
    scales always equal the deterministic quantiser's."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = to_dev(synth.gaussian(79, (256, 2048)))
    say("quantize_sr seeds")
    a = fp4.quantize(x, fp4.NVFP4, sr_seed=1)
    b = fp4.quantize(x, fp4.NVFP4, sr_seed=1)
    c = fp4.quantize(x, fp4.NVFP4, sr_seed=2)
    d = fp4.quantize(x, fp4.NVFP4)
    assert torch.equal(a.codes, b.codes) and not torch.equal(a.codes, c.codes)
    assert torch.equal(a.scales, c.scales) and torch.equal(a.scales, d.scales)
    assert torch.equal(a.tensor_scale, d.tensor_scale)


def test_sr_gradient_sized(orc):
    """A 4096 x 4096 BF16 tensor (the size of the MLP activation) with outliers,
    NVFP4, computed tensor scale (two-launch path): bit-exact."""
    x = synth.to_bf16_bits(synth.gaussian(80, (4096, 4096), std=1e-3, bernoulli=0.001))
    _run(orc, 1, x, seed=0xC0FFEE)


def test_sr_full_size_8192(orc):
    """The stochastic-rounding workload the benchmark times: 8192 x 8192 BF16,
    N(0, 1e-3^2) with 0.1% outliers x20, NVFP4 with its own tensor scale,
    seed 1, through the same two-launch path: bit-exact."""
    x = synth.to_bf16_bits(synth.gaussian(81, (8192, 8192), std=1e-3, bernoulli=0.001))
    _run(orc, 1, x, seed=1)
