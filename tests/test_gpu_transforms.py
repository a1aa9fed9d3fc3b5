"""The training-recipe steps before quantisation (NVFP4 video transcript):
the random Hadamard transform (fp4_hadamard16) and 2-D 16 x 16 NVFP4 weight
scaling (fp4_quantize_ex with FP4_Q_2D), against the oracle bit for bit."""
import numpy as np
import pytest

import synth
from gpu_helpers import say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,K", [(1, 16), (3, 48), (37, 528), (300, 1024), (5000, 160)])
@pytest.mark.parametrize("bf16_in", [False, True])
def test_hadamard_fp32_out_bit_exact(orc, rows, K, bf16_in):
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = synth.gaussian(rows + K, (rows, K), every=37)
    if bf16_in:
        x = synth.to_bf16_bits(x)
    say("hadamard16 rows=%d K=%d bf16_in=%s" % (rows, K, bf16_in))
    y = fp4.hadamard16(to_dev(x), seed=rows * 7 + K, out_dtype=torch.float32)
    np.testing.assert_array_equal(to_host(y), orc.rht16(x, rows * 7 + K))


def test_hadamard_bf16_out_and_in_place(orc):
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = synth.to_bf16_bits(synth.gaussian(7, (64, 2048)))
    say("hadamard16 bf16 out, in place")
    ref32 = orc.rht16(x, 99)
    ref16 = orc.f32_to_bf16_bits(ref32)
    xd = to_dev(x)
    y = fp4.hadamard16(xd, seed=99)                        # BF16 -> BF16
    np.testing.assert_array_equal(to_host(y), ref16)
    fp4.hadamard16(xd, seed=99, out=xd)                     # in place
    np.testing.assert_array_equal(to_host(xd), ref16)
    x32 = to_dev(synth.gaussian(8, (64, 2048)))
    fp4.hadamard16(x32, seed=5, out=x32)
    np.testing.assert_array_equal(to_host(x32), orc.rht16(synth.gaussian(8, (64, 2048)), 5))


def test_hadamard_full_size_8192(orc):
    """The Hadamard workload the benchmark times: 8192 x 8192 BF16 N(0, 1)
    through the BF16 -> BF16 launch, one of its seeds: bit-exact."""
    import block_scaled_fp4_03_amd as fp4
    x = synth.to_bf16_bits(synth.gaussian(82, (8192, 8192)))
    say("hadamard16 8192^2 bf16 -> bf16 seed 3")
    y = fp4.hadamard16(to_dev(x), seed=3)
    np.testing.assert_array_equal(to_host(y), orc.f32_to_bf16_bits(orc.rht16(x, 3)))


@pytest.mark.parametrize("fmt", [0, 1])
def test_hadamard_then_quantise(orc, fmt):
    """Transform then quantise, as the recipe orders it: bit-exact."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = synth.gaussian(9, (128, 1024))
    x[:, ::16] *= np.float32(30.0)
    say("hadamard16 + quantise fmt=%d" % fmt)
    y = fp4.hadamard16(to_dev(x), seed=3, out_dtype=torch.float32)
    q = fp4.quantize(y, fmt)
    c, s, _, ts = orc.quantize(orc.rht16(x, 3), fmt)
    np.testing.assert_array_equal(to_host(q.codes), c)
    np.testing.assert_array_equal(to_host(q.scales), s)


@pytest.mark.parametrize("rows,K", [(16, 64), (48, 1024), (40, 96), (300, 2880), (33, 528)])
@pytest.mark.parametrize("bf16", [False, True])
def test_2d_scales_bit_exact(orc, rows, K, bf16):
    import block_scaled_fp4_03_amd as fp4
    x = synth.gaussian(rows * 3 + K, (rows, K), std=0.02, bernoulli=0.01)
    if bf16:
        x = synth.to_bf16_bits(x)
    say("quantize 2d rows=%d K=%d bf16=%s" % (rows, K, bf16))
    q = fp4.quantize(to_dev(x), fp4.NVFP4, two_d=True)
    c, s, _, ts = orc.quantize(x, orc.FMT_NVFP4, two_d=True)
    np.testing.assert_array_equal(to_host(q.codes), c)
    np.testing.assert_array_equal(to_host(q.scales), s)
    assert to_host(q.tensor_scale)[0] == np.float32(ts)


def test_2d_with_sr_and_given_scale(orc):
    import block_scaled_fp4_03_amd as fp4
    import torch
    x = synth.gaussian(12, (80, 512))
    say("quantize 2d + sr + given ts")
    ts = torch.tensor([0.004], dtype=torch.float32, device="cuda")
    q = fp4.quantize(to_dev(x), fp4.NVFP4, tensor_scale=ts, two_d=True, sr_seed=77)
    c, s, _, _ = orc.quantize(x, orc.FMT_NVFP4, tensor_scale=0.004, two_d=True, sr_seed=77)
    np.testing.assert_array_equal(to_host(q.codes), c)
    np.testing.assert_array_equal(to_host(q.scales), s)


def test_2d_w_and_wt_dequantise_to_transposes(orc):
    """The point of 2-D scaling, on the GPU: W (14336 x 4096 rows cut to 1024
    x 512 here) and W^T dequantise to exact transposes of each other."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    w = synth.gaussian(13, (1024, 512), std=0.02, bernoulli=0.001)
    say("quantize 2d W vs W^T")
    wd = to_dev(w)
    q = fp4.quantize(wd, fp4.NVFP4, two_d=True)
    qt = fp4.quantize(wd.t().contiguous(), fp4.NVFP4, two_d=True)
    d = fp4.dequantize(q)
    dt = fp4.dequantize(qt)
    assert torch.equal(q.tensor_scale, qt.tensor_scale)
    assert torch.equal(d, dt.t())
