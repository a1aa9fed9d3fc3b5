"""Oracle number-format codecs pinned against what the pages print and against
library routines (torch's float8_e4m3fn and bfloat16 casts, numpy frexp).

Pages: Ultralytics glossary "FP4" (E2M1 value set, nearest-grid rounding);
NVFP4 video transcript (E4M3 block scale); "Rubin FP4 GEMM deep dive" §3.1
(E8M0 power-of-two scale)."""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_grid():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    return np.array(vals)


def test_e2m1_value_set_matches_printed(orc):
    grid = _golden_grid()
    dec = np.array([orc.e2m1_value(c) for c in range(16)])
    np.testing.assert_array_equal(dec[:8], grid)
    np.testing.assert_array_equal(dec[8:], -grid)
    assert len(set(dec.tolist())) == 15  # +0 and -0 coincide
    assert np.all(np.isfinite(dec))  # no inf/NaN codes exist
    assert np.signbit(dec[8]) and not np.signbit(dec[0])


def _f32_from_bits(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def test_e2m1_rounding_is_nearest_grid_point(orc):
    """Away from ties, the code is the page's argmin over the printed grid."""
    grid = _golden_grid()
    hi = np.float32(8.0).view(np.uint32)
    bits = np.arange(0, int(hi), 61, dtype=np.uint32)
    y = _f32_from_bits(bits)
    got = orc.e2m1_encode_mag(y)
    for lo in range(0, y.size, 1 << 20):
        yy = y[lo:lo + (1 << 20)].astype(np.float64)
        d = np.abs(yy[:, None] - grid[None, :])
        ds = np.sort(d, axis=1)
        tie = ds[:, 0] == ds[:, 1]
        ref = np.argmin(d, axis=1)
        np.testing.assert_array_equal(got[lo:lo + (1 << 20)][~tie], ref[~tie])


def test_e2m1_ties_go_to_even_code(orc):
    # Each midpoint between neighbouring grid values; round-to-nearest-even
    # picks the neighbour whose code has mantissa bit 0.
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    expect = np.array([0, 2, 2, 4, 4, 6, 6], np.uint8)
    np.testing.assert_array_equal(orc.e2m1_encode_mag(mids), expect)
    # One ulp either side goes to the nearer neighbour.
    below = np.nextafter(mids, np.float32(0))
    above = np.nextafter(mids, np.float32(np.inf))
    np.testing.assert_array_equal(orc.e2m1_encode_mag(below), [0, 1, 2, 3, 4, 5, 6])
    np.testing.assert_array_equal(orc.e2m1_encode_mag(above), [1, 2, 3, 4, 5, 6, 7])


def test_e2m1_saturates_at_six(orc):
    y = np.array([6.0, 6.5, 100.0, 3.0e38, np.inf], np.float32)
    np.testing.assert_array_equal(orc.e2m1_encode_mag(y), [7] * 5)


def test_e4m3_decode_matches_torch(orc):
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([orc.e4m3_value(c) for c in codes])
    np.testing.assert_array_equal(mine, t)
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast(orc):
    """Round-to-nearest-even into E4M3 against torch's float8_e4m3fn cast, on
    a stride through every FP32 in [0, 448] plus every representable value,
    every midpoint, and one ulp either side of each midpoint."""
    top = np.float32(448.0).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 1009, dtype=np.uint32)
    vals = np.array([orc.e4m3_value(c) for c in range(127)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    r = np.concatenate([_f32_from_bits(bits), vals.astype(np.float32), mids,
                        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    mine = orc.e4m3_encode(r)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_e4m3_encode_saturates(orc):
    r = np.array([448.0, 449.0, 463.9, 464.0, 1e6, 3.0e38, np.inf], np.float32)
    np.testing.assert_array_equal(orc.e4m3_encode(r), [0x7E] * r.size)


def test_bf16_rounding_matches_torch(orc):
    g = np.random.default_rng(7)
    bits = g.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    f = _f32_from_bits(bits)
    f = f[np.isfinite(f)]
    # exact ties: low 16 bits == 0x8000
    ties = _f32_from_bits((bits[:4096] & 0xFFFF0000) | 0x8000)
    f = np.concatenate([f, ties[np.isfinite(ties)], np.array([3.4e38, -3.4e38, 3.3895e38], np.float32)])
    mine = orc.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def _amax_sample():
    # every exponent, including subnormals, with a spread of mantissas
    bits = np.arange(1, 0x7F7FFFFF, 4099, dtype=np.uint64).astype(np.uint32)
    a = _f32_from_bits(bits)
    six = np.ldexp(np.float32(6.0), np.arange(-127, 126)).astype(np.float32)
    six = six[(six > 0) & np.isfinite(six)]
    return np.concatenate([np.zeros(1, np.float32), a, six])


def test_mx_exponent_invariants(orc):
    """Power of two, never clips (amax <= 6*2^e), and minimal."""
    a = _amax_sample()
    e = orc.mx_exponent(a).astype(np.int64)
    assert e.min() >= -127 and e.max() <= 127
    a64 = a.astype(np.float64)
    assert np.all(a64 <= 6.0 * np.ldexp(1.0, e))
    assert np.all((e == -127) | (a64 > 6.0 * np.ldexp(1.0, e - 1)))
    # amax exactly 6 * 2^j gives e = j: the block max lands on 6.
    j = np.arange(-120, 126)
    six = np.ldexp(6.0, j).astype(np.float32)
    np.testing.assert_array_equal(orc.mx_exponent(six), j)
    # The transcript's example: an ideal scale of 70 is not a power of two;
    # the block max 420 = 6*70 gets 2^7 = 128 under this rule.
    assert orc.mx_exponent(np.array([420.0], np.float32))[0] == 7


def test_mx_exponent_ocp_rule(orc):
    a = _amax_sample()
    a = a[a > 0]
    e = orc.mx_exponent(a, ocp=True).astype(np.int64)
    _, ex = np.frexp(a.astype(np.float64))
    ref = np.clip(ex - 1 - 2, -127, 127)
    np.testing.assert_array_equal(e, ref)
    assert orc.mx_exponent(np.zeros(1, np.float32), ocp=True)[0] == -127


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("rows,K", [(1, 32), (16, 512), (17, 96), (33, 2880), (40, 1024)])
def test_scale_layout_is_a_bijection(orc, fmt, rows, K):
    bs = orc.block_size(fmt)
    if K % bs:
        pytest.skip("shape not defined for this block size")
    KB = K // bs
    total = orc.scale_bytes(fmt, rows, K)
    assert total == ((rows + 31) // 32) * ((K + 255) // 256) * (512 if fmt == 1 else 256)
    offs = np.array([orc.scale_offset(fmt, rows, K, r, b) for r in range(rows) for b in range(KB)])
    assert offs.min() >= 0 and offs.max() < total
    assert np.unique(offs).size == offs.size
