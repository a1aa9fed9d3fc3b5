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


@pytest.mark.parametrize("rows,K,bf16", [(32, 8192, True), (64, 4096, False), (65, 4096, False), (33, 2064, False),
                                          (100, 4992, True)])
def test_nvfp4_one_launch_grid_path(orc, rows, K, bf16):
    """Inputs above 256 KB and at most 1 MB take the one-launch path whose
    workgroups exchange the maximum through the workspace: (32, 8192) BF16 is
    a 32-row decode activation (512 KB), (64, 4096) FP32 exactly 1 MB, (65,
    4096) FP32 one row more (two launches), (100, 4992) BF16 ragged in both
    directions.  Three calls in a row share one workspace, with the maximum
    in a different place each time: each call must leave the workspace's
    words zero for the next, so every s_t equals the oracle's."""
    import block_scaled_fp4_03_amd as fp4
    import torch
    ws = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, rows, 0, K)
    assert ws is not None and ws.numel() == 16
    for i, (r, k, big) in enumerate([(-1, -1, 777.0), (0, 0, 12.5), (rows // 2, K // 3, -3.0e4)]):
        x = synth.gaussian(31 + rows + i, (rows, K))
        x[r, k] = big
        if bf16:
            x = synth.to_bf16_bits(x)
        say("nvfp4 grid path rows=%d K=%d bf16=%s call %d" % (rows, K, bf16, i))
        q = fp4.quantize(to_dev(x), fp4.NVFP4, ws=ws)
        codes, scales, _, ts = orc.quantize(x, 1)
        assert to_host(q.tensor_scale)[0] == np.float32(ts)
        np.testing.assert_array_equal(to_host(q.scales), scales)
        np.testing.assert_array_equal(to_host(q.codes), codes)
        assert (to_host(ws) == 0).all(), "workspace words left non-zero"


@pytest.mark.parametrize("rows,K,bf16", [(32, 8192, True), (64, 4096, False)])
def test_nvfp4_grid_path_wait_cut_short(orc, monkeypatch, rows, K, bf16):
    """The one-launch path's wait for the other workgroups, cut to one sleep
    from the host (FP4_TEST_NV_GRID_SPIN): workgroups that stop waiting reduce
    the whole maximum themselves, the others read the exchanged one.  Either
    way every bit equals the oracle's, and the workspace ends zero."""
    import block_scaled_fp4_03_amd as fp4
    monkeypatch.setenv("FP4_TEST_NV_GRID_SPIN", "1")
    ws = fp4.workspace(fp4.OP_QUANTIZE, fp4.NVFP4, rows, 0, K)
    for i in range(2):
        x = synth.gaussian(41 + rows + i, (rows, K))
        x[rows - 1 - i, K // (2 + i)] = 99.0 + i
        if bf16:
            x = synth.to_bf16_bits(x)
        say("nvfp4 grid path, wait cut short, rows=%d K=%d bf16=%s call %d" % (rows, K, bf16, i))
        q = fp4.quantize(to_dev(x), fp4.NVFP4, ws=ws)
        codes, scales, _, ts = orc.quantize(x, 1)
        assert to_host(q.tensor_scale)[0] == np.float32(ts)
        np.testing.assert_array_equal(to_host(q.scales), scales)
        np.testing.assert_array_equal(to_host(q.codes), codes)
        assert (to_host(ws) == 0).all(), "workspace words left non-zero"


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


# ---- dense sweeps of the hardware rounding paths ------------------------------
# Every E2M1 code the quantisers write comes from the matrix core's FP32 ->
# FP4 converter, and every NVFP4 quotient |x| / d from a correctly rounded
# reciprocal with two corrections: the sweeps below put inputs on and next to
# every decision point of both.
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


def _around(v):
    """v and its float32 neighbours one ulp below and above."""
    v = np.asarray(v, np.float32)
    return np.concatenate([np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))])


def _e2m1_sweep_matrix():
    """One 32-block per (binade e, sign): element 0 is +-6 * 2^e (so the block
    exponent is e under both MXFP4 rules), the other 31 hold every E2M1
    midpoint t * 2^e and its two float32 neighbours (21 values), the grid
    points 0.5, 1, 1.5, 2, 3, 4, 6 and 6 one ulp below, and -0 / 0, with signs
    alternating.  e runs over every binade whose block maximum is a finite
    FP32 value, 2^-127 .. 2^125 (midpoints reach FP32 subnormals)."""
    rows = []
    for e in range(-127, 126):
        for sign in (1.0, -1.0):
            p = np.float32(2.0) ** np.float32(e) if e > -127 else np.float32(np.ldexp(1.0, -127))
            mids = _around(MIDPOINTS * p)                             # 21
            grid = np.array([0.5, 1.0, 2.0, 4.0], np.float32) * p      # 4
            extra = np.concatenate([grid, [np.nextafter(np.float32(6.0) * p, np.float32(0))],
                                    [np.float32(0.0), np.float32(-0.0)], grid[:2] * np.float32(3.0),
                                    [np.float32(6.0) * p]])
            blk = np.concatenate([[np.float32(6.0) * p], mids, extra]).astype(np.float32)
            assert blk.size == 32
            sgn = np.where(np.arange(32) % 2 == 0, sign, -sign).astype(np.float32)
            sgn[0] = sign
            rows.append(blk * sgn)
    blocks = np.stack(rows)                      # (506, 32)
    return blocks.reshape(-1, 32 * 22)           # 23 rows of 22 blocks


@pytest.mark.parametrize("fmt", [0, 2])
def test_e2m1_converter_sweep_every_binade(orc, fmt):
    x = _e2m1_sweep_matrix()
    assert np.isfinite(x).all()
    _run(orc, fmt, x)


def _nvfp4_division_sweep(s_t):
    """For every finite nonzero E4M3 byte sb (1..126): two 16-blocks whose
    maximum is 6 * d, d = e4m3(sb) * s_t (FP32), so the block scale is sb; the
    other 30 elements put |x| / d on and one ulp next to each E2M1 decision
    point (0.25, 0.75, ..., 5), both signs."""
    import oracle
    blocks = []
    for sb in range(1, 127):
        d = np.float32(np.float32(oracle.e4m3_value(sb)) * np.float32(s_t))
        amax = np.float32(np.float32(6.0) * d)
        probes = _around(MIDPOINTS * d)                               # 21
        probes = np.concatenate([probes, -probes[:9]])                # 30
        for h in range(2):
            blk = np.concatenate([[amax if h == 0 else -amax], probes[15 * h:15 * h + 15]]).astype(np.float32)
            blocks.append(blk)
    return np.concatenate(blocks).reshape(9, -1)                      # 9 rows of 28 blocks


@pytest.mark.parametrize("s_t", [1.0, 2.0 ** -10, 0.0123, 3.7e-5, 1.3e-30, 5.5e3])
def test_nvfp4_division_sweep_every_scale_byte(orc, s_t):
    x = _nvfp4_division_sweep(s_t)
    assert np.isfinite(x).all()
    q, ref = _run(orc, 1, x, ts=float(np.float32(s_t)))
    # every E4M3 byte 1..126 occurs as a block scale
    canon = orc.quantize(x, 1, tensor_scale=float(np.float32(s_t)))[2]
    assert set(range(1, 127)) <= set(np.unique(canon).tolist())


@pytest.mark.parametrize("rows,K", [(16, 4096), (40, 4096), (512, 4096)])
@pytest.mark.parametrize("bf16", [False, True])
def test_nvfp4_nan_skipped_by_tensor_maximum(orc, rows, K, bf16):
    """One NaN in the tensor: every path's tensor maximum skips it, as the
    oracle's does, below the one-launch threshold (256 KB: 16 x 4096), on
    the one-launch grid path (40 x 4096: 320 KB FP32; BF16 160 KB takes the
    small path) and above 1 MB (512 x 4096: amax kernel, then quantise).  s_t and every scale
    byte equal the oracle's; codes equal everywhere except at the NaN
    itself (a NaN input has no defined code)."""
    x = synth.gaussian(77 + rows, (rows, K))
    r, k = rows // 2, 123
    x[r, k] = np.float32(np.nan)
    if bf16:
        x = synth.to_bf16_bits(x)
    import block_scaled_fp4_03_amd as fp4
    say("nvfp4 NaN rows=%d K=%d bf16=%s" % (rows, K, bf16))
    q = fp4.quantize(to_dev(x), fp4.NVFP4)
    codes, scales, _, ts = orc.quantize(x, 1)
    assert np.isfinite(ts)
    assert to_host(q.tensor_scale)[0] == np.float32(ts)
    np.testing.assert_array_equal(to_host(q.scales), scales)
    got = to_host(q.codes).copy()
    got[r, k // 2] = codes[r, k // 2] = 0
    np.testing.assert_array_equal(got, codes)
